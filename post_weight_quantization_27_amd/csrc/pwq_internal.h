// Host-side launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pwq {

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Opt-in kernel timing (pwq_profile_enable): events around one launch of a class, with its
// algorithmic work; no-ops while timing is off.
void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s, double work);

// Hessian build: H += 2 X^T X (float32 MFMA, upper tiles, deterministic split-K, mirror).
struct HessPlan {
    int bm;            // tile edge (64, 128, or 256 on the direct-load engine)
    int tiles;         // tiles per edge
    int splits;        // token chunks of the split tiles
    int full;          // tiles [0, full) run over all tokens; the rest are split
    int64_t kchunk;    // tokens per chunk (multiple of the engine's k tile)
    int dl;            // direct-load engine: 1 = bfloat16 X transposed, 4 = float32 X as a transposed
                       // bfloat16 pair (four products), 0 = register-staged engines
    int64_t npad;      // tokens of the transposed copy (multiple of 64, zero tail)
    size_t xt_bytes;   // transposed copy or pair (0 unless dl)
    size_t ws_bytes;   // transposed copy + partial tiles (0 when neither is needed)
};
HessPlan hessian_plan(int64_t n_tok, int64_t d_in, int x_dtype);
hipError_t hessian_launch(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, float* H,
                          void* ws, hipStream_t s);
hipError_t damp_launch(float* H, int64_t n, float damp, float* lambda_out, hipStream_t s);
hipError_t act_order_launch(const float* H, int64_t n, int32_t* perm, hipStream_t s);

// Inverse-Hessian factor.
constexpr int CHOL_NB = 128;
constexpr int64_t PERM_MAX_N = 32768;     // row staging through LDS for permuted copies
size_t chol_ws_bytes(int64_t n);
hipError_t chol_launch(const float* H, int64_t n, const int32_t* perm, float* U, int32_t* info, void* ws,
                       hipStream_t s);

// GPTQ column loop.  The quantize, dequant and MSE launchers take the zero-point form when
// given zeros (zeros_out for the quantizers, zeros for the decoders): codes are then the
// unsigned bytes 0 .. 2^bits - 1 and nibbles hold the code itself.
struct GptqWs {
    size_t wf, err, codes, inv, pcs, total;
    bool has_pcs;
};
GptqWs gptq_ws_layout(int64_t d_out, int64_t d_in, int block_size, int group_size, int act_order);
hipError_t gptq_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* U,
                       const int32_t* info, int bits, int group_size, int block_size, int act_order,
                       const int32_t* perm, const uint16_t* scales_in, int8_t* codes, uint8_t* packed,
                       uint16_t* scales_out, int32_t* g_idx, void* ws, hipStream_t s,
                       const uint16_t* zeros_in = nullptr, uint16_t* zeros_out = nullptr);

// RTN, dequant.
hipError_t rtn_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, int bits, int group_size,
                      const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out,
                      hipStream_t s, const uint16_t* zeros_in = nullptr, uint16_t* zeros_out = nullptr);
hipError_t dequant_launch(const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                          const int32_t* g_idx, int64_t m, int64_t n, int bits, int group_size, void* out,
                          int out_dtype, hipStream_t s, const uint16_t* zeros = nullptr);

// Per-tensor quantizer, replicated per row.
size_t tensor_scales_ws_bytes();
hipError_t tensor_scales_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, int bits,
                                uint16_t* scales, uint16_t* zeros, void* ws, hipStream_t s);

// Activation-aware channel scaling.
size_t chan_abs_ws_bytes(int64_t N, int64_t n);
hipError_t chan_abs_launch(const void* X, int x_dtype, int64_t N, int64_t n, int64_t ldx, float* a, void* ws,
                           hipStream_t s);
size_t awq_ws_bytes(int64_t m, int64_t n);
hipError_t awq_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* H, int64_t N,
                      const float* absmean, int bits, int group_size, int K, int zp, double* mse, int32_t* best,
                      float* s_out, int8_t* codes, uint8_t* packed, uint16_t* scales, uint16_t* zeros, void* ws,
                      hipStream_t s);

// Y = X What^T with the quantized weights (float16 X, decode regime).
size_t w4a16_ws_bytes(int64_t T, int64_t n, int64_t m);
// this device's copy of the allocation-free entry point's scratch array (looked up once per device)
hipError_t w4a16_scratch(void** out);
hipError_t w4a16_launch(const uint16_t* X, int64_t T, int64_t n, int64_t ldx, const uint8_t* packed,
                        const uint16_t* scales, const uint16_t* zeros, int64_t m, int group_size, void* Y,
                        int y_dtype, int64_t ldy, void* ws, hipStream_t s);

// Reconstruction MSE.
size_t mse_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out);
// the split product of the Hessian-route MSE (layers of >= 256 output tiles of 256 x 256):
// G's pieces from H once, dW's pieces per dW, then per-tile trace sums
bool split_route(int64_t d_out, int64_t d_in);
size_t split_pieces_bytes(int64_t d_out, int64_t d_in);
size_t split_g_bytes(int64_t d_in);
int64_t split_tiles(int64_t d_out, int64_t d_in);
hipError_t split_g_launch(const float* H, int64_t ldh, int64_t n, uint16_t* b3, hipStream_t s);
hipError_t split_pieces_launch(const float* dW, int64_t ld, int64_t m, int64_t n, uint16_t* a3, hipStream_t s);
hipError_t split_trace_launch(const uint16_t* a3, const uint16_t* b3, const float* dW, int64_t ld, int64_t m, int64_t n,
                              const float* shift, double* part, hipStream_t s);
size_t mse_h_ws_bytes(int64_t d_in, int64_t d_out);
hipError_t mse_h_launch(const float* H, int64_t ldh, int64_t d_in, int64_t n_tok, const float* shift, const void* W,
                        int w_dtype, int64_t ldw, const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                        const uint16_t* zeros, const int32_t* g_idx, int64_t d_out, int group_size, double* mse,
                        void* ws, hipStream_t s);
hipError_t mse_launch(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W,
                      int w_dtype, int64_t ldw, const uint8_t* packed, const int8_t* codes,
                      const uint16_t* scales, const int32_t* g_idx, int64_t d_out, int bits, int group_size,
                      double* mse, void* ws, hipStream_t s, const uint16_t* zeros = nullptr);

}  // namespace pwq
