// Per-layer reconstruction error ("GPT-2 Quantization Reconstruction Error", "What this
// project does", step 5; the layer objective ||WX - What X||^2 of "GPTQ: Post-Training
// INT4", "OBQ Foundation"), with the same calibration X for W and its quantized copy:
//
//   mse = sum_{t, o} (X (W - What)^T)[t, o]^2 / (n_tok * d_out)
//
// Two passes.  A decode pass forms dW = W - What (What from the INT4 nibbles or 8-bit codes
// and the scales, and the zeros of the zero-point form, the product exact in float32) and rounds it once to bfloat16, rows padded
// to a multiple of 64 with zeros.  The contraction X dW^T then runs on the bfloat16 MFMA
// engine, X rounded once to bfloat16 (exact for bfloat16 X; large bfloat16 problems run on
// the 256 x 256 direct-load engine); the epilogue squares and sums the output tile in
// registers, so the product is never written.  Each rounding is unbiased with relative
// size at most 2^-9, so it moves the mean square by O(2^-18) in expectation plus a
// fluctuation that averages over the n_tok x d_out outputs: well under 1e-4 relative on
// the layers measured, against a 0.5 % bar.  Per-workgroup partial sums (float64) are
// added in a fixed order.
#include "gemm_bf16_dl.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// dW[o][c] = W[o][c] - s[o][group(c)] * (code[o][c] - z[o][group(c)]) (float32: the product
// is exact, the difference rounded once), z = 0 for symmetric codes, stored as bf16 (rounded
// once more) or, F32, as float32; ld = kseg (a multiple of 8, columns d_in .. kseg-1 zero).
// One thread per 8 columns of a row.
template <int DTW, bool ZP>
__device__ __forceinline__ void dw8(const void* __restrict__ Wv, int64_t ldw, int64_t n,
                                    const uint8_t* __restrict__ packed, const int8_t* __restrict__ codes,
                                    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
                                    const int32_t* __restrict__ g_idx, int64_t ng, int g, int vec, int64_t o, int64_t c,
                                    float (&d)[8]) {
    typedef typename Elem<DTW>::T T;
    const T* W = (const T*)Wv;
    if (vec && c + 8 <= n) {
        const float4 w0 = Elem<DTW>::get4(W, o * ldw + c), w1 = Elem<DTW>::get4(W, o * ldw + c + 4);
        const int64_t gi = o * ng + (g == 0 ? 0 : c / g);
        const int z = ZP ? (int)zeros[gi] : 0;
        int q[8];
        if (packed) {
            const uint32_t b = *(const uint32_t*)(packed + o * (n / 2) + c / 2);
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = (int)((b >> (4 * k)) & 15) - (ZP ? z : 8);
        } else {
            const uint2 b = *(const uint2*)(codes + o * n + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (ZP) {
                    q[k] = (int)((b.x >> (8 * k)) & 0xff) - z;
                    q[4 + k] = (int)((b.y >> (8 * k)) & 0xff) - z;
                } else {
                    q[k] = (int8_t)((b.x >> (8 * k)) & 0xff);
                    q[4 + k] = (int8_t)((b.y >> (8 * k)) & 0xff);
                }
            }
        }
        const float sc = f16_bits_to_f32(scales[gi]);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = wv[k] - sc * (float)q[k];
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t cc = c + k;
            if (cc >= n) { d[k] = 0.f; continue; }
            const int64_t G = g == 0 ? 0 : (g_idx ? (int64_t)g_idx[cc] : cc / g);
            int q;
            if (packed) {
                const uint8_t b = packed[o * (n / 2) + cc / 2];
                q = (int)((cc & 1) ? (b >> 4) : (b & 15)) - (ZP ? 0 : 8);
            } else {
                q = ZP ? (int)(uint8_t)codes[o * n + cc] : (int)codes[o * n + cc];
            }
            if (ZP) q -= (int)zeros[o * ng + G];
            d[k] = Elem<DTW>::get(W, o * ldw + cc) - f16_bits_to_f32(scales[o * ng + G]) * (float)q;
        }
    }
}

template <int DTW, bool ZP, bool F32 = false>
__global__ __launch_bounds__(256) void mse_decode_kernel(const void* __restrict__ Wv, int64_t ldw, int64_t m, int64_t n,
                                                         int64_t kseg, const uint8_t* __restrict__ packed,
                                                         const int8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros,
                                                         const int32_t* __restrict__ g_idx, int64_t ng, int g,
                                                         int vec, void* __restrict__ dwv) {
    const int64_t per_row = kseg / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= m * per_row) return;
    const int64_t o = idx / per_row, c = (idx - o * per_row) * 8;
    float d[8];
    dw8<DTW, ZP>(Wv, ldw, n, packed, codes, scales, zeros, g_idx, ng, g, vec, o, c, d);
    if (F32) {
        float* dw = (float*)dwv + o * kseg + c;
        *(float4*)dw = make_float4(d[0], d[1], d[2], d[3]);
        *(float4*)(dw + 4) = make_float4(d[4], d[5], d[6], d[7]);
    } else {
        uint16_t* dw = (uint16_t*)dwv;
        *(uint4*)(dw + o * kseg + c) = make_uint4(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]),
                                                  pack_bf16x2(d[4], d[5]), pack_bf16x2(d[6], d[7]));
    }
}

// float32 X (element (t, c) at p[t * ld + c]) rounded once to bfloat16 while staging
struct F32RowsBf16 {
    const float* p;
    int64_t ld, M, K;
    int vec;                         // ld % 4 == 0 and p 16-byte aligned
    template <int ROWS>
    struct Regs { uint4 v[ROWS * 8 / GEMM_THREADS]; };
    template <int ROWS>
    __device__ __forceinline__ void load(Regs<ROWS>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = ROWS * 8 / GEMM_THREADS;
        const int64_t kk = k0;
        const int rl = tid >> 3, c = tid & 7;
        const uint32_t loff = (uint32_t)(((int64_t)rl * ld + 8 * c) * 4);
        const bool full = vec && (m0 + ROWS <= M) && (kk + BK16 <= K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const float* ub = p + (m0 + 32 * i) * ld + kk;
            float x[8];
            if (full) {
                const float4 x0 = *(const float4*)((const char*)ub + loff);
                const float4 x1 = *(const float4*)((const char*)ub + loff + 16);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const bool rok = m0 + 32 * i + rl < M;
                const float* e = (const float*)((const char*)ub + loff);
                const int64_t kc = kk + 8 * c;
#pragma unroll
                for (int q = 0; q < 8; ++q) x[q] = (rok && kc + q < K) ? e[q] : 0.f;
            }
            r.v[i] = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                                pack_bf16x2(x[6], x[7]));
        }
    }
    template <int ROWS>
    __device__ __forceinline__ void store(uint16_t* S, const Regs<ROWS>& r, int tid) const {
        constexpr int NV = ROWS * 8 / GEMM_THREADS;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            *(uint4*)(S + lds_off(idx >> 3, idx & 7)) = r.v[i];
        }
    }
};

// squares of the tile, summed per workgroup into part[blockIdx.x] (float64)
struct EpiSq {
    double* part;
    int64_t M, N;
    float acc;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row < M && col < N) acc = fmaf(v, v, acc);
    }
    __device__ __forceinline__ void finish(const Tile&, int tid, bool) {
        __shared__ double red[GEMM_THREADS / 64];
        double d = wave_sum_d((double)acc);
        if ((tid & 63) == 0) red[tid >> 6] = d;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < GEMM_THREADS / 64; ++w) s += red[w];
            part[blockIdx.x] = s;
        }
    }
};

__global__ __launch_bounds__(256) void mse_final_kernel(const double* __restrict__ part, int64_t nparts, double denom,
                                                        double* __restrict__ mse) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < nparts; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *mse = red[0] / denom;
}

__global__ void set_double_kernel(double* p, double v) { *p = v; }

constexpr int MSE_TILE = 128;

inline int64_t mse_kseg(int64_t d_in) { return cdiv(d_in, BK16) * BK16; }

template <class LA>
hipError_t mse_gemm(const LA& a, int64_t n_tok, int64_t d_out, int64_t kseg, const uint16_t* dw, double* part,
                    hipStream_t s, int64_t* nblocks) {
    Bf16Rows b{dw, nullptr, kseg, d_out, kseg, kseg, (int)aligned(dw, 16)};
    RectMap mp{};
    mp.M = n_tok; mp.N = d_out; mp.K = kseg;
    mp.tiles_m = (int)cdiv(n_tok, MSE_TILE);
    mp.tiles_n = (int)cdiv(d_out, MSE_TILE);
    mp.splits = 1;
    mp.kchunk = kseg;
    mp.tri_k = 0;
    mp.guard = nullptr;
    EpiSq ep{part, n_tok, d_out, 0.f};
    *nblocks = (int64_t)mp.tiles_m * mp.tiles_n;
    hipLaunchKernelGGL((gemm_bf16_kernel<MSE_TILE, MSE_TILE, LA, Bf16Rows, RectMap, EpiSq>), dim3((unsigned)*nblocks),
                       dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

}  // namespace

// workspace: dW (d_out x kseg bfloat16), then one float64 partial per tile
size_t mse_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out) {
    const size_t dw = align_up((size_t)(d_out * mse_kseg(d_in)) * sizeof(uint16_t), 256);
    const int64_t nb = cdiv(n_tok, MSE_TILE) * cdiv(d_out, MSE_TILE);
    return dw + (size_t)nb * sizeof(double);
}

hipError_t mse_launch(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W, int w_dtype,
                      int64_t ldw, const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                      const int32_t* g_idx, int64_t d_out, int bits, int group_size, double* mse, void* ws, hipStream_t s,
                      const uint16_t* zeros) {
    (void)bits;
    hipError_t e;
    if (n_tok == 0 || d_out == 0) {
        hipLaunchKernelGGL(set_double_kernel, dim3(1), dim3(1), 0, s, mse, 0.0);
        return hipGetLastError();
    }
    const int64_t kseg = mse_kseg(d_in);
    uint16_t* dw = (uint16_t*)ws;
    double* part = (double*)((char*)ws + align_up((size_t)(d_out * kseg) * sizeof(uint16_t), 256));

    const int64_t ng = group_size == 0 ? 1 : cdiv(d_in, group_size);
    const size_t wsz = w_dtype == 0 ? 4 : 2;
    const int vec = (ldw % 8 == 0) && (d_in % 8 == 0) && aligned(W, 8 * wsz) && !g_idx &&
                    (group_size == 0 || group_size % 8 == 0) && (!packed || aligned(packed, 4)) &&
                    (!codes || aligned(codes, 8));
    const unsigned dgrid = (unsigned)cdiv(d_out * (kseg / 8), 256);
    auto dec = w_dtype == 0 ? (zeros ? mse_decode_kernel<0, true> : mse_decode_kernel<0, false>)
                            : (zeros ? mse_decode_kernel<1, true> : mse_decode_kernel<1, false>);
    hipLaunchKernelGGL(dec, dim3(dgrid), dim3(256), 0, s, W, ldw, d_out, d_in, kseg, packed, codes, scales, zeros, g_idx,
                       ng, group_size, vec, dw);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    int64_t nb = 0;
    const bool dl = x_dtype == 2 && (ldx % 8 == 0) && aligned(X, 16) && (d_in % 8 == 0) &&
                    cdiv(n_tok, DL_TILE) * cdiv(d_out, DL_TILE) >= 256;
    if (dl) {
        // large bfloat16 problems: direct-load engine, 256 x 256 tiles (dW's zero tail covers
        // the clamped X chunks past d_in)
        DlRows a{{(const uint16_t*)X, nullptr, nullptr, nullptr}, 1, ldx, n_tok, d_in, kseg};
        DlRows b{{dw, nullptr, nullptr, nullptr}, 1, kseg, d_out, kseg, kseg};
        RectMap mp{};
        mp.M = n_tok; mp.N = d_out; mp.K = kseg;
        mp.tiles_m = (int)cdiv(n_tok, DL_TILE);
        mp.tiles_n = (int)cdiv(d_out, DL_TILE);
        mp.splits = 1;
        mp.kchunk = kseg;
        mp.tri_k = 0;
        mp.guard = nullptr;
        // output columns fastest: the workgroups in flight share a few X row blocks (X is
        // the large operand, tokens x d_in), and dW's blocks are the ones re-read
        mp.nfast = 1;
        EpiSq ep{part, n_tok, d_out, 0.f};
        nb = (int64_t)mp.tiles_m * mp.tiles_n;
        hipLaunchKernelGGL((gemm_dl_kernel<DlRows, DlRows, RectMap, EpiSq>), dim3((unsigned)nb), dim3(GEMM_THREADS), 0, s,
                           a, b, mp, ep);
        e = hipGetLastError();
    } else if (x_dtype == 2) {
        Bf16Rows a{(const uint16_t*)X, nullptr, ldx, n_tok, d_in, kseg, (int)((ldx % 8 == 0) && aligned(X, 16))};
        e = mse_gemm(a, n_tok, d_out, kseg, dw, part, s, &nb);
    } else {
        F32RowsBf16 a{(const float*)X, ldx, n_tok, d_in, (int)((ldx % 4 == 0) && aligned(X, 16))};
        e = mse_gemm(a, n_tok, d_out, kseg, dw, part, s, &nb);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(256), 0, s, part, nb, (double)n_tok * (double)d_out, mse);
    return hipGetLastError();
}

// ------------------------------------------------------------------ through the Hessian
// sum over tokens and outputs of (X dW^T)^2 = tr(dW X^T X dW^T) = tr(dW H dW^T) / 2 with
// H = 2 X^T X: one d_out x d_in x d_in product instead of n_tok x d_in x d_out, for H already
// formed (its damping, shift, taken off in the epilogue).
//
// Small layers: the float32 engine over the whole of H.  Layers of at least 256 output tiles
// of 256 x 256: H symmetric gives tr(dW H dW^T) = sum_i sum_c dW[i][c] (dW G)[i][c] with
// G = diag(H) + 2 (strict upper part of H), so output column block cb only contracts over
// the column blocks 0 .. cb (half the products).  That product runs on the bfloat16
// 256 x 256 engine (register-staged) as a three-term split: a = a_hi + a_lo (each
// bfloat16, a_hi = bf16(a), a_lo = bf16(a - a_hi), so |a - a_hi - a_lo| <= 2^-18 |a|), and
// a b ~ a_hi b_hi + a_hi b_lo + a_lo b_hi, each product exact in float32, the dropped terms
// (a_lo b_lo and the residuals) below 2^-16 |a b| and of either sign.  The three pieces are
// interleaved per 256-column block jb along k (k = 768 jb + 256 s + offset, pieces s = 0, 1,
// 2 of dW = hi, hi, lo and of G = hi, lo, hi), so a tile's k range is the prefix
// k < 768 (cb + 1).  G is stored as the lower-triangular B(c, j) = G[j][c] (row c of H, j <= c).
namespace {
inline int64_t mse_h_k8(int64_t d_in) { return cdiv(d_in, 8) * 8; }
inline bool mse_h_big(int64_t d_out, int64_t d_in) { return cdiv(d_out, 128) * cdiv(d_in, 128) >= 512; }
inline int64_t mse_h_tiles(int64_t d_out, int64_t d_in) {
    return mse_h_big(d_out, d_in) ? cdiv(d_out, 128) * cdiv(d_in, 128) : cdiv(d_out, 64) * cdiv(d_in, 64);
}
inline bool mse_h_split(int64_t d_out, int64_t d_in) { return cdiv(d_out, DL_TILE) * cdiv(d_in, DL_TILE) >= 256; }

constexpr int SPLIT_KT = 3 * DL_TILE / DL_BK;            // k-tiles per 256-column block (three pieces)

__device__ __forceinline__ void bf16_hi_lo(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(v);
    lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// row o, columns c .. c+7 (c % 8 == 0) of dW as the pieces hi, hi, lo in the tile-major layout
// of k per row 3 npad
__device__ __forceinline__ void put_pieces(uint16_t* __restrict__ a3, int64_t o, int64_t c, int64_t npad,
                                           const float (&d)[8]) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint16_t h0, l0, h1, l1;
        bf16_hi_lo(d[2 * k], h0, l0);
        bf16_hi_lo(d[2 * k + 1], h1, l1);
        hw[k] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[k] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const int64_t kl = 3 * npad, k0 = (c >> 8) * (3 * DL_TILE) + (c & (DL_TILE - 1));
    *(uint4*)(a3 + dl_tiled_index(o, k0, kl)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *(uint4*)(a3 + dl_tiled_index(o, k0 + DL_TILE, kl)) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *(uint4*)(a3 + dl_tiled_index(o, k0 + 2 * DL_TILE, kl)) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}

// dW in float32 (row-major, ld k8, for the epilogue) and as the pieces hi, hi, lo, tile-major
// over 256-row panels with k per row 3 npad; rows past m and columns past n are zero.
// One thread per 8 columns of a row (npad a multiple of 256, so 8 columns share a block).
template <int DTW, bool ZP>
__global__ __launch_bounds__(256) void mse_decode3_kernel(const void* __restrict__ Wv, int64_t ldw, int64_t m, int64_t n,
                                                          int64_t mpad, int64_t npad, int64_t k8,
                                                          const uint8_t* __restrict__ packed,
                                                          const int8_t* __restrict__ codes,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ zeros,
                                                          const int32_t* __restrict__ g_idx, int64_t ng, int g, int vec,
                                                          float* __restrict__ dw, uint16_t* __restrict__ a3) {
    const int64_t per_row = npad / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= mpad * per_row) return;
    const int64_t o = idx / per_row, c = (idx - o * per_row) * 8;
    float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (o < m && c < n) dw8<DTW, ZP>(Wv, ldw, n, packed, codes, scales, zeros, g_idx, ng, g, vec, o, c, d);
    if (o < m && c < k8) {
        float* p = dw + o * k8 + c;
        *(float4*)p = make_float4(d[0], d[1], d[2], d[3]);
        *(float4*)(p + 4) = make_float4(d[4], d[5], d[6], d[7]);
    }
    put_pieces(a3, o, c, npad, d);
}

// the pieces of a float32 dW (row-major, ld) that is already formed; zero past m and n
__global__ __launch_bounds__(256) void mse_pieces_kernel(const float* __restrict__ dw, int64_t ld, int64_t m, int64_t n,
                                                         int64_t mpad, int64_t npad, int vec, uint16_t* __restrict__ a3) {
    const int64_t per_row = npad / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= mpad * per_row) return;
    const int64_t o = idx / per_row, c = (idx - o * per_row) * 8;
    float d[8];
    if (vec && o < m && c + 8 <= n) {
        const float4 v0 = *(const float4*)(dw + o * ld + c), v1 = *(const float4*)(dw + o * ld + c + 4);
        d[0] = v0.x; d[1] = v0.y; d[2] = v0.z; d[3] = v0.w; d[4] = v1.x; d[5] = v1.y; d[6] = v1.z; d[7] = v1.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = (o < m && c + k < n) ? dw[o * ld + c + k] : 0.f;
    }
    put_pieces(a3, o, c, npad, d);
}

// B(c, j) = G[j][c] = 2 H[c][j] (j < c), H[c][c] (j = c), 0 (j > c, or past n), as the
// pieces hi, lo, hi in the triangular tile-major layout (panel p = c / 256 holds k-tiles
// 0 .. SPLIT_KT (p + 1) - 1).  One thread per 8 columns j; blocks past the diagonal block are
// not stored.
__global__ __launch_bounds__(256) void mse_gsplit_kernel(const float* __restrict__ H, int64_t ldh, int64_t n, int64_t npad,
                                                         int vec, uint16_t* __restrict__ b3) {
    const int64_t per_row = npad / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= npad * per_row) return;
    const int64_t c = idx / per_row, j = (idx - c * per_row) * 8;
    const int64_t pan = c >> 8;
    if ((j >> 8) > pan) return;
    float h[8];
    if (vec && c < n && j + 8 <= n) {
        const float4 h0 = *(const float4*)(H + c * ldh + j), h1 = *(const float4*)(H + c * ldh + j + 4);
        h[0] = h0.x; h[1] = h0.y; h[2] = h0.z; h[3] = h0.w; h[4] = h1.x; h[5] = h1.y; h[6] = h1.z; h[7] = h1.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = (c < n && j + k < n) ? H[c * ldh + j + k] : 0.f;
    }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint16_t hb[2], lb[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int64_t jj = j + 2 * k + u;
            const float gv = jj < c ? 2.f * h[2 * k + u] : (jj == c ? h[2 * k + u] : 0.f);
            bf16_hi_lo(gv, hb[u], lb[u]);
        }
        hw[k] = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
        lw[k] = (uint32_t)lb[0] | ((uint32_t)lb[1] << 16);
    }
    const int64_t k0 = (j >> 8) * (3 * DL_TILE) + (j & (DL_TILE - 1));
    uint16_t* base = b3 + (int64_t)SPLIT_KT * (pan * (pan + 1) / 2) * (DL_TILE * DL_BK) + (c & (DL_TILE - 1)) * DL_BK;
    const int64_t ks[3] = {k0, k0 + DL_TILE, k0 + 2 * DL_TILE};
    const uint4 v[3] = {make_uint4(hw[0], hw[1], hw[2], hw[3]), make_uint4(lw[0], lw[1], lw[2], lw[3]),
                        make_uint4(hw[0], hw[1], hw[2], hw[3])};
#pragma unroll
    for (int s = 0; s < 3; ++s) *(uint4*)(base + (ks[s] >> 5) * (DL_TILE * DL_BK) + (ks[s] & 31)) = v[s];
}

// Output tiles (ib, cb) of dW G, the longest k ranges first: column blocks from the last,
// row blocks fastest (a workgroup b runs on XCD b % 8, which then holds a few row blocks of
// dW and the column blocks in flight).  Tile (ib, cb) contracts k < 768 (cb + 1).
struct SplitTriMap {
    int tiles_m, tiles_n;
    const int32_t* guard;
    __device__ __forceinline__ bool get(int bid, int BM, int BN, Tile& t) const {
        const int ib = bid % tiles_m, cb = tiles_n - 1 - bid / tiles_m;
        t.m0 = (int64_t)ib * BM;
        t.n0 = (int64_t)cb * BN;
        t.kbeg = 0;
        t.kend = (int64_t)SPLIT_KT * DL_BK * (cb + 1);
        t.split = -1;
        t.tile = bid;
        return true;
    }
};

struct SplitWs {
    int64_t mpad, npad;
    size_t dw_bytes, a3_bytes, b3_bytes;
    int64_t tiles;
};

SplitWs split_ws(int64_t d_out, int64_t d_in) {
    SplitWs w{};
    w.mpad = cdiv(d_out, DL_TILE) * DL_TILE;
    w.npad = cdiv(d_in, DL_TILE) * DL_TILE;
    const int64_t nb = w.npad / DL_TILE;
    w.dw_bytes = align_up((size_t)(d_out * mse_h_k8(d_in)) * sizeof(float), 256);
    w.a3_bytes = align_up((size_t)(w.mpad * 3 * w.npad) * sizeof(uint16_t), 256);
    w.b3_bytes = align_up((size_t)SPLIT_KT * (size_t)(nb * (nb + 1) / 2) * DL_TILE * DL_BK * sizeof(uint16_t), 256);
    w.tiles = (w.mpad / DL_TILE) * nb;
    return w;
}

template <int T>
hipError_t mse_h_product(const float* dW, int64_t lddw, const float* H, int64_t ldh, int64_t m, int64_t n,
                         const float* shift, double* part, int64_t* nparts, hipStream_t s) {
    const int va = (int)((lddw % 4 == 0) && aligned(dW, 16));
    const int vb = (int)((ldh % 4 == 0) && aligned(H, 16));
    OpMMajor<0> la{dW, lddw, m, n, va};
    OpKMajor<0> lb{H, ldh, n, n, vb};
    RectMap mp{};
    mp.M = m; mp.N = n; mp.K = n;
    mp.tiles_m = (int)cdiv(m, T);
    mp.tiles_n = (int)cdiv(n, T);
    mp.splits = 1;
    mp.kchunk = cdiv(n, GEMM_BK) * GEMM_BK;
    mp.tri_k = 0;
    mp.guard = nullptr;
    EpiTrace ep{dW, lddw, m, n, part, shift, 0.f};
    *nparts = (int64_t)mp.tiles_m * mp.tiles_n;
    hipLaunchKernelGGL((gemm_f32_kernel<T, T, OpMMajor<0>, OpKMajor<0>, RectMap, EpiTrace>), dim3((unsigned)*nparts),
                       dim3(GEMM_THREADS), 0, s, la, lb, mp, ep);
    return hipGetLastError();
}
}  // namespace

// ---- the split product, also used by the AWQ search (per candidate dW, G formed once)
bool split_route(int64_t d_out, int64_t d_in) { return mse_h_split(d_out, d_in); }
size_t split_pieces_bytes(int64_t d_out, int64_t d_in) { return split_ws(d_out, d_in).a3_bytes; }
size_t split_g_bytes(int64_t d_in) { return split_ws(1, d_in).b3_bytes; }
int64_t split_tiles(int64_t d_out, int64_t d_in) { return split_ws(d_out, d_in).tiles; }

hipError_t split_g_launch(const float* H, int64_t ldh, int64_t n, uint16_t* b3, hipStream_t s) {
    const int64_t npad = cdiv(n, DL_TILE) * DL_TILE;
    const int hvec = (ldh % 4 == 0) && aligned(H, 16);
    hipLaunchKernelGGL(mse_gsplit_kernel, dim3((unsigned)cdiv(npad * (npad / 8), 256)), dim3(256), 0, s, H, ldh, n, npad,
                       hvec, b3);
    return hipGetLastError();
}

hipError_t split_pieces_launch(const float* dW, int64_t ld, int64_t m, int64_t n, uint16_t* a3, hipStream_t s) {
    const int64_t mpad = cdiv(m, DL_TILE) * DL_TILE, npad = cdiv(n, DL_TILE) * DL_TILE;
    const int vec = (ld % 4 == 0) && aligned(dW, 16);
    hipLaunchKernelGGL(mse_pieces_kernel, dim3((unsigned)cdiv(mpad * (npad / 8), 256)), dim3(256), 0, s, dW, ld, m, n,
                       mpad, npad, vec, a3);
    return hipGetLastError();
}

// part[t] = sum over output tile t of ((dW G) - shift dW) dW, t < split_tiles(m, n)
hipError_t split_trace_launch(const uint16_t* a3, const uint16_t* b3, const float* dW, int64_t ld, int64_t m, int64_t n,
                              const float* shift, double* part, hipStream_t s) {
    const int64_t mpad = cdiv(m, DL_TILE) * DL_TILE, npad = cdiv(n, DL_TILE) * DL_TILE;
    DlTiled1 a{a3, 3 * npad};
    DlTri b{b3, SPLIT_KT};
    SplitTriMap mp{(int)(mpad / DL_TILE), (int)(npad / DL_TILE), nullptr};
    EpiTrace ep{dW, ld, m, n, part, shift, 0.f};
    // register-staged loads, two k-tiles per unrolled step: every k range is 768 (cb + 1)
    static_assert((SPLIT_KT * DL_BK) % (2 * DL_BK) == 0, "k ranges must hold whole pairs of k-tiles");
    hipLaunchKernelGGL((gemm_rs_kernel<2, DlTiled1, DlTri, SplitTriMap, EpiTrace>),
                       dim3((unsigned)((mpad / DL_TILE) * (npad / DL_TILE))), dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

// workspace: float32 route: dW (d_out x k8 float32), then one float64 partial per tile;
// split route: dW float32, dW's pieces, G's pieces, then one float64 partial per tile
size_t mse_h_ws_bytes(int64_t d_in, int64_t d_out) {
    if (mse_h_split(d_out, d_in)) {
        const SplitWs w = split_ws(d_out, d_in);
        return w.dw_bytes + w.a3_bytes + w.b3_bytes + (size_t)w.tiles * sizeof(double);
    }
    return align_up((size_t)(d_out * mse_h_k8(d_in)) * sizeof(float), 256) +
           (size_t)mse_h_tiles(d_out, d_in) * sizeof(double);
}

hipError_t mse_h_launch(const float* H, int64_t ldh, int64_t d_in, int64_t n_tok, const float* shift, const void* W,
                        int w_dtype, int64_t ldw, const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                        const uint16_t* zeros, const int32_t* g_idx, int64_t d_out, int group_size, double* mse,
                        void* ws, hipStream_t s) {
    hipError_t e;
    if (n_tok == 0 || d_out == 0) {
        hipLaunchKernelGGL(set_double_kernel, dim3(1), dim3(1), 0, s, mse, 0.0);
        return hipGetLastError();
    }
    const int64_t k8 = mse_h_k8(d_in);
    float* dw = (float*)ws;
    const int64_t ng = group_size == 0 ? 1 : cdiv(d_in, group_size);
    const size_t wsz = w_dtype == 0 ? 4 : 2;
    const int vec = (ldw % 8 == 0) && (d_in % 8 == 0) && aligned(W, 8 * wsz) && !g_idx &&
                    (group_size == 0 || group_size % 8 == 0) && (!packed || aligned(packed, 4)) &&
                    (!codes || aligned(codes, 8));
    int64_t np = 0;
    double* part;
    if (mse_h_split(d_out, d_in)) {
        const SplitWs w = split_ws(d_out, d_in);
        uint16_t* a3 = (uint16_t*)((char*)ws + w.dw_bytes);
        uint16_t* b3 = (uint16_t*)((char*)a3 + w.a3_bytes);
        part = (double*)((char*)b3 + w.b3_bytes);
        auto dec = w_dtype == 0 ? (zeros ? mse_decode3_kernel<0, true> : mse_decode3_kernel<0, false>)
                                : (zeros ? mse_decode3_kernel<1, true> : mse_decode3_kernel<1, false>);
        hipLaunchKernelGGL(dec, dim3((unsigned)cdiv(w.mpad * (w.npad / 8), 256)), dim3(256), 0, s, W, ldw, d_out, d_in,
                           w.mpad, w.npad, k8, packed, codes, scales, zeros, g_idx, ng, group_size, vec, dw, a3);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = split_g_launch(H, ldh, d_in, b3, s)) != hipSuccess) return e;
        np = w.tiles;
        if ((e = split_trace_launch(a3, b3, dw, k8, d_out, d_in, shift, part, s)) != hipSuccess) return e;
    } else {
        part = (double*)((char*)ws + align_up((size_t)(d_out * k8) * sizeof(float), 256));
        const unsigned dgrid = (unsigned)cdiv(d_out * (k8 / 8), 256);
        auto dec = w_dtype == 0 ? (zeros ? mse_decode_kernel<0, true, true> : mse_decode_kernel<0, false, true>)
                                : (zeros ? mse_decode_kernel<1, true, true> : mse_decode_kernel<1, false, true>);
        hipLaunchKernelGGL(dec, dim3(dgrid), dim3(256), 0, s, W, ldw, d_out, d_in, k8, packed, codes, scales, zeros,
                           g_idx, ng, group_size, vec, (void*)dw);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        e = mse_h_big(d_out, d_in) ? mse_h_product<128>(dw, k8, H, ldh, d_out, d_in, shift, part, &np, s)
                                   : mse_h_product<64>(dw, k8, H, ldh, d_out, d_in, shift, part, &np, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(256), 0, s, part, np, 2.0 * (double)n_tok * (double)d_out, mse);
    return hipGetLastError();
}

}  // namespace pwq
