// C ABI of libpwq: argument checks on the host, then the kernel launchers.
// Every check runs before the first HIP call, so a rejected call enqueues nothing.
#include <math.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/pwq.h"
#include "pwq_internal.h"

using namespace pwq;

namespace {

thread_local int g_last_hip_error = 0;

pwq_status hip_status(hipError_t e) {
    if (e == hipSuccess) return PWQ_OK;
    g_last_hip_error = (int)e;
    return PWQ_EHIP;
}

constexpr int64_t MAX_DIM = (int64_t)1 << 30;

bool bad_dim(int64_t v) { return v < 0 || v > MAX_DIM; }
constexpr int64_t QMM_MAX_COLS = (int64_t)1 << 24;     // ldx (>= d_in) of the quantized product

bool group_ok(int32_t g, int64_t d_in) {
    (void)d_in;
    return g == 0 || (g >= 2 && g % 2 == 0);
}

int64_t n_groups(int64_t d_in, int32_t g) { return g == 0 ? 1 : cdiv(d_in, g); }

// ------------------------------------------------------------------ kernel timing
struct ProfRec {
    int cls;
    hipEvent_t a, b;
    double work;
};
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;          // recorded, not yet read
std::vector<hipEvent_t> g_prof_pool;       // events free for reuse
thread_local hipEvent_t t_prof_open[PWQ_PROF_CLASSES] = {};

hipEvent_t prof_event() {                  // g_prof_mu held
    if (!g_prof_pool.empty()) {
        hipEvent_t e = g_prof_pool.back();
        g_prof_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}

void prof_recycle() {                      // g_prof_mu held
    for (auto& r : g_prof_recs) {
        g_prof_pool.push_back(r.a);
        g_prof_pool.push_back(r.b);
    }
    g_prof_recs.clear();
}

}  // namespace

namespace pwq {

void prof_begin(int cls, hipStream_t s) {
    if (!g_prof_on.load(std::memory_order_relaxed) || cls < 0 || cls >= PWQ_PROF_CLASSES) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t e = prof_event();
    if (e && hipEventRecord(e, s) != hipSuccess) {
        g_prof_pool.push_back(e);
        e = nullptr;
    }
    t_prof_open[cls] = e;
}

void prof_end(int cls, hipStream_t s, double work) {
    if (!g_prof_on.load(std::memory_order_relaxed) || cls < 0 || cls >= PWQ_PROF_CLASSES) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    hipEvent_t a = t_prof_open[cls];
    t_prof_open[cls] = nullptr;
    if (!a) return;
    hipEvent_t b = prof_event();
    if (!b || hipEventRecord(b, s) != hipSuccess) {
        g_prof_pool.push_back(a);
        if (b) g_prof_pool.push_back(b);
        return;
    }
    g_prof_recs.push_back({cls, a, b, work});
}

}  // namespace pwq

extern "C" {

pwq_status pwq_profile_enable(int on) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof_recycle();
    g_prof_on.store(on != 0);
    return PWQ_OK;
}

pwq_status pwq_profile_read(double* ms, double* work, int64_t* launches, int n_classes) {
    if (n_classes < 1 || !ms || !work || !launches) return PWQ_EINVAL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (int c = 0; c < n_classes; ++c) {
        ms[c] = 0.0;
        work[c] = 0.0;
        launches[c] = 0;
    }
    hipError_t err = hipSuccess;
    for (const auto& r : g_prof_recs) {
        if (r.cls >= n_classes) continue;
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
        if (e != hipSuccess) {
            err = e;
            continue;
        }
        ms[r.cls] += t;
        work[r.cls] += r.work;
        launches[r.cls] += 1;
    }
    prof_recycle();
    return hip_status(err);
}

int pwq_version(void) { return PWQ_ABI_VERSION; }

const char* pwq_status_string(int status) {
    switch (status) {
        case PWQ_OK: return "ok";
        case PWQ_EINVAL: return "invalid argument";
        case PWQ_EDTYPE: return "unsupported dtype";
        case PWQ_EWORKSPACE: return "workspace missing or too small";
        case PWQ_EHIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

int pwq_last_hip_error(void) { return g_last_hip_error; }

// ------------------------------------------------------------------ Hessian
size_t pwq_hessian_workspace_size(int64_t n_tok, int64_t d_in, int x_dtype) {
    if (n_tok <= 0 || d_in <= 0 || bad_dim(n_tok) || bad_dim(d_in)) return 0;
    return hessian_plan(n_tok, d_in, x_dtype).ws_bytes;
}

pwq_status pwq_hessian_accumulate(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, float* H,
                                  void* ws, size_t ws_bytes, void* stream) {
    if (x_dtype != PWQ_F32 && x_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (bad_dim(n_tok) || d_in <= 0 || bad_dim(d_in) || ldx < d_in || !H) return PWQ_EINVAL;
    if (d_in > 65535 * 2) return PWQ_EINVAL;
    if (n_tok == 0) return PWQ_OK;
    if (!X) return PWQ_EINVAL;
    const size_t need = pwq_hessian_workspace_size(n_tok, d_in, x_dtype);
    if (need && (!ws || ws_bytes < need)) return PWQ_EWORKSPACE;
    return hip_status(hessian_launch(X, x_dtype, n_tok, d_in, ldx, H, ws, (hipStream_t)stream));
}

pwq_status pwq_hessian_damp(float* H, int64_t d_in, float damp, float* lambda_out, void* stream) {
    if (!H || d_in <= 0 || bad_dim(d_in) || !(damp >= 0.f) || isinf(damp)) return PWQ_EINVAL;
    return hip_status(damp_launch(H, d_in, damp, lambda_out, (hipStream_t)stream));
}

pwq_status pwq_act_order_perm(const float* H, int64_t d_in, int32_t* perm, void* stream) {
    if (!H || !perm || d_in <= 0 || bad_dim(d_in) || d_in > INT32_MAX) return PWQ_EINVAL;
    return hip_status(act_order_launch(H, d_in, perm, (hipStream_t)stream));
}

// ------------------------------------------------------------------ factor
size_t pwq_chol_workspace_size(int64_t n) {
    if (n <= 0 || bad_dim(n)) return 0;
    return chol_ws_bytes(n);
}

pwq_status pwq_chol_inverse_upper(const float* H, int64_t n, const int32_t* perm, float* U, int32_t* info, void* ws,
                                  size_t ws_bytes, void* stream) {
    if (!H || !U || !info || n <= 0 || n > 65535) return PWQ_EINVAL;
    if (perm && n > PERM_MAX_N) return PWQ_EINVAL;
    const size_t need = pwq_chol_workspace_size(n);
    if (!ws || ws_bytes < need) return PWQ_EWORKSPACE;
    return hip_status(chol_launch(H, n, perm, U, info, ws, (hipStream_t)stream));
}

// ------------------------------------------------------------------ GPTQ
static bool gptq_params_ok(const pwq_params* p) {
    if (!p) return false;
    if (p->bits < 2 || p->bits > 8) return false;
    if (p->block_size != 32 && p->block_size != 64 && p->block_size != 128) return false;
    const int g = p->group_size;
    if (g < 0) return false;
    if (g != 0 && (g % 32 != 0 || !((g % p->block_size) == 0 || (p->block_size % g) == 0))) return false;
    return true;
}

size_t pwq_gptq_workspace_size(int64_t d_out, int64_t d_in, const pwq_params* params) {
    if (d_out <= 0 || d_in <= 0 || bad_dim(d_out) || bad_dim(d_in) || !gptq_params_ok(params)) return 0;
    return gptq_ws_layout(d_out, d_in, params->block_size, params->group_size, params->act_order != 0).total;
}

static pwq_status gptq_checked(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, const float* U,
                               const int32_t* info, const pwq_params* params, const int32_t* perm,
                               const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out,
                               int32_t* g_idx, void* ws, size_t ws_bytes, void* stream, const uint16_t* zeros_in,
                               uint16_t* zeros_out) {
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (!gptq_params_ok(params)) return PWQ_EINVAL;
    if (bad_dim(d_out) || d_out > INT32_MAX || d_in <= 0 || bad_dim(d_in) || ldw < d_in) return PWQ_EINVAL;
    if (!U || !info || !scales_out || (!codes && !packed)) return PWQ_EINVAL;
    if (packed && (params->bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    const int act = params->act_order != 0;
    if (act && (!perm || !g_idx || d_in > PERM_MAX_N)) return PWQ_EINVAL;
    if (d_out == 0) return PWQ_OK;
    if (!W) return PWQ_EINVAL;
    const size_t need = pwq_gptq_workspace_size(d_out, d_in, params);
    if (!ws || ws_bytes < need) return PWQ_EWORKSPACE;
    return hip_status(gptq_launch(W, w_dtype, d_out, d_in, ldw, U, info, params->bits, params->group_size,
                                  params->block_size, act, perm, scales_in, codes, packed, scales_out, g_idx, ws,
                                  (hipStream_t)stream, zeros_in, zeros_out));
}

pwq_status pwq_gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                                   const float* U, const int32_t* info, const pwq_params* params,
                                   const int32_t* perm, const uint16_t* scales_in,
                                   int8_t* codes, uint8_t* packed, uint16_t* scales_out, int32_t* g_idx,
                                   void* ws, size_t ws_bytes, void* stream) {
    return gptq_checked(W, w_dtype, d_out, d_in, ldw, U, info, params, perm, scales_in, codes, packed, scales_out,
                        g_idx, ws, ws_bytes, stream, nullptr, nullptr);
}

pwq_status pwq_gptq_quantize_layer_zp(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw,
                                      const float* U, const int32_t* info, const pwq_params* params,
                                      const int32_t* perm, const uint16_t* scales_in, const uint16_t* zeros_in,
                                      uint8_t* codes, uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out,
                                      int32_t* g_idx, void* ws, size_t ws_bytes, void* stream) {
    if (!zeros_out || ((scales_in != nullptr) != (zeros_in != nullptr))) return PWQ_EINVAL;
    return gptq_checked(W, w_dtype, d_out, d_in, ldw, U, info, params, perm, scales_in, (int8_t*)codes, packed,
                        scales_out, g_idx, ws, ws_bytes, stream, zeros_in, zeros_out);
}

// ------------------------------------------------------------------ RTN / dequant
static pwq_status rtn_checked(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, int32_t bits,
                              int32_t group_size, const uint16_t* scales_in, int8_t* codes, uint8_t* packed,
                              uint16_t* scales_out, void* stream, const uint16_t* zeros_in, uint16_t* zeros_out) {
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldw < d_in) return PWQ_EINVAL;
    if (bits < 2 || bits > 8 || !group_ok(group_size, d_in)) return PWQ_EINVAL;
    if (!scales_out || (!codes && !packed)) return PWQ_EINVAL;
    if (packed && (bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    if (d_out == 0) return PWQ_OK;
    if (!W) return PWQ_EINVAL;
    // bytes the call must move: W once, the outputs once, fixed quantizers once
    const double per_group = (zeros_out ? 4.0 : 2.0) * (double)d_out * (double)n_groups(d_in, group_size);
    const double bytes = (double)d_out * d_in * (w_dtype == PWQ_F32 ? 4 : 2) + (codes ? (double)d_out * d_in : 0.0) +
                         (packed ? (double)d_out * d_in / 2 : 0.0) + per_group * (scales_in ? 2 : 1);
    prof_begin(PWQ_PROF_RTN, (hipStream_t)stream);
    const hipError_t e = rtn_launch(W, w_dtype, d_out, d_in, ldw, bits, group_size, scales_in, codes, packed,
                                    scales_out, (hipStream_t)stream, zeros_in, zeros_out);
    prof_end(PWQ_PROF_RTN, (hipStream_t)stream, bytes);
    return hip_status(e);
}

pwq_status pwq_rtn_quantize(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, int32_t bits,
                            int32_t group_size, const uint16_t* scales_in, int8_t* codes, uint8_t* packed,
                            uint16_t* scales_out, void* stream) {
    return rtn_checked(W, w_dtype, d_out, d_in, ldw, bits, group_size, scales_in, codes, packed, scales_out, stream,
                       nullptr, nullptr);
}

pwq_status pwq_rtn_quantize_zp(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, int32_t bits,
                               int32_t group_size, const uint16_t* scales_in, const uint16_t* zeros_in,
                               uint8_t* codes, uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out,
                               void* stream) {
    if (!zeros_out || ((scales_in != nullptr) != (zeros_in != nullptr))) return PWQ_EINVAL;
    return rtn_checked(W, w_dtype, d_out, d_in, ldw, bits, group_size, scales_in, (int8_t*)codes, packed, scales_out,
                       stream, zeros_in, zeros_out);
}

static pwq_status dequant_checked(const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                                  const uint16_t* zeros, const int32_t* g_idx, int64_t d_out, int64_t d_in, int32_t bits,
                                  int32_t group_size, void* W_out, int out_dtype, void* stream) {
    if (out_dtype != PWQ_F32 && out_dtype != PWQ_F16 && out_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (bad_dim(d_out) || d_in <= 0 || bad_dim(d_in)) return PWQ_EINVAL;
    if (bits < 2 || bits > 8 || !group_ok(group_size, d_in)) return PWQ_EINVAL;
    if ((packed != nullptr) == (codes != nullptr)) return PWQ_EINVAL;
    if (packed && (bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    if (g_idx && group_size == 0) return PWQ_EINVAL;
    if (!scales || !W_out) return PWQ_EINVAL;
    const double bytes = (packed ? (double)d_out * d_in / 2 : (double)d_out * d_in) +
                         (zeros ? 4.0 : 2.0) * (double)d_out * (double)n_groups(d_in, group_size) +
                         (double)d_out * d_in * (out_dtype == PWQ_F32 ? 4 : 2) + (g_idx ? 4.0 * d_in : 0.0);
    prof_begin(PWQ_PROF_DEQUANT, (hipStream_t)stream);
    const hipError_t e = dequant_launch(packed, codes, scales, g_idx, d_out, d_in, bits, group_size, W_out, out_dtype,
                                        (hipStream_t)stream, zeros);
    prof_end(PWQ_PROF_DEQUANT, (hipStream_t)stream, bytes);
    return hip_status(e);
}

pwq_status pwq_dequant(const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                       int64_t d_out, int64_t d_in, int32_t bits, int32_t group_size, void* W_out, int out_dtype,
                       void* stream) {
    return dequant_checked(packed, codes, scales, nullptr, g_idx, d_out, d_in, bits, group_size, W_out, out_dtype,
                           stream);
}

pwq_status pwq_dequant_zp(const uint8_t* packed, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                          const int32_t* g_idx, int64_t d_out, int64_t d_in, int32_t bits, int32_t group_size,
                          void* W_out, int out_dtype, void* stream) {
    if (!zeros) return PWQ_EINVAL;
    return dequant_checked(packed, (const int8_t*)codes, scales, zeros, g_idx, d_out, d_in, bits, group_size, W_out,
                           out_dtype, stream);
}

// ------------------------------------------------------------------ MSE
size_t pwq_recon_mse_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out) {
    if (n_tok <= 0 || d_in <= 0 || d_out <= 0 || bad_dim(n_tok) || bad_dim(d_in) || bad_dim(d_out)) return 0;
    return mse_ws_bytes(n_tok, d_in, d_out);
}

static pwq_status mse_checked(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W,
                              int w_dtype, int64_t ldw, const uint8_t* packed, const int8_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, const int32_t* g_idx, int64_t d_out,
                              int32_t bits, int32_t group_size, double* mse, void* ws, size_t ws_bytes, void* stream) {
    if (x_dtype != PWQ_F32 && x_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (bad_dim(n_tok) || bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldx < d_in || ldw < d_in) return PWQ_EINVAL;
    if (bits < 2 || bits > 8 || !group_ok(group_size, d_in)) return PWQ_EINVAL;
    if ((packed != nullptr) == (codes != nullptr)) return PWQ_EINVAL;
    if (packed && (bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    if (g_idx && group_size == 0) return PWQ_EINVAL;
    if (!mse || !scales) return PWQ_EINVAL;
    if (n_tok > 0 && d_out > 0) {
        if (!X || !W) return PWQ_EINVAL;
        const size_t need = pwq_recon_mse_workspace_size(n_tok, d_in, d_out);
        if (!ws || ws_bytes < need) return PWQ_EWORKSPACE;
    }
    return hip_status(mse_launch(X, x_dtype, n_tok, d_in, ldx, W, w_dtype, ldw, packed, codes, scales, g_idx, d_out, bits,
                                 group_size, mse, ws, (hipStream_t)stream, zeros));
}

pwq_status pwq_recon_mse(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                         const void* W, int w_dtype, int64_t ldw,
                         const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                         int64_t d_out, int32_t bits, int32_t group_size,
                         double* mse, void* ws, size_t ws_bytes, void* stream) {
    return mse_checked(X, x_dtype, n_tok, d_in, ldx, W, w_dtype, ldw, packed, codes, scales, nullptr, g_idx, d_out, bits,
                       group_size, mse, ws, ws_bytes, stream);
}

pwq_status pwq_recon_mse_zp(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                            const void* W, int w_dtype, int64_t ldw,
                            const uint8_t* packed, const uint8_t* codes, const uint16_t* scales, const uint16_t* zeros,
                            const int32_t* g_idx, int64_t d_out, int32_t bits, int32_t group_size,
                            double* mse, void* ws, size_t ws_bytes, void* stream) {
    if (!zeros) return PWQ_EINVAL;
    return mse_checked(X, x_dtype, n_tok, d_in, ldx, W, w_dtype, ldw, packed, (const int8_t*)codes, scales, zeros, g_idx,
                       d_out, bits, group_size, mse, ws, ws_bytes, stream);
}

size_t pwq_recon_mse_hessian_workspace_size(int64_t d_in, int64_t d_out) {
    if (d_in <= 0 || d_out <= 0 || bad_dim(d_in) || bad_dim(d_out)) return 0;
    return mse_h_ws_bytes(d_in, d_out);
}

pwq_status pwq_recon_mse_hessian(const float* H, int64_t ldh, int64_t d_in, int64_t n_tok, const float* h_shift,
                                 const void* W, int w_dtype, int64_t ldw, const uint8_t* packed, const void* codes,
                                 const uint16_t* scales, const uint16_t* zeros, const int32_t* g_idx, int64_t d_out,
                                 int32_t bits, int32_t group_size, double* mse, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (bad_dim(n_tok) || bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldh < d_in || ldw < d_in) return PWQ_EINVAL;
    if (bits < 2 || bits > 8 || !group_ok(group_size, d_in)) return PWQ_EINVAL;
    if (packed && (bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    if (g_idx && group_size == 0) return PWQ_EINVAL;
    if (!mse) return PWQ_EINVAL;
    if (n_tok > 0 && d_out > 0) {                // the data pointers only matter when read
        if (!H || !W || !scales || (packed != nullptr) == (codes != nullptr)) return PWQ_EINVAL;
        if (!ws || ws_bytes < pwq_recon_mse_hessian_workspace_size(d_in, d_out)) return PWQ_EWORKSPACE;
    }
    return hip_status(mse_h_launch(H, ldh, d_in, n_tok, h_shift, W, w_dtype, ldw, packed, (const int8_t*)codes, scales,
                                   zeros, g_idx, d_out, group_size, mse, ws, (hipStream_t)stream));
}

// ------------------------------------------------------------------ per-tensor quantizer
size_t pwq_tensor_scales_workspace_size(void) { return tensor_scales_ws_bytes(); }

pwq_status pwq_tensor_scales(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, int32_t bits,
                             uint16_t* scales_out, uint16_t* zeros_out, void* ws, size_t ws_bytes, void* stream) {
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldw < d_in || bits < 2 || bits > 8) return PWQ_EINVAL;
    if (!scales_out) return PWQ_EINVAL;
    if (d_out == 0) return PWQ_OK;
    if (!W) return PWQ_EINVAL;
    if (!ws || ws_bytes < tensor_scales_ws_bytes()) return PWQ_EWORKSPACE;
    return hip_status(tensor_scales_launch(W, w_dtype, d_out, d_in, ldw, bits, scales_out, zeros_out, ws,
                                           (hipStream_t)stream));
}

// ------------------------------------------------------------------ activation-aware scaling
size_t pwq_channel_abs_mean_workspace_size(int64_t n_tok, int64_t d_in) {
    if (n_tok <= 0 || d_in <= 0 || bad_dim(n_tok) || bad_dim(d_in)) return 0;
    return chan_abs_ws_bytes(n_tok, d_in);
}

pwq_status pwq_channel_abs_mean(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, float* abs_mean,
                                void* ws, size_t ws_bytes, void* stream) {
    if (x_dtype != PWQ_F32 && x_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (n_tok <= 0 || bad_dim(n_tok) || n_tok > (int64_t)65535 * 1024 || d_in <= 0 || bad_dim(d_in) || ldx < d_in)
        return PWQ_EINVAL;
    if (!X || !abs_mean) return PWQ_EINVAL;
    if (!ws || ws_bytes < pwq_channel_abs_mean_workspace_size(n_tok, d_in)) return PWQ_EWORKSPACE;
    return hip_status(chan_abs_launch(X, x_dtype, n_tok, d_in, ldx, abs_mean, ws, (hipStream_t)stream));
}

size_t pwq_awq_search_workspace_size(int64_t d_out, int64_t d_in) {
    if (d_out <= 0 || d_in <= 0 || bad_dim(d_out) || bad_dim(d_in)) return 0;
    return awq_ws_bytes(d_out, d_in);
}

pwq_status pwq_awq_search(const void* W, int w_dtype, int64_t d_out, int64_t d_in, int64_t ldw, const float* H,
                          int64_t n_tok, const float* abs_mean, int32_t bits, int32_t group_size, int32_t n_alpha,
                          int32_t zero_point, double* mse_out, int32_t* best_out, float* s_out, void* codes,
                          uint8_t* packed, uint16_t* scales_out, uint16_t* zeros_out, void* ws, size_t ws_bytes,
                          void* stream) {
    if (w_dtype != PWQ_F32 && w_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (d_out <= 0 || bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldw < d_in || n_tok <= 0) return PWQ_EINVAL;
    if (bits < 2 || bits > 8 || !group_ok(group_size, d_in) || n_alpha < 1 || n_alpha > 1024) return PWQ_EINVAL;
    if (!W || !H || !abs_mean || !mse_out || !best_out || !s_out || !scales_out || (!codes && !packed))
        return PWQ_EINVAL;
    if (zero_point && !zeros_out) return PWQ_EINVAL;
    if (packed && (bits != 4 || d_in % 2 != 0)) return PWQ_EINVAL;
    if (!ws || ws_bytes < pwq_awq_search_workspace_size(d_out, d_in)) return PWQ_EWORKSPACE;
    return hip_status(awq_launch(W, w_dtype, d_out, d_in, ldw, H, n_tok, abs_mean, bits, group_size, n_alpha,
                                 zero_point != 0, mse_out, best_out, s_out, (int8_t*)codes, packed, scales_out,
                                 zero_point ? zeros_out : nullptr, ws, (hipStream_t)stream));
}

// ------------------------------------------------------------------ product with What
size_t pwq_quantized_matmul_workspace_size(int64_t n_tok, int64_t d_in, int64_t d_out) {
    if (n_tok <= 0 || d_in <= 0 || d_out <= 0 || bad_dim(n_tok) || bad_dim(d_in) || bad_dim(d_out)) return 0;
    return w4a16_ws_bytes(n_tok, d_in, d_out);
}

pwq_status pwq_quantized_matmul(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                                const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                                int64_t d_out, int32_t group_size, void* Y, int y_dtype, int64_t ldy,
                                void* ws, size_t ws_bytes, void* stream) {
    if (x_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (y_dtype != PWQ_F32 && y_dtype != PWQ_F16 && y_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (bad_dim(n_tok) || bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldx < d_in || ldy < d_out) return PWQ_EINVAL;
    if (n_tok > (int64_t)65535 * 16 || d_in % 32 != 0 || ldx % 8 != 0 || ldx > QMM_MAX_COLS) return PWQ_EINVAL;
    if (group_size != 0 && (group_size < 0 || group_size % 128 != 0)) return PWQ_EINVAL;
    if (n_tok == 0 || d_out == 0) return PWQ_OK;
    if (!packed || !scales || !Y) return PWQ_EINVAL;
    if (!X || !aligned(X, 16) || !aligned(packed, 16)) return PWQ_EINVAL;
    const size_t need = pwq_quantized_matmul_workspace_size(n_tok, d_in, d_out);
    if (need && (!ws || ws_bytes < need)) return PWQ_EWORKSPACE;
    return hip_status(w4a16_launch((const uint16_t*)X, n_tok, d_in, ldx, packed, scales, zeros, d_out, group_size, Y,
                                   y_dtype, ldy, ws, (hipStream_t)stream));
}

pwq_status pwq_quantized_matmul_noalloc(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx,
                                        const uint8_t* packed, const uint16_t* scales, const uint16_t* zeros,
                                        int64_t d_out, int32_t group_size, void* Y, int y_dtype, int64_t ldy,
                                        void* stream) {
    if (x_dtype != PWQ_F16) return PWQ_EDTYPE;
    if (y_dtype != PWQ_F32 && y_dtype != PWQ_F16 && y_dtype != PWQ_BF16) return PWQ_EDTYPE;
    if (bad_dim(n_tok) || bad_dim(d_out) || d_in <= 0 || bad_dim(d_in) || ldx < d_in || ldy < d_out) return PWQ_EINVAL;
    if (n_tok > (int64_t)65535 * 16 || d_in % 32 != 0 || ldx % 8 != 0 || ldx > QMM_MAX_COLS) return PWQ_EINVAL;
    if (group_size != 0 && (group_size < 0 || group_size % 128 != 0)) return PWQ_EINVAL;
    if (n_tok == 0 || d_out == 0) return PWQ_OK;
    if (!packed || !scales || !Y) return PWQ_EINVAL;
    if (!X || !aligned(X, 16) || !aligned(packed, 16)) return PWQ_EINVAL;
    const size_t need = pwq_quantized_matmul_workspace_size(n_tok, d_in, d_out);
    if (need > PWQ_QMM_SCRATCH_BYTES) return PWQ_EWORKSPACE;
    void* ws = nullptr;
    if (need) {
        const hipError_t e = w4a16_scratch(&ws);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(w4a16_launch((const uint16_t*)X, n_tok, d_in, ldx, packed, scales, zeros, d_out, group_size, Y,
                                   y_dtype, ldy, ws, (hipStream_t)stream));
}

}  // extern "C"
