// Activation-aware channel scaling ("Model Quantization Mechanics", 2.2 "AWQ"; the AWQ-style
// extension of "GPT-2 Quantization Reconstruction Error", "Possible extensions"): input
// channels whose activations are large are scaled up in W (and down in X) before RTN.
//
// The size of channel c is a_c = mean over tokens of |X_tc|; a candidate alpha gives
// s_c = a_c^alpha (1 where a_c = 0), and is scored by the reconstruction MSE of
// What = RTN(W diag(s)) diag(1/s) against W on the calibration set.  With H = 2 X^T X that
// MSE is tr(dW H dW^T) / (2 N m), dW = W - What, so each candidate costs one m x n x n
// product instead of a pass over the N tokens (N >> n for the large layers): on the float32
// MFMA engine, or from 256 output tiles of 256 x 256 on as the MSE's split bfloat16 product
// over one triangle of H (H's pieces formed once per search).  The grid is alpha = k / (K - 1); the least score wins, ties to the smaller
// alpha; the winner's W diag(s) is then quantized by the RTN kernels.
//
// Kernels: channel sums of |X| (float64 per token chunk, chunks added in order), the scale
// vector (double pow, rounded once to float32), dW per candidate (the RTN segment walk of
// rtn.hip with a column scale), the product with its summing epilogue, and small fixed-order
// reductions.
#include "gemm_f32.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int CHAN_CHUNK = 1024;     // tokens per partial sum of |X|

// part[chunk][c] = sum over the chunk's tokens of |X_tc| in float64, one thread per column
template <int DT>
__global__ __launch_bounds__(256) void chan_abs_kernel(const void* __restrict__ Xv, int64_t ldx, int64_t N, int64_t n,
                                                       double* __restrict__ part) {
    typedef typename Elem<DT>::T T;
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n) return;
    const int64_t t0 = (int64_t)blockIdx.y * CHAN_CHUNK;
    const int64_t t1 = t0 + CHAN_CHUNK < N ? t0 + CHAN_CHUNK : N;
    const T* X = (const T*)Xv;
    double s = 0.0;
#pragma unroll 8
    for (int64_t t = t0; t < t1; ++t) s += (double)fabsf(Elem<DT>::get(X, t * ldx + c));
    part[blockIdx.y * n + c] = s;
}

__global__ __launch_bounds__(256) void chan_mean_kernel(const double* __restrict__ part, int64_t nchunks, int64_t N,
                                                        int64_t n, float* __restrict__ a) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n) return;
    double s = 0.0;
    for (int64_t k = 0; k < nchunks; ++k) s += part[k * n + c];
    a[c] = (float)(s / (double)N);
}

// s_c = a_c^alpha (float64 pow, one rounding to float32), 1 where a_c = 0; alpha = k / (K - 1)
// with k given, or read from *best when best is not NULL
__global__ __launch_bounds__(256) void awq_scale_kernel(const float* __restrict__ a, int64_t n, int k, int K,
                                                        const int32_t* __restrict__ best, float* __restrict__ s) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= n) return;
    const int kk = best ? *best : k;
    const double alpha = K > 1 ? (double)kk / (double)(K - 1) : 0.0;
    const float ac = a[c];
    s[c] = ac > 0.f ? (float)pow((double)ac, alpha) : 1.f;
}

struct AwqArgs {
    const void* W;
    int64_t ldw, m, n, ng, nseg;
    int gl, L, qmax, top, vec;
    const float* s;       // column scales
    float* out;           // dW (m x n, ld n), or W diag(s) when scaled_only
    int scaled_only;
};

template <int DT>
__device__ __forceinline__ float4 load_q(const typename Elem<DT>::T* row, int64_t c, int64_t c1, bool vec) {
    if (vec && c + 3 < c1) return Elem<DT>::get4(row, c);
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = c + k < c1 ? Elem<DT>::get(row, c + k) : 0.f;
    return make_float4(t[0], t[1], t[2], t[3]);
}

// One segment (row, group) per L lanes.  ws = fp32(w * s_c); the group's quantizer from ws by
// the RTN rules; What_c = fp32(S (q - Z)) / s_c; out = w - What_c.  scaled_only: out = ws.
template <int DT, bool ZP>
__global__ __launch_bounds__(256) void awq_delta_kernel(AwqArgs a) {
    typedef typename Elem<DT>::T T;
    const int lane = threadIdx.x & 63;
    const int L = a.L, spw = 64 / L;
    const int sub = lane / L, li = lane % L;
    const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int64_t iters = cdiv(a.nseg, spw);
    for (int64_t it = wave_id; it < iters; it += nwaves) {
        const int64_t seg = it * spw + sub;
        const bool live = seg < a.nseg;
        const int64_t r = live ? seg / a.ng : 0, G = live ? seg % a.ng : 0;
        const int64_t c0 = G * a.gl;
        const int64_t c1 = live ? (c0 + a.gl < a.n ? c0 + a.gl : a.n) : c0;
        const T* row = (const T*)a.W + r * a.ldw;
        float* orow = a.out + r * a.n;
        if (a.scaled_only) {
            for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L) {
                const float4 v = load_q<DT>(row, c, c1, a.vec);
                const float vv[4] = {v.x, v.y, v.z, v.w};
                for (int k = 0; k < 4; ++k)
                    if (c + k < c1) orow[c + k] = vv[k] * a.s[c + k];
            }
            continue;
        }
        float hi = 0.f, nlo = 0.f;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L) {
            const float4 v = load_q<DT>(row, c, c1, a.vec);
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float x = c + k < c1 ? vv[k] * a.s[c + k] : 0.f;
                if (ZP) { hi = fmaxf(hi, x); nlo = fmaxf(nlo, -x); }
                else hi = fmaxf(hi, fabsf(x));
            }
        }
        hi = group_max(hi, L);
        if (ZP) nlo = group_max(nlo, L);
        const uint16_t sb = ZP ? zp_scale_bits(nlo, hi, a.top) : scale_bits_from_absmax(hi, a.qmax);
        const float S = f16_bits_to_f32(sb);
        const float rs = S > 0.f ? 1.0f / S : 0.f;
        const float z = ZP ? zp_zero(nlo, S, (float)a.top) : 0.f;
        const float qlo = ZP ? -z : -(float)a.qmax, qhi = ZP ? (float)a.top - z : (float)a.qmax;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L) {
            const float4 v = load_q<DT>(row, c, c1, a.vec);
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (!live || c + k >= c1) continue;
                const float sc = a.s[c + k];
                const float x = vv[k] * sc;
                const float qd = S > 0.f ? round_quot_clamp(x, S, rs, qlo, qhi) : 0.f;   // q - z
                orow[c + k] = vv[k] - (S * qd) / sc;                                        // S (q - z) is exact
            }
        }
    }
}

// mse[k] = sum of the parts in order / denom
__global__ __launch_bounds__(256) void awq_score_kernel(const double* __restrict__ part, int64_t nparts, double denom,
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

// the first minimum of mse[0 .. K)
__global__ void awq_argmin_kernel(const double* __restrict__ mse, int K, int32_t* __restrict__ best) {
    int b = 0;
    for (int k = 1; k < K; ++k)
        if (mse[k] < mse[b]) b = k;
    *best = b;
}

template <int BM, int BN>
hipError_t awq_product(const float* dW, const float* H, int64_t m, int64_t n, double* part, int64_t* nparts,
                       hipStream_t s) {
    const int vec = (int)((n % 4 == 0) && aligned(dW, 16) && aligned(H, 16));
    OpMMajor<0> la{dW, n, m, n, vec};
    OpKMajor<0> lb{H, n, n, n, vec};
    RectMap mp{};
    mp.M = m; mp.N = n; mp.K = n;
    mp.tiles_m = (int)cdiv(m, BM);
    mp.tiles_n = (int)cdiv(n, BN);
    mp.splits = 1;
    mp.kchunk = cdiv(n, GEMM_BK) * GEMM_BK;
    mp.tri_k = 0;
    mp.guard = nullptr;
    EpiTrace ep{dW, n, m, n, part, nullptr, 0.f};
    *nparts = (int64_t)mp.tiles_m * mp.tiles_n;
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, OpMMajor<0>, OpKMajor<0>, RectMap, EpiTrace>), dim3((unsigned)*nparts),
                       dim3(GEMM_THREADS), 0, s, la, lb, mp, ep);
    return hipGetLastError();
}

int64_t awq_tiles(int64_t m, int64_t n) {
    const int64_t big = cdiv(m, 128) * cdiv(n, 128);
    return big >= 512 ? big : cdiv(m, 64) * cdiv(n, 64);
}

}  // namespace

size_t chan_abs_ws_bytes(int64_t N, int64_t n) { return (size_t)cdiv(N, CHAN_CHUNK) * (size_t)n * sizeof(double); }

hipError_t chan_abs_launch(const void* X, int x_dtype, int64_t N, int64_t n, int64_t ldx, float* a, void* ws,
                           hipStream_t s) {
    const int64_t nchunks = cdiv(N, CHAN_CHUNK);
    double* part = (double*)ws;
    const dim3 grid((unsigned)cdiv(n, 256), (unsigned)nchunks);
    if (x_dtype == 0) hipLaunchKernelGGL(chan_abs_kernel<0>, grid, dim3(256), 0, s, X, ldx, N, n, part);
    else hipLaunchKernelGGL(chan_abs_kernel<2>, grid, dim3(256), 0, s, X, ldx, N, n, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chan_mean_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, part, nchunks, N, n, a);
    return hipGetLastError();
}

// workspace: dW / W diag(s) (m x n float32), s (n float32), the product's partial sums; on
// the split route (large layers) then dW's and G's bfloat16 pieces
size_t awq_ws_bytes(int64_t m, int64_t n) {
    const bool sp = split_route(m, n);
    const int64_t tiles = sp ? split_tiles(m, n) : awq_tiles(m, n);
    size_t b = align_up((size_t)m * n * sizeof(float), 256) + align_up((size_t)n * sizeof(float), 256) +
               align_up((size_t)tiles * sizeof(double), 256);
    if (sp) b += split_pieces_bytes(m, n) + split_g_bytes(n);
    return b;
}

hipError_t awq_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* H, int64_t N,
                      const float* absmean, int bits, int group_size, int K, int zp, double* mse, int32_t* best,
                      float* s_out, int8_t* codes, uint8_t* packed, uint16_t* scales, uint16_t* zeros, void* ws,
                      hipStream_t s) {
    hipError_t e;
    char* base = (char*)ws;
    float* dW = (float*)base;
    float* sv = (float*)(base + align_up((size_t)m * n * sizeof(float), 256));
    double* part = (double*)(base + align_up((size_t)m * n * sizeof(float), 256) + align_up((size_t)n * sizeof(float), 256));
    const bool sp = split_route(m, n);
    uint16_t* a3 = nullptr;
    uint16_t* b3 = nullptr;
    if (sp) {
        a3 = (uint16_t*)((char*)part + align_up((size_t)split_tiles(m, n) * sizeof(double), 256));
        b3 = (uint16_t*)((char*)a3 + split_pieces_bytes(m, n));
        if ((e = split_g_launch(H, n, n, b3, s)) != hipSuccess) return e;
    }

    AwqArgs a{};
    a.W = W; a.ldw = ldw; a.m = m; a.n = n;
    a.gl = group_size == 0 ? (int)n : group_size;
    a.ng = group_size == 0 ? 1 : cdiv(n, group_size);
    a.nseg = m * a.ng;
    int L = 1;
    while (L < 64 && 4 * L < a.gl) L <<= 1;
    a.L = L;
    a.qmax = (1 << (bits - 1)) - 1;
    a.top = (1 << bits) - 1;
    const size_t es = w_dtype == 0 ? 4 : 2;
    a.vec = (ldw % 4 == 0) && (a.gl % 4 == 0) && aligned(W, 4 * es);
    a.s = sv;
    a.out = dW;
    int64_t blocks = cdiv(cdiv(a.nseg, 64 / L), 4);
    if (blocks > 65536) blocks = 65536;
    const unsigned sg = (unsigned)cdiv(n, 256);
    auto delta = [&]() {
        if (w_dtype == 0) {
            if (zp) hipLaunchKernelGGL((awq_delta_kernel<0, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
            else hipLaunchKernelGGL((awq_delta_kernel<0, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        } else {
            if (zp) hipLaunchKernelGGL((awq_delta_kernel<1, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
            else hipLaunchKernelGGL((awq_delta_kernel<1, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        }
        return hipGetLastError();
    };
    const bool big = cdiv(m, 128) * cdiv(n, 128) >= 512;
    for (int k = 0; k < K; ++k) {
        hipLaunchKernelGGL(awq_scale_kernel, dim3(sg), dim3(256), 0, s, absmean, n, k, K, (const int32_t*)nullptr, sv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        a.scaled_only = 0;
        if ((e = delta()) != hipSuccess) return e;
        int64_t np = 0;
        if (sp) {
            // large layers: the split bfloat16 product over one triangle of H (G's pieces formed once)
            if ((e = split_pieces_launch(dW, n, m, n, a3, s)) != hipSuccess) return e;
            np = split_tiles(m, n);
            e = split_trace_launch(a3, b3, dW, n, m, n, nullptr, part, s);
        } else {
            e = big ? awq_product<128, 128>(dW, H, m, n, part, &np, s) : awq_product<64, 64>(dW, H, m, n, part, &np, s);
        }
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(awq_score_kernel, dim3(1), dim3(256), 0, s, part, np, 2.0 * (double)N * (double)m, mse + k);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(awq_argmin_kernel, dim3(1), dim3(1), 0, s, mse, K, best);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(awq_scale_kernel, dim3(sg), dim3(256), 0, s, absmean, n, 0, K, (const int32_t*)best, s_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.s = s_out;
    a.scaled_only = 1;                                       // W diag(s) of the winner, float32, in dW's place
    if ((e = delta()) != hipSuccess) return e;
    return rtn_launch(dW, 0, m, n, n, bits, group_size, nullptr, codes, packed, scales, s, nullptr, zp ? zeros : nullptr);
}

}  // namespace pwq
