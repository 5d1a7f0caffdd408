// GPTQ column loop ("GPTQ: Post-Training INT4", section "The GPTQ Algorithm"): columns in
// processing order, blocks of B, per column quantize / scaled error / in-block rank-1
// update, then one trailing product per block.  Scales follow "Group Quantization" of the
// same page (one float16 scale per row and group) and the per-row quantizer of
// "GPT-2 Quantization Reconstruction Error".
//
// Kernels per layer:
//   prologue : float32 working copy Wf of W (columns permuted for act-order), per-row
//              scales from the original row, copy of caller-fixed scales
//   block    : one wave64 per row; lane l holds panel columns l and l+64 in registers, the
//              B x B diagonal block of U sits in LDS.  For each column j the owner value is
//              broadcast with readlane, quantized (exact-quotient rounding), e = (w - s q) /
//              U_jj, and every lane applies w -= e U[j][col] to its two columns (U is upper
//              triangular, so columns <= j are unaffected or already final).  Group scales
//              are a wave max-reduction over the group's current values.  Writes codes (or
//              INT4 nibbles directly), scales, and the error panel Err (m x B).
//   trailing : Wf[:, end:] -= Err U[block, end:]  (float32 MFMA engine)
//   finish   : act-order only: codes back to the original column order, nibble packing and
//              g_idx.
#include "gemm_f32.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int GB = 128;   // panel width held per wave (two columns per lane)

template <int DT, bool PERM>
__global__ __launch_bounds__(256) void gptq_prologue_kernel(const void* __restrict__ W, int64_t ldw, int64_t m, int64_t n,
                                                            const int32_t* __restrict__ perm, float* __restrict__ Wf,
                                                            int row_scales, int qmax, const uint16_t* __restrict__ scales_in,
                                                            uint16_t* __restrict__ scales_out, int64_t ng,
                                                            const int32_t* __restrict__ info) {
    if (*info) return;
    typedef typename Elem<DT>::T T;
    __shared__ float row[PERM ? PERM_MAX_N : 1];
    __shared__ float red[4];
    const int64_t r = blockIdx.x;
    const T* src = (const T*)W + r * ldw;
    float* dst = Wf + r * n;
    float amax = 0.f;
    if (PERM) {
        for (int64_t j = threadIdx.x; j < n; j += 256) {
            const float v = Elem<DT>::get(src, j);
            row[j] = v;
            amax = fmaxf(amax, fabsf(v));
        }
        __syncthreads();
        for (int64_t p = threadIdx.x; p < n; p += 256) dst[p] = row[perm[p]];
    } else {
        for (int64_t j = threadIdx.x; j < n; j += 256) {
            const float v = Elem<DT>::get(src, j);
            dst[j] = v;
            amax = fmaxf(amax, fabsf(v));
        }
    }
    if (scales_in) {
        for (int64_t g = threadIdx.x; g < ng; g += 256) scales_out[r * ng + g] = scales_in[r * ng + g];
    } else if (row_scales) {
        amax = wave_max(amax);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
        __syncthreads();
        if (threadIdx.x == 0) {
            const float a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            scales_out[r] = scale_bits_from_absmax(a, qmax);
        }
    }
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

struct BlockArgs {
    float* Wf;
    const float* U;
    const int32_t* info;
    int64_t m, n, b0;
    int bw, group_size, qmax, fixed_scales, rows_per_wave;
    int gsmall, glog, gstart0;   // g <= B: groups start where (j & (g-1)) == 0; g > B: at j == 0 iff gstart0
    int64_t gbase;               // group index of the panel's first column
    uint16_t* scales;        // d_out x ng (already holds per-row / fixed scales)
    int64_t ng;
    int8_t* codes;           // processing order, ld n (nullable)
    uint8_t* packed;         // ld n/2 (nullable; only without act-order)
    float* err;              // m x GB
};

// NS = 1: panel of 64 columns (block sizes 32 and 64), NS = 2: 128 columns.
template <int NT, int NS>
__global__ __launch_bounds__(NT) void gptq_block_kernel(BlockArgs a) {
    if (*a.info) return;
    constexpr int PW = 64 * NS;
    constexpr int NW = NT / 64;
    __shared__ __attribute__((aligned(16))) float Ub[PW][PW];
    __shared__ float dinv[PW];
    __shared__ float esh[NW][PW];      // per-wave staging of the column results
    __shared__ int8_t qsh[NW][PW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // diagonal block of U, zero outside the bw x bw panel (so padded columns never move)
    {
        constexpr int Q = PW * PW / 4 / NT;          // float4 per thread
        if (a.bw == PW && (a.n % 4 == 0)) {          // full panel: plain 16-byte loads
            float4 v[Q];
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int e = (tid + q * NT) * 4;
                v[q] = *(const float4*)(a.U + (a.b0 + e / PW) * a.n + a.b0 + e % PW);
            }
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int e = (tid + q * NT) * 4;
                *(float4*)&Ub[e / PW][e % PW] = v[q];
            }
        } else {                                     // ragged last panel
            for (int e = tid; e < PW * PW; e += NT) {
                const int j = e / PW, c = e % PW;
                Ub[j][c] = (j < a.bw && c < a.bw) ? a.U[(a.b0 + j) * a.n + a.b0 + c] : 0.f;
            }
        }
        for (int j = tid; j < PW; j += NT) dinv[j] = j < a.bw ? 1.0f / a.U[(a.b0 + j) * a.n + a.b0 + j] : 0.f;
    }
    __syncthreads();

    const int g = a.group_size;
    const int64_t rbase = (int64_t)blockIdx.x * NW * a.rows_per_wave;
    // columns sharing one scale inside the panel: a group (g <= B) or the whole panel
    const int seg = (g != 0 && a.gsmall) ? g : PW;
    for (int rr = 0; rr < a.rows_per_wave; ++rr) {
        const int64_t r = rbase + (int64_t)rr * NW + wave;
        if (r >= a.m) break;
        float* wrow = a.Wf + r * a.n;
        float w[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) w[k] = lane + 64 * k < a.bw ? wrow[a.b0 + 64 * k + lane] : 0.f;
        float s = 0.f, rs = 0.f;
        if (g == 0) {
            s = f16_bits_to_f32(a.scales[r]);
        } else if (!a.gsmall && !a.gstart0) {
            // a group wider than the panel that began in an earlier panel: its scale was
            // fixed (and stored) when the loop reached the group's first column
            s = f16_bits_to_f32(a.scales[r * a.ng + a.gbase]);
        }
        for (int j0 = 0; j0 < a.bw; j0 += seg) {
            if (g != 0 && (a.gsmall || (j0 == 0 && a.gstart0))) {
                const int64_t col = a.b0 + j0;
                const int64_t G = a.gbase + (a.gsmall ? (j0 >> a.glog) : 0);
                uint16_t sb;
                if (a.fixed_scales) {
                    sb = a.scales[r * a.ng + G];
                } else {
                    // current values of the group's columns: panel columns [j0, j0+g) and, for a
                    // group wider than the panel (it then starts at the panel's first column),
                    // the columns right of the panel, which hold every earlier update
                    const int64_t gend = col + g < a.n ? col + g : a.n;
                    float v = 0.f;
#pragma unroll
                    for (int k = 0; k < NS; ++k) {
                        const int c = lane + 64 * k;
                        if (c >= j0 && a.b0 + c < gend && c < a.bw) v = fmaxf(v, fabsf(w[k]));
                    }
                    for (int64_t c = a.b0 + a.bw + lane; c < gend; c += 64) v = fmaxf(v, fabsf(wrow[c]));
                    v = wave_max(v);
                    sb = scale_bits_from_absmax(v, a.qmax);
                    if (lane == 0) a.scales[r * a.ng + G] = sb;
                }
                s = f16_bits_to_f32(sb);
            }
            rs = s > 0.f ? 1.0f / s : 0.f;
            const int j1 = j0 + seg < a.bw ? j0 + seg : a.bw;
            // one column per step; wj, s and rs are the same in every lane, so the branches
            // are uniform.  Columns [0, 64) live in w[0], [64, 128) in w[1].
            auto column = [&](int j, float wj) {
                int q = 0;
                if (s > 0.f) {
                    const float t = wj * rs;
                    const float lim = (float)(a.qmax + 1);
                    const float k = fminf(fmaxf(rintf(t), -lim), lim);
                    // |t - w/s| < 2e-6 here, so a distance below 0.49 from k already decides the
                    // nearest integer; only quotients near a half take the exact residual test
                    q = fabsf(t - k) <= 0.49f ? (int)fminf(fmaxf(k, (float)-a.qmax), (float)a.qmax)
                                              : quant_code(wj, s, rs, a.qmax);
                }
                const float e = (wj - s * (float)q) * dinv[j];
                if (lane == 0) {
                    esh[wave][j] = e;
                    qsh[wave][j] = (int8_t)q;
                }
                return e;
            };
            const int jm = j1 < 64 ? j1 : 64;
#pragma unroll 4
            for (int j = j0; j < jm; ++j) {
                const float e = column(j, readlane_f(w[0], j));
#pragma unroll
                for (int k = 0; k < NS; ++k) w[k] = fmaf(-e, Ub[j][64 * k + lane], w[k]);
            }
            if (NS == 2) {
#pragma unroll 4
                for (int j = j0 > 64 ? j0 : 64; j < j1; ++j) {
                    const float e = column(j, readlane_f(w[NS - 1], j - 64));
                    w[NS - 1] = fmaf(-e, Ub[j][64 * (NS - 1) + lane], w[NS - 1]);
                }
            }
        }
        float e_own[NS];
        int q_own[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            e_own[k] = esh[wave][64 * k + lane];
            q_own[k] = qsh[wave][64 * k + lane];
        }
        float* erow = a.err + r * GB;
#pragma unroll
        for (int k = 0; k < NS; ++k) erow[64 * k + lane] = e_own[k];
        if (NS == 1) erow[64 + lane] = 0.f;
        if (a.codes) {
            int8_t* crow = a.codes + r * a.n + a.b0;
#pragma unroll
            for (int k = 0; k < NS; ++k)
                if (lane + 64 * k < a.bw) crow[64 * k + lane] = (int8_t)q_own[k];
        }
        if (a.packed) {
            // byte l of the panel holds columns 2l (low nibble) and 2l+1 (high nibble)
            const int src = (2 * lane) & 63;
            const int lo0 = __shfl(q_own[0], src, 64), hi0 = __shfl(q_own[0], src + 1, 64);
            int lo = lo0, hi = hi0;
            if (NS == 2) {
                const int lo1 = __shfl(q_own[NS - 1], src, 64), hi1 = __shfl(q_own[NS - 1], src + 1, 64);
                lo = lane < 32 ? lo0 : lo1;
                hi = lane < 32 ? hi0 : hi1;
            }
            if (2 * lane < a.bw && (NS == 2 || lane < 32))
                a.packed[r * (a.n / 2) + a.b0 / 2 + lane] = (uint8_t)((lo + 8) | ((hi + 8) << 4));
        }
    }
}

// Wf[r][c0 + col] -= acc
struct EpiSub {
    float* out;
    int64_t ld, M, N;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row < M && col < N) out[row * ld + col] -= v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

__global__ __launch_bounds__(256) void inv_perm_kernel(const int32_t* __restrict__ perm, int64_t n, int g,
                                                       int32_t* __restrict__ inv, int32_t* __restrict__ g_idx) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n) return;
    const int32_t c = perm[p];
    inv[c] = (int32_t)p;
    g_idx[c] = g == 0 ? 0 : (int32_t)(p / g);
}

// codes back to original column order (row staged in LDS) + optional nibble packing
__global__ __launch_bounds__(256) void unpermute_codes_kernel(const int8_t* __restrict__ cp, const int32_t* __restrict__ inv,
                                                              int64_t n, int8_t* __restrict__ codes, uint8_t* __restrict__ packed,
                                                              const int32_t* __restrict__ info) {
    if (*info) return;
    __shared__ int8_t row[PERM_MAX_N];
    const int64_t r = blockIdx.x;
    for (int64_t j = threadIdx.x; j < n; j += 256) row[j] = cp[r * n + j];
    __syncthreads();
    if (codes)
        for (int64_t c = threadIdx.x; c < n; c += 256) codes[r * n + c] = row[inv[c]];
    if (packed)
        for (int64_t b = threadIdx.x; b < n / 2; b += 256) {
            const int lo = row[inv[2 * b]], hi = row[inv[2 * b + 1]];
            packed[r * (n / 2) + b] = (uint8_t)((lo + 8) | ((hi + 8) << 4));
        }
}

template <int BM, int BN>
hipError_t trailing(float* Wf, const float* err, const float* U, const int32_t* info, int64_t m, int64_t n, int64_t b0,
                    int64_t b1, int bw, hipStream_t s) {
    const int64_t N = n - b1;
    OpMMajor<0> a{err, GB, m, bw, 1};
    OpKMajor<0> b{U + b0 * n + b1, n, N, bw, (int)((n % 4 == 0) && aligned(U, 16) && (b1 % 4 == 0))};
    RectMap mp{};
    mp.M = m; mp.N = N; mp.K = bw;
    mp.tiles_m = (int)cdiv(m, BM);
    mp.tiles_n = (int)cdiv(N, BN);
    mp.splits = 1;
    mp.kchunk = cdiv(bw, GEMM_BK) * GEMM_BK;
    mp.tri_k = 0;
    mp.guard = info;
    EpiSub ep{Wf + b1, n, m, N};
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, OpMMajor<0>, OpKMajor<0>, RectMap, EpiSub>),
                       dim3(mp.tiles_m * mp.tiles_n), dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

}  // namespace

GptqWs gptq_ws_layout(int64_t d_out, int64_t d_in, int block_size, int act_order) {
    (void)block_size;
    GptqWs w{};
    size_t off = 0;
    w.wf = off;    off = align_up(off + (size_t)d_out * d_in * sizeof(float), 256);
    w.err = off;   off = align_up(off + (size_t)d_out * GB * sizeof(float), 256);
    w.codes = off; if (act_order) off = align_up(off + (size_t)d_out * d_in, 256);
    w.inv = off;   if (act_order) off = align_up(off + (size_t)d_in * sizeof(int32_t), 256);
    w.total = off;
    return w;
}

hipError_t gptq_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* U, const int32_t* info,
                       int bits, int group_size, int block_size, int act_order, const int32_t* perm,
                       const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out, int32_t* g_idx,
                       void* ws, hipStream_t s) {
    if (m == 0 || n == 0) return hipSuccess;
    hipError_t e;
    const GptqWs L = gptq_ws_layout(m, n, block_size, act_order);
    char* base = (char*)ws;
    float* Wf = (float*)(base + L.wf);
    float* err = (float*)(base + L.err);
    int8_t* cproc = act_order ? (int8_t*)(base + L.codes) : codes;
    int32_t* inv = act_order ? (int32_t*)(base + L.inv) : nullptr;
    const int qmax = (1 << (bits - 1)) - 1;
    const int64_t ng = group_size == 0 ? 1 : cdiv(n, group_size);

    {
        auto k = w_dtype == 0 ? (act_order ? gptq_prologue_kernel<0, true> : gptq_prologue_kernel<0, false>)
                              : (act_order ? gptq_prologue_kernel<1, true> : gptq_prologue_kernel<1, false>);
        hipLaunchKernelGGL(k, dim3((unsigned)m), dim3(256), 0, s, W, ldw, m, n, act_order ? perm : nullptr, Wf,
                           (int)(group_size == 0), qmax, scales_in, scales_out, ng, info);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    BlockArgs a{};
    a.Wf = Wf; a.U = U; a.info = info; a.m = m; a.n = n;
    a.group_size = group_size; a.qmax = qmax; a.fixed_scales = scales_in != nullptr;
    a.scales = scales_out; a.ng = ng; a.codes = cproc; a.packed = act_order ? nullptr : packed; a.err = err;
    const bool big = m > 4096;
    a.rows_per_wave = m > 8192 ? 2 : 1;
    const int nw = big ? 16 : 4;
    const unsigned nblk = (unsigned)cdiv(m, (int64_t)nw * a.rows_per_wave);
    const bool wide = block_size > 64;

    for (int64_t b0 = 0; b0 < n; b0 += block_size) {
        const int bw = (int)((n - b0) < block_size ? (n - b0) : block_size);
        a.b0 = b0;
        a.bw = bw;
        if (group_size != 0) {
            a.gsmall = group_size <= block_size;
            a.glog = 0;
            while ((1 << a.glog) < group_size) ++a.glog;
            a.gstart0 = (b0 % group_size) == 0;
            a.gbase = b0 / group_size;
        }
        if (big && wide) hipLaunchKernelGGL((gptq_block_kernel<1024, 2>), dim3(nblk), dim3(1024), 0, s, a);
        else if (big) hipLaunchKernelGGL((gptq_block_kernel<1024, 1>), dim3(nblk), dim3(1024), 0, s, a);
        else if (wide) hipLaunchKernelGGL((gptq_block_kernel<256, 2>), dim3(nblk), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((gptq_block_kernel<256, 1>), dim3(nblk), dim3(256), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t b1 = b0 + bw;
        if (b1 < n) {
            const int64_t big_tiles = cdiv(m, 128) * cdiv(n - b1, 128);
            e = big_tiles >= 512 ? trailing<128, 128>(Wf, err, U, info, m, n, b0, b1, bw, s)
                                 : trailing<64, 64>(Wf, err, U, info, m, n, b0, b1, bw, s);
            if (e != hipSuccess) return e;
        }
    }
    if (act_order) {
        hipLaunchKernelGGL(inv_perm_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, perm, n, group_size, inv, g_idx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(unpermute_codes_kernel, dim3((unsigned)m), dim3(256), 0, s, cproc, inv, n, codes, packed, info);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pwq
