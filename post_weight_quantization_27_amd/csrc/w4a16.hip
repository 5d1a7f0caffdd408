// Product with the quantized weights, Y = X What^T (tokens x d_out), What decoded on the fly
// from the INT4 nibbles, the float16 scales and, in the zero-point form, the zeros: the
// inference use of the quantized layer ("GPTQ: Post-Training INT4", "Running GPTQ with
// AutoGPTQ"; What as in "Model Quantization Mechanics", "Affine Quantization").
//
// Designed for few tokens (decode), where the 4-bit weights are the traffic: 0.5 byte per
// weight plus 2 (or 4) bytes per group.  Each wave owns 32 rows and 16 tokens and walks the
// columns of its split (at most 8 steps of 128) with every step's nibbles loaded up front.  The multiply runs on float16 MFMA 16x16x16 with the
// integer codes q - z as the weight operand: they are small integers, exact in float16, so the
// products x (q - z) are exact, and each group's sum is scaled once by its s (the algebra
// sum_c x s (q - z) = s sum_c x (q - z) with no rounding of What).  A group must therefore
// hold whole chunks: per-row scales or groups of a multiple of 128 columns.
//
// Decoding: a 32-bit word holds eight nibbles (columns c .. c+7, two per byte, even column
// low).  Masking gives the even-column nibbles in its bytes, a shift and mask the odd ones,
// and a byte permute against a word of 0x64 bytes turns two of those bytes into the float16
// pair (1024 + q, 1024 + q'); one packed float16 subtract of 1024 + z leaves (q - z)
// exactly.  The MFMA sums over its k in any order, so X's columns are paired the same way
// (one byte permute per pair, when X is staged) instead of moving nibbles.
//
// The columns are split in pieces of at most 1024; the splits' partial sums go to the
// workspace and one more pass adds them in split order (deterministic).
#include <mutex>

#include "../../include/pwq.h"
#include "pwq_internal.h"
#include "pwq_common.h"

// Partial sums of the allocation-free entry point: one copy per GPU, held until the process
// ends.  Host code never uses this name as an address (on the host it is a stand-in symbol);
// it takes each device's address from hipGetSymbolAddress (w4a16_scratch below).
static __device__ __align__(256) unsigned char scratch[PWQ_QMM_SCRATCH_BYTES];

namespace pwq {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int W4_CHUNK = 128;      // columns per step of a wave
constexpr int W4_ROWS = 32;        // rows per wave (two 16-row MFMA tiles)
constexpr int W4_TOK = 16;         // tokens per wave
constexpr int W4_MAXC = 8;         // steps per split (all loaded at once); 4 * 32 * W4_MAXC a multiple of 256
constexpr int64_t W4_MAX_COLS = (int64_t)1 << 24;   // d_in and ldx limit (32-bit buffer ranges)

struct W4Args {
    const uint16_t* X;             // float16 bits, T x n, leading dimension ldx
    int64_t ldx, T, n, m, ng;
    int64_t cpg;                   // steps of 128 columns per group (all of them for one scale per row)
    const uint8_t* packed;         // m x n/2
    const uint16_t* scales;        // m x ng float16 bits
    const uint16_t* zeros;         // m x ng (zero-point form) or NULL (symmetric: nibble - 8)
    int64_t cps;                   // chunks per split
    int splits;
    float* part;                   // splits > 1: splits x T x m float32 partial sums
    void* Y;
    int64_t ldy;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// Buffer loads with a range: an offset at or past `bytes` reads 0.  Loads that are out of
// range (past the rows, columns, tokens or steps of a workgroup) take W4_OOB as their
// offset instead of being skipped, so every load is issued unconditionally and the compiler
// can count the loads in flight (a load behind a branch makes it wait for all of them).
// Each range starts at the workgroup's first row or token, so it spans at most 128 rows or
// 16 tokens; d_in and ldx up to W4_MAX_COLS keep it below 2^31 bytes.
constexpr uint32_t W4_OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t w4_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 w4_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int YT>
__device__ __forceinline__ void store4(void* Y, int64_t off, const float* v, int cnt) {
    if (YT == 0) {
        float* y = (float*)Y + off;
        for (int e = 0; e < cnt; ++e) y[e] = v[e];
    } else {
        uint16_t* y = (uint16_t*)Y + off;
        for (int e = 0; e < cnt; ++e) y[e] = YT == 1 ? f32_to_f16_bits(v[e]) : f32_to_bf16_bits(v[e]);
    }
}

// Workgroup barrier without a memory fence (the nibble loads stay in flight across it); the
// LDS stores before it are waited for explicitly.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// grid: x = row blocks of 128 (four waves of 32 rows), y = splits of at most W4_MAXC steps,
// z = token tiles of 16.  The workgroup first issues the loads of the split's X (already
// paired for the B operand) and of its rows' scales and zeros, then every wave issues the
// loads of all its nibbles (16 KB); vector-memory waits are in order, so the staging waits
// only for its own loads, and each step then waits only for its own nibbles.
template <bool ZP, int YT>
__global__ __launch_bounds__(256) void w4a16_kernel(W4Args a) {
    // X of the split: [step][quarter][word][token] x 16 bytes = the B operands (x0,x2,x1,x3 | x4,x6,x5,x7)
    __shared__ uint4 xl[W4_MAXC * 4 * 4 * W4_TOK];
    __shared__ uint16_t sl[4 * W4_ROWS * W4_MAXC];                 // scales [row][group of the split]
    __shared__ uint16_t zl[ZP ? 4 * W4_ROWS * W4_MAXC : 1];         // zeros, same layout
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, q = lane >> 4;
    const int64_t R0 = (int64_t)blockIdx.x * 4 * W4_ROWS;
    const int64_t o0 = R0 + wave * W4_ROWS;
    const int64_t t0 = (int64_t)blockIdx.z * W4_TOK;
    const int64_t nchunks = cdiv(a.n, W4_CHUNK);
    const int64_t k0 = (int64_t)blockIdx.y * a.cps;
    const int nk = (int)(k0 + a.cps < nchunks ? a.cps : nchunks - k0);       // 1 .. W4_MAXC
    const int64_t G0 = k0 / a.cpg;
    const int ngs = (int)((k0 + nk - 1) / a.cpg - G0 + 1);                  // groups the split touches
    const int64_t half_n = a.n / 2;

    // 1. staging loads: thread tid holds (quarter, word, token) = (tid / 64, tid / 16 % 4, tid % 16)
    //    of every step, and up to four (row, group) scales and zeros
    uint4 xr[W4_MAXC];
    {
        const int tok = tid % W4_TOK, wd = (tid / W4_TOK) % 4, qq = tid / (4 * W4_TOK);
        const int64_t t = t0 + tok;
        const int64_t nt = a.T - t0 < W4_TOK ? a.T - t0 : W4_TOK;
        const __amdgpu_buffer_rsrc_t rx = w4_rsrc(a.X + t0 * a.ldx, ((nt - 1) * a.ldx + a.n) * 2);
#pragma unroll
        for (int c = 0; c < W4_MAXC; ++c) {
            const int64_t col = (k0 + c) * W4_CHUNK + 32 * qq + 8 * wd;
            const bool ok = c < nk && t < a.T && col < a.n;
            xr[c] = w4_load16(rx, ok ? (uint32_t)(((t - t0) * a.ldx + col) * 2) : W4_OOB);
        }
    }
    constexpr int SPT = 4 * W4_ROWS * W4_MAXC / 256;        // (row, group) entries per thread
    uint16_t sv[SPT], zv[SPT];
    const int64_t nrow = a.m - R0 < 4 * W4_ROWS ? a.m - R0 : 4 * W4_ROWS;     // rows of the workgroup
    const __amdgpu_buffer_rsrc_t rsc = w4_rsrc(a.scales + R0 * a.ng, nrow * a.ng * 2);
    const __amdgpu_buffer_rsrc_t rz = w4_rsrc((ZP ? a.zeros : a.scales) + R0 * a.ng, nrow * a.ng * 2);
#pragma unroll
    for (int c = 0; c < SPT; ++c) {
        const int idx = c * 256 + tid;
        const int row = idx / W4_MAXC, gg = idx % W4_MAXC;
        const int64_t o = R0 + row;
        const bool ok = gg < ngs && o < a.m;
        const uint32_t off = ok ? (uint32_t)(((o - R0) * a.ng + G0 + gg) * 2) : W4_OOB;
        sv[c] = __builtin_amdgcn_raw_buffer_load_b16(rsc, off, 0, 0);
        zv[c] = ZP ? __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0) : (uint16_t)0;
    }

    // 2. the nibbles of every step, for this lane's rows of both tiles
    int64_t orow[2];
    bool row_ok[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        orow[r] = o0 + 16 * r + i;
        row_ok[r] = orow[r] < a.m;
    }
    uint4 w[W4_MAXC][2];
    const __amdgpu_buffer_rsrc_t rw = w4_rsrc(a.packed + R0 * half_n, nrow * half_n);
#pragma unroll
    for (int c = 0; c < W4_MAXC; ++c) {
        const int64_t col = (k0 + c) * W4_CHUNK + 32 * q;
        const bool ok = c < nk && col < a.n;                // n % 32 == 0: a lane's 32 columns are all in or all out
#pragma unroll
        for (int r = 0; r < 2; ++r)
            w[c][r] = w4_load16(rw, (ok && row_ok[r]) ? (uint32_t)((orow[r] - R0) * half_n + col / 2) : W4_OOB);
    }

    // 3. staging stores: X paired (c, c+2), (c+1, c+3) per four columns, like the decoded nibbles
#pragma unroll
    for (int c = 0; c < W4_MAXC; ++c) {
        const uint4 u = xr[c];
        uint4 v;
        v.x = __builtin_amdgcn_perm(u.y, u.x, 0x05040100u);    // (x0, x2)
        v.y = __builtin_amdgcn_perm(u.y, u.x, 0x07060302u);    // (x1, x3)
        v.z = __builtin_amdgcn_perm(u.w, u.z, 0x05040100u);    // (x4, x6)
        v.w = __builtin_amdgcn_perm(u.w, u.z, 0x07060302u);    // (x5, x7)
        if (c < nk) xl[c * 256 + tid] = v;
    }
#pragma unroll
    for (int c = 0; c < SPT; ++c) {
        sl[c * 256 + tid] = sv[c];
        if (ZP) zl[c * 256 + tid] = zv[c];
    }
    lds_barrier();
    if (o0 >= a.m) return;                                  // wave-uniform; no barriers below

    // 4. per step: decode, 16 MFMAs, and at a group's end its scale
    float4_t acc[2], part[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) { acc[r] = (float4_t){0.f, 0.f, 0.f, 0.f}; part[r] = acc[r]; }
    const int lrow = wave * W4_ROWS;                        // this wave's first row in sl / zl
    auto zero_pair = [&](int r, int gg) -> half2_t {
        const float z = ZP ? (float)zl[(lrow + 16 * r + i) * W4_MAXC + gg] : 8.f;
        const _Float16 h = (_Float16)(-(1024.f + z));
        return (half2_t){h, h};
    };
    int gg = 0;
    int64_t left = a.cpg - (k0 - G0 * a.cpg);               // steps left in the first group
    half2_t zp[2] = {zero_pair(0, 0), zero_pair(1, 0)};
#pragma unroll
    for (int c = 0; c < W4_MAXC; ++c) {
        if (c < nk) {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
                const uint4 bv = xl[((c * 4 + q) * 4 + wd) * W4_TOK + i];
                const half4_t b0 = __builtin_bit_cast(half4_t, make_uint2(bv.x, bv.y));
                const half4_t b1 = __builtin_bit_cast(half4_t, make_uint2(bv.z, bv.w));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const uint32_t word = wd == 0 ? w[c][r].x : wd == 1 ? w[c][r].y : wd == 2 ? w[c][r].z : w[c][r].w;
                    // nibbles n0..n7 of columns c..c+7: lo bytes (n0, n2, n4, n6), hi bytes (n1, n3, n5, n7);
                    // a byte permute against 0x64 bytes makes the float16 pairs 1024 + n
                    const uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
                    const half2_t p02 = as_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) + zp[r];
                    const half2_t p46 = as_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) + zp[r];
                    const half2_t p13 = as_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) + zp[r];
                    const half2_t p57 = as_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) + zp[r];
                    const half4_t a0 = (half4_t){p02[0], p02[1], p13[0], p13[1]};   // columns 0, 2, 1, 3
                    const half4_t a1 = (half4_t){p46[0], p46[1], p57[0], p57[1]};   // columns 4, 6, 5, 7
                    part[r] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, b0, part[r], 0, 0, 0);
                    part[r] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, b1, part[r], 0, 0, 0);
                }
            }
            --left;
            if (left == 0 || c + 1 == nk) {                 // group end (or split end): scale once
#pragma unroll
                for (int r = 0; r < 2; ++r) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float sc = f16_bits_to_f32(sl[(lrow + 16 * r + 4 * q + e) * W4_MAXC + gg]);
                        acc[r][e] = fmaf(sc, part[r][e], acc[r][e]);
                        part[r][e] = 0.f;
                    }
                }
                if (left == 0 && c + 1 < nk) {
                    ++gg;
                    left = a.cpg;
                    zp[0] = zero_pair(0, gg);
                    zp[1] = zero_pair(1, gg);
                }
            }
        }
    }

    // 5. D layout: this lane holds rows 4 q + e (e < 4) of each tile, for token t0 + i
    const int64_t t = t0 + i;
    if (t >= a.T) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t ob = o0 + 16 * r + 4 * q;
        if (ob >= a.m) continue;
        const int cnt = a.m - ob < 4 ? (int)(a.m - ob) : 4;
        const float v[4] = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
        if (a.splits > 1) {
            float* p = a.part + ((int64_t)blockIdx.y * a.T + t) * a.m + ob;
            for (int e = 0; e < cnt; ++e) p[e] = v[e];
        } else {
            store4<YT>(a.Y, t * a.ldy + ob, v, cnt);
        }
    }
}

// Y[t][o] = sum over splits in order of part[s][t][o]; eight splits' loads in flight at a time
template <int YT>
__global__ __launch_bounds__(256) void w4a16_reduce_kernel(const float* __restrict__ part, int splits, int64_t T,
                                                           int64_t m, void* Y, int64_t ldy) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * m) return;
    const int64_t t = idx / m, o = idx - t * m;
    const int64_t stride = T * m;
    float s = 0.f;
    for (int k0 = 0; k0 < splits; k0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = k0 + k < splits ? part[(int64_t)(k0 + k) * stride + idx] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s += v[k];
    }
    store4<YT>(Y, t * ldy + o, &s, 1);
}

struct W4Plan {
    int64_t cps;
    int splits;
};

// splits of at most W4_MAXC steps (a wave holds all its nibbles in registers)
W4Plan w4_plan(int64_t T, int64_t n, int64_t m) {
    (void)T; (void)m;
    const int64_t nchunks = cdiv(n, W4_CHUNK);
    const int64_t s = cdiv(nchunks, W4_MAXC);
    const int64_t cps = cdiv(nchunks, s);
    return W4Plan{cps, (int)s};
}

}  // namespace

size_t w4a16_ws_bytes(int64_t T, int64_t n, int64_t m) {
    const W4Plan p = w4_plan(T, n, m);
    return p.splits > 1 ? (size_t)p.splits * (size_t)T * (size_t)m * sizeof(float) : 0;
}

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

hipError_t w4a16_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));     // this device is current
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t w4a16_launch(const uint16_t* X, int64_t T, int64_t n, int64_t ldx, const uint8_t* packed,
                        const uint16_t* scales, const uint16_t* zeros, int64_t m, int group_size, void* Y,
                        int y_dtype, int64_t ldy, void* ws, hipStream_t s) {
    if (T == 0 || m == 0) return hipSuccess;
    if (n > W4_MAX_COLS || ldx > W4_MAX_COLS) return hipErrorInvalidValue;
    const W4Plan p = w4_plan(T, n, m);
    W4Args a{};
    a.X = X; a.ldx = ldx; a.T = T; a.n = n; a.m = m;
    a.cpg = group_size == 0 ? cdiv(n, W4_CHUNK) : group_size / W4_CHUNK;
    a.ng = group_size == 0 ? 1 : cdiv(n, group_size);
    a.packed = packed; a.scales = scales; a.zeros = zeros;
    a.cps = p.cps; a.splits = p.splits;
    a.part = (float*)ws;
    a.Y = Y; a.ldy = ldy;
    const dim3 grid((unsigned)cdiv(m, 4 * W4_ROWS), (unsigned)p.splits, (unsigned)cdiv(T, W4_TOK));
#define PWQ_W4(ZPV, YTV) hipLaunchKernelGGL((w4a16_kernel<ZPV, YTV>), grid, dim3(256), 0, s, a)
    if (zeros) {
        if (y_dtype == 0) PWQ_W4(true, 0); else if (y_dtype == 1) PWQ_W4(true, 1); else PWQ_W4(true, 2);
    } else {
        if (y_dtype == 0) PWQ_W4(false, 0); else if (y_dtype == 1) PWQ_W4(false, 1); else PWQ_W4(false, 2);
    }
#undef PWQ_W4
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const unsigned rg = (unsigned)cdiv(T * m, 256);
    if (y_dtype == 0) hipLaunchKernelGGL(w4a16_reduce_kernel<0>, dim3(rg), dim3(256), 0, s, a.part, p.splits, T, m, Y, ldy);
    else if (y_dtype == 1) hipLaunchKernelGGL(w4a16_reduce_kernel<1>, dim3(rg), dim3(256), 0, s, a.part, p.splits, T, m, Y, ldy);
    else hipLaunchKernelGGL(w4a16_reduce_kernel<2>, dim3(rg), dim3(256), 0, s, a.part, p.splits, T, m, Y, ldy);
    return hipGetLastError();
}

}  // namespace pwq
