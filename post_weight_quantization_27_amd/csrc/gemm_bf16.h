// Tiled bfloat16 MFMA contraction engine for gfx950 (v_mfma_f32_32x32x16_bf16), float32
// accumulate:
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k)      (NSPLIT = 1)
//   acc(m, n) = sum_k A(m, k) * (Bhi(n, k) + Blo(n, k))      (NSPLIT = 2: B carried as a
//               bfloat16 pair hi + lo, so float32 B values keep 16 significant bits)
//
// 256 threads (4 wave64 in 2 x 2) own a BM x BN tile; a wave owns (BM/2) x (BN/2) as 32 x 32
// MFMA blocks.  Operand tiles of BK = 64 are staged in LDS as [row][k] with k contiguous
// (rows padded by 8 bfloat16 = 16 bytes, which keeps 16-byte fragment reads conflict free),
// so each lane reads its 8 consecutive k of a fragment with one 16-byte load.  The next
// k-tile is fetched into registers while the current one is multiplied.
#pragma once

#include "gemm_f32.h"

namespace pwq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BK16 = 64;             // k per LDS tile
constexpr int LROW = BK16 + 8;       // padded LDS row, in bfloat16

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------ loaders
// Element (m, k) at p[m * ld + k], bfloat16 (k contiguous): copied straight into [m][k].
struct Bf16MMajor {
    const uint16_t* p;
    int64_t ld, M, K;
    int vec;                         // ld % 8 == 0 and p 16-byte aligned
    template <int BM>
    struct Regs { uint4 v[BM * BK16 / 8 / GEMM_THREADS]; };
    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = BM * BK16 / 8 / GEMM_THREADS;
        const bool full = vec && (m0 + BM <= M) && (k0 + BK16 <= K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int row = idx >> 3, kc = (idx & 7) * 8;
            const int64_t m = m0 + row, k = k0 + kc;
            if (full) {
                r.v[i] = *(const uint4*)(p + m * ld + k);
            } else {
                uint32_t w[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t lo = (m < M && k + 2 * c < K) ? p[m * ld + k + 2 * c] : 0u;
                    const uint32_t hi = (m < M && k + 2 * c + 1 < K) ? p[m * ld + k + 2 * c + 1] : 0u;
                    w[c] = lo | (hi << 16);
                }
                r.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(uint16_t* S, const Regs<BM>& r, int tid) const {
        constexpr int NV = BM * BK16 / 8 / GEMM_THREADS;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int row = idx >> 3, kc = (idx & 7) * 8;
            *(uint4*)(S + row * LROW + kc) = r.v[i];
        }
    }
};

// Element (m, k) at p[k * ld + m], bfloat16 (m contiguous): each thread moves 8 x 8 blocks
// (8 rows of k, 8 consecutive m) and transposes them in registers into [m][k].
struct Bf16KMajor {
    const uint16_t* p;
    int64_t ld, M, K;
    int vec;
    int toff;                        // thread offset, so two operands spread over all threads
    template <int BM>
    struct Regs { uint4 v[8 * (BM * BK16 / 64 + GEMM_THREADS - 1) / GEMM_THREADS]; };
    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NB = BM * BK16 / 64;                // 8 x 8 blocks per tile
        constexpr int PER = (NB + GEMM_THREADS - 1) / GEMM_THREADS;
        const bool full = vec && (m0 + BM <= M) && (k0 + BK16 <= K);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int b = ((tid + toff) & (GEMM_THREADS - 1)) + q * GEMM_THREADS;
            if (b >= NB) break;
            const int mb = b % (BM / 8), kb = b / (BM / 8);
            const int64_t m = m0 + 8 * mb;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int64_t k = k0 + 8 * kb + rr;
                if (full) {
                    r.v[8 * q + rr] = *(const uint4*)(p + k * ld + m);
                } else {
                    uint32_t w[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t lo = (k < K && m + 2 * c < M) ? p[k * ld + m + 2 * c] : 0u;
                        const uint32_t hi = (k < K && m + 2 * c + 1 < M) ? p[k * ld + m + 2 * c + 1] : 0u;
                        w[c] = lo | (hi << 16);
                    }
                    r.v[8 * q + rr] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(uint16_t* S, const Regs<BM>& r, int tid) const {
        constexpr int NB = BM * BK16 / 64;
        constexpr int PER = (NB + GEMM_THREADS - 1) / GEMM_THREADS;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int b = ((tid + toff) & (GEMM_THREADS - 1)) + q * GEMM_THREADS;
            if (b >= NB) break;
            const int mb = b % (BM / 8), kb = b / (BM / 8);
            // row rr of the block holds m = 0..7 at k = rr; column c of the output is m = c
            uint32_t d[8][4];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                d[rr][0] = r.v[8 * q + rr].x; d[rr][1] = r.v[8 * q + rr].y;
                d[rr][2] = r.v[8 * q + rr].z; d[rr][3] = r.v[8 * q + rr].w;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint32_t o[4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const uint32_t x0 = d[2 * pp][c >> 1], x1 = d[2 * pp + 1][c >> 1];
                    o[pp] = (c & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
                }
                *(uint4*)(S + (8 * mb + c) * LROW + 8 * kb) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
};

// ------------------------------------------------------------------ kernel body
template <int BM, int BN, int NSPLIT, class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_bf16_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, uint16_t* lds) {
    constexpr int FM = BM / 64, FN = BN / 64;
    uint16_t* As = lds;
    uint16_t* Bs = lds + BM * LROW;                 // NSPLIT tiles of BN rows
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    typename LA::template Regs<BM> ra;
    typename LB::template Regs<BN> rb;
    la.template load<BM>(ra, t.m0, t.kbeg, tid);
    lb.template load<BN>(rb, t.n0, t.kbeg, tid);
    for (int64_t k0 = t.kbeg; k0 < t.kend; k0 += BK16) {
        __syncthreads();
        la.template store<BM>(As, ra, tid);
        lb.template store<BN>(Bs, rb, tid);
        __syncthreads();
        if (k0 + BK16 < t.kend) {
            la.template load<BM>(ra, t.m0, k0 + BK16, tid);
            lb.template load<BN>(rb, t.n0, k0 + BK16, tid);
        }
#pragma unroll
        for (int ks = 0; ks < BK16; ks += 16) {
            const int kof = ks + 8 * (lane >> 5);
            bf16x8 a[FM], b[FN][NSPLIT];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = *(const bf16x8*)(As + (wm * (BM / 2) + i * 32 + (lane & 31)) * LROW + kof);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int s = 0; s < NSPLIT; ++s)
                    b[j][s] = *(const bf16x8*)(Bs + s * BN * LROW + (wn * (BN / 2) + j * 32 + (lane & 31)) * LROW + kof);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int s = 0; s < NSPLIT; ++s)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j][s], acc[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = t.m0 + wm * (BM / 2) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t col = t.n0 + wn * (BN / 2) + j * 32 + (lane & 31);
                epi.element(t, row, col, acc[i][j][v]);
            }
}

template <int BM, int BN, int NSPLIT>
struct Bf16Lds {
    static constexpr int ELEMS = (BM + NSPLIT * BN) * LROW;
};

template <int BM, int BN, int NSPLIT, class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_bf16_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    __shared__ __attribute__((aligned(16))) uint16_t lds[Bf16Lds<BM, BN, NSPLIT>::ELEMS];
    Tile t;
    if (!map.get((int)blockIdx.x, BM, BN, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_bf16_tile<BM, BN, NSPLIT>(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

}  // namespace pwq
