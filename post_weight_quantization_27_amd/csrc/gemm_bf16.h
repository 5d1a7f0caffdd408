// Tiled bfloat16 MFMA contraction engine for gfx950 (v_mfma_f32_32x32x16_bf16), float32
// accumulate:
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k)
//
// 256 threads (4 wave64 in 2 x 2) own a BM x BN tile (BM, BN in {128, 256}); a wave owns
// (BM/2) x (BN/2) as 32 x 32 MFMA blocks, so at 256 x 256 each wave holds 16 accumulator
// blocks and reads 8 operand fragments per 16 MFMAs (LDS traffic half of what 64 x 64 per
// wave needs).  Operand tiles of BK = 64 are staged in LDS as [row][k] with k contiguous,
// 128 bytes per row, the 16-byte chunk c of row r stored at chunk c ^ (r & 7): the
// fragment reads (8 consecutive rows at one chunk per group of 8 lanes) and the row stores
// hit 8 distinct 16-byte bank groups.  LDS is double buffered: while the MFMAs read one
// buffer the registers fetched during the previous k-tile are stored into the other, and
// the next global loads are issued, with one barrier per k-tile.
#pragma once

#include "gemm_f32.h"

namespace pwq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BK16 = 64;             // k per LDS tile

__device__ __forceinline__ int lds_off(int row, int chunk) { return row * BK16 + ((chunk ^ (row & 7)) << 3); }

// 16-byte load at a workgroup-uniform base plus a 32-bit per-lane byte offset, so the
// address is an SGPR pair plus one VGPR instead of a 64-bit VGPR pair per load
__device__ __forceinline__ uint4 ld16(const uint16_t* ubase, uint32_t byte_off) {
    return *(const uint4*)((const char*)ubase + byte_off);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------ loaders
// Element (m, k) at p[m * ld + k], bfloat16, k contiguous.  With p2 set, the logical k range
// is two segments of kseg (a multiple of BK16): k in [kseg, 2 kseg) reads p2 at k - kseg.
// Columns at or past K inside a segment, and rows at or past M, read as 0.
struct Bf16Rows {
    const uint16_t* p;
    const uint16_t* p2;
    int64_t ld, M, K, kseg;
    int vec;                         // ld % 8 == 0 and p, p2 16-byte aligned
    template <int ROWS>
    struct Regs { uint4 v[ROWS * 8 / GEMM_THREADS]; };
    // thread t moves chunk t & 7 of rows t >> 3 + 32 i
    template <int ROWS>
    __device__ __forceinline__ void load(Regs<ROWS>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = ROWS * 8 / GEMM_THREADS;
        const uint16_t* base = p;
        int64_t kk = k0;
        if (p2 && k0 >= kseg) { base = p2; kk = k0 - kseg; }
        const int rl = tid >> 3, c = tid & 7;
        const uint32_t loff = (uint32_t)(((int64_t)rl * ld + 8 * c) * 2);
        const bool full = vec && (m0 + ROWS <= M) && (kk + BK16 <= K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint16_t* ub = base + (m0 + 32 * i) * ld + kk;
            if (full) {
                r.v[i] = ld16(ub, loff);
            } else {
                const bool rok = m0 + 32 * i + rl < M;
                const uint16_t* e = (const uint16_t*)((const char*)ub + loff);
                const int64_t kc = kk + 8 * c;
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = (rok && kc + 2 * q < K) ? e[2 * q] : 0u;
                    const uint32_t hi = (rok && kc + 2 * q + 1 < K) ? e[2 * q + 1] : 0u;
                    w[q] = lo | (hi << 16);
                }
                r.v[i] = make_uint4(w[0], w[1], w[2], w[3]);
            }
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

// Element (m, k) at p[k * ld + m], bfloat16, m contiguous.  A thread moves 8 x 8 blocks
// (8 consecutive k of 8 consecutive m) and transposes them in registers into [m][k].  Block
// b of the tile is (m block b >> 3, k block b & 7), so the 8 lanes of a store group write
// 8 different chunks of one LDS row group.  toff spreads two operands with fewer blocks
// than threads over all threads.
struct Bf16Cols {
    const uint16_t* p;
    int64_t ld, M, K;
    int vec;
    int toff;
    template <int ROWS>
    struct Regs { uint4 v[8 * ((ROWS + GEMM_THREADS - 1) / GEMM_THREADS)]; };
    template <int ROWS>
    __device__ __forceinline__ void load(Regs<ROWS>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int PER = (ROWS + GEMM_THREADS - 1) / GEMM_THREADS;
        const bool full = vec && (m0 + ROWS <= M) && (k0 + BK16 <= K);
        const int bl = (tid + toff) & (GEMM_THREADS - 1);
        const int kl = 8 * (bl & 7), ml = 8 * (bl >> 3);
        const uint32_t loff = (uint32_t)(((int64_t)kl * ld + ml) * 2);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (bl + q * GEMM_THREADS >= ROWS) break;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const uint16_t* ub = p + (k0 + rr) * ld + m0 + q * GEMM_THREADS;
                if (full) {
                    r.v[8 * q + rr] = ld16(ub, loff);
                } else {
                    const int64_t k = k0 + kl + rr, m = m0 + q * GEMM_THREADS + ml;
                    const uint16_t* e = (const uint16_t*)((const char*)ub + loff);
                    uint32_t w[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t lo = (k < K && m + 2 * c < M) ? e[2 * c] : 0u;
                        const uint32_t hi = (k < K && m + 2 * c + 1 < M) ? e[2 * c + 1] : 0u;
                        w[c] = lo | (hi << 16);
                    }
                    r.v[8 * q + rr] = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    }
    template <int ROWS>
    __device__ __forceinline__ void store(uint16_t* S, const Regs<ROWS>& r, int tid) const {
        constexpr int PER = (ROWS + GEMM_THREADS - 1) / GEMM_THREADS;
        const int bl = (tid + toff) & (GEMM_THREADS - 1);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int b = bl + q * GEMM_THREADS;
            if (b >= ROWS) break;
            const int mb = b >> 3, kc = b & 7;
            // register rr holds k = 8 kc + rr for m = 8 mb .. 8 mb + 7; LDS row 8 mb + c wants
            // that row's 8 k values, i.e. half-word c of every register
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
                *(uint4*)(S + lds_off(8 * mb + c, kc)) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
};

// ------------------------------------------------------------------ kernel body
template <int BM, int BN>
struct Bf16Lds {
    static constexpr int STAGE = (BM + BN) * BK16;   // bfloat16 elements per buffer
    static constexpr int ELEMS = 2 * STAGE;
};

// Host side guarantees: kbeg and every chunk boundary are multiples of BK16.
template <int BM, int BN, class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_bf16_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, uint16_t* lds) {
    constexpr int FM = BM / 64, FN = BN / 64;
    constexpr int STAGE = Bf16Lds<BM, BN>::STAGE;
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
    la.template store<BM>(lds, ra, tid);
    lb.template store<BN>(lds + BM * BK16, rb, tid);
    if (t.kbeg + BK16 < t.kend) {
        la.template load<BM>(ra, t.m0, t.kbeg + BK16, tid);
        lb.template load<BN>(rb, t.n0, t.kbeg + BK16, tid);
    }
    __syncthreads();

    const int arow = wm * (BM / 2) + (lane & 31);
    const int brow = wn * (BN / 2) + (lane & 31);
    const int half = lane >> 5;
    int buf = 0;
    for (int64_t k0 = t.kbeg; k0 < t.kend; k0 += BK16) {
        const uint16_t* As = lds + buf * STAGE;
        const uint16_t* Bs = As + BM * BK16;
        // fragments are read one k-step ahead of the MFMAs that use them
        bf16x8 a[2][FM], b[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) a[0][i] = *(const bf16x8*)(As + lds_off(arow + 32 * i, half));
#pragma unroll
        for (int j = 0; j < FN; ++j) b[0][j] = *(const bf16x8*)(Bs + lds_off(brow + 32 * j, half));
#pragma unroll
        for (int ks = 0; ks < BK16 / 16; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK16 / 16) {
                const int chunk = 2 * (ks + 1) + half;
#pragma unroll
                for (int i = 0; i < FM; ++i) a[cur ^ 1][i] = *(const bf16x8*)(As + lds_off(arow + 32 * i, chunk));
#pragma unroll
                for (int j = 0; j < FN; ++j) b[cur ^ 1][j] = *(const bf16x8*)(Bs + lds_off(brow + 32 * j, chunk));
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][i], b[cur][j], acc[i][j], 0, 0, 0);
        }
        if (k0 + BK16 < t.kend) {
            // the other buffer was last read before the previous barrier
            uint16_t* An = lds + (buf ^ 1) * STAGE;
            la.template store<BM>(An, ra, tid);
            lb.template store<BN>(An + BM * BK16, rb, tid);
            if (k0 + 2 * BK16 < t.kend) {
                la.template load<BM>(ra, t.m0, k0 + 2 * BK16, tid);
                lb.template load<BN>(rb, t.n0, k0 + 2 * BK16, tid);
            }
        }
        __syncthreads();
        buf ^= 1;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t r0 = t.m0 + wm * (BM / 2) + i * 32 + 4 * (lane >> 5);
            const int64_t col = t.n0 + wn * (BN / 2) + j * 32 + (lane & 31);
            epi_block16(epi, t, acc[i][j], [&](int v) { return r0 + 8 * (v >> 2) + (v & 3); }, col);
        }
}

template <int BM, int BN, class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_bf16_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    __shared__ __attribute__((aligned(16))) uint16_t lds[Bf16Lds<BM, BN>::ELEMS];
    Tile t;
    if (!map.get((int)blockIdx.x, BM, BN, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_bf16_tile<BM, BN>(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

}  // namespace pwq
