// Large-tile bfloat16 MFMA contraction for gfx950 with direct global -> LDS loads
// (global_load_lds_dwordx4), float32 accumulate:
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k),   A, B row-major with k contiguous.
//
// 256 threads (4 wave64 in 2 x 2) own a 256 x 256 tile; a wave owns 128 x 128 as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, i.e. 8 operand fragments (16-byte LDS reads) per 16 MFMAs: half
// the LDS read traffic per MFMA of a 64 x 64 wave tile.  Operand tiles of 64 k are copied by
// the load unit straight into LDS (no staging registers, which leaves room for 256
// accumulators per lane): one wave instruction moves 8 rows x 128 bytes, lane i carrying
// row i / 8 and the 16-byte chunk that lands at position i % 8.  Rows are stored with the
// chunk c of row r at position c ^ (r & 7), the same swizzle the fragment reads undo.  Two
// LDS stages: the loads of tile t + 1 are in flight while tile t is multiplied.
//
// Operand requirements (checked by the host side): ld % 8 == 0, 16-byte aligned bases, and
// for every k at or past an operand's K inside a segment the OTHER operand is 0 there (a
// chunk start is clamped to K - 8, so reads stay inside the row; rows at or past M are
// clamped to M - 1, and their outputs are discarded by the epilogue).
#pragma once

#include "gemm_bf16.h"

namespace pwq {

constexpr int DL_TILE = 256;
constexpr int DL_STAGE = 2 * DL_TILE * BK16;             // bfloat16 elements per stage (A + B)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dl_load16(const uint16_t* g, uint16_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// Rows of bfloat16 over up to four k segments of kseg each (a multiple of BK16): logical k in
// [s kseg, (s+1) kseg) reads seg[s] at k - s kseg.  One segment: kseg is unused.
struct DlRows {
    const uint16_t* seg[4];
    int nseg;
    int64_t ld, M, K, kseg;
    // 256 rows x 64 k of logical k0 into LDS tile S (256 x 64, swizzled): wave w issues the
    // eight 8-row groups g = w + 4 q
    __device__ __forceinline__ void load(uint16_t* S, int64_t m0, int64_t k0, int wave, int lane) const {
        const uint16_t* base = seg[0];
        int64_t kk = k0;
        if (nseg > 1) {
            const int sg = (int)(k0 / kseg);
            base = seg[sg];
            kk = k0 - (int64_t)sg * kseg;
        }
        const int pc = lane & 7, rl = lane >> 3;           // position in the row, row in the group
        const int lc = pc ^ rl;                            // logical chunk landing at pc
        int64_t kc = kk + 8 * lc;
        if (kc > K - 8) kc = K - 8;                        // the other operand is 0 there
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r0 = 8 * (wave + 4 * q);
            int64_t row = m0 + r0 + rl;
            if (row > M - 1) row = M - 1;
            dl_load16(base + row * ld + kc, S + r0 * BK16);
        }
    }
};

// s_waitcnt with only the vector-memory count constrained: vmcnt <= N (N < 64)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: __syncthreads() would wait for every
// outstanding load, including the next tile's copies that are meant to stay in flight.
// The waits that matter are explicit (wait_vmcnt before, and LDS reads are consumed
// before the next barrier); the empty asm keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_dl_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, uint16_t* lds) {
    constexpr int FM = 4, FN = 4;
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

    const int64_t nk = (t.kend - t.kbeg) / BK16;         // host guarantees whole tiles
    la.load(lds, t.m0, t.kbeg, wave, lane);
    lb.load(lds + DL_TILE * BK16, t.n0, t.kbeg, wave, lane);
    if (nk > 1) {
        la.load(lds + DL_STAGE, t.m0, t.kbeg + BK16, wave, lane);
        lb.load(lds + DL_STAGE + DL_TILE * BK16, t.n0, t.kbeg + BK16, wave, lane);
    }

    const int arow = wm * 128 + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    const int half = lane >> 5;
    for (int64_t it = 0; it < nk; ++it) {
        // this wave's loads of tile it have landed (those of it + 1 may still fly), and after
        // the barrier every wave's have
        if (it + 1 < nk) wait_vmcnt<16>();
        else wait_vmcnt<0>();
        barrier_nofence();
        const uint16_t* As = lds + (it & 1) * DL_STAGE;
        const uint16_t* Bs = As + DL_TILE * BK16;
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
        // every wave is done with this stage before it is refilled with tile it + 2 (its
        // fragment reads were consumed by the MFMAs above)
        __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0) only
        barrier_nofence();
        if (it + 2 < nk) {
            uint16_t* Sn = lds + (it & 1) * DL_STAGE;
            la.load(Sn, t.m0, t.kbeg + (it + 2) * BK16, wave, lane);
            lb.load(Sn + DL_TILE * BK16, t.n0, t.kbeg + (it + 2) * BK16, wave, lane);
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t r0 = t.m0 + wm * 128 + i * 32 + 4 * (lane >> 5);
            const int64_t col = t.n0 + wn * 128 + j * 32 + (lane & 31);
            epi_block16(epi, t, acc[i][j], [&](int v) { return r0 + 8 * (v >> 2) + (v & 3); }, col);
        }
}

template <class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_dl_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * DL_STAGE];
    Tile t;
    if (!map.get((int)blockIdx.x, DL_TILE, DL_TILE, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_dl_tile(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

}  // namespace pwq
