// Large-tile bfloat16 MFMA contraction for gfx950 with direct global -> LDS loads
// (global_load_lds_dwordx4), float32 accumulate:
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k),   A, B row-major with k contiguous.
//
// 256 threads (4 wave64 in 2 x 2) own a 256 x 256 tile; a wave owns 128 x 128 as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, i.e. 8 operand fragments (16-byte LDS reads) per 16 MFMAs: half
// the LDS read traffic per MFMA of a 64 x 64 wave tile.  Operand tiles of 32 k are copied by
// the load unit straight into LDS (no staging registers, which leaves room for 256
// accumulators per lane): one wave instruction moves 16 rows x 64 bytes, lane i carrying
// row i / 4 and the 16-byte chunk that lands at position i % 4.  Row r keeps its chunk c at
// position c ^ ((r / 4) % 4), the swizzle the fragment reads undo (8 or 16 consecutive rows
// of one chunk then hit distinct banks).
//
// Four LDS stages (128 KiB), one barrier per k-tile, placed after the first half of the
// tile's MFMAs: past it, every wave has its share of the next tile in LDS and is done with
// the tile before this one, whose stage then takes the loads three tiles ahead; the next
// tile's first fragments are read while the second half's MFMAs issue.  So neither the
// barrier nor the first LDS reads of a tile stand between two tiles' MFMAs.
//
// Operand requirements (checked by the host side): ld % 8 == 0, 16-byte aligned bases, k
// ranges in whole tiles of 32, and for every k at or past an operand's K inside a segment
// the OTHER operand is 0 there (a chunk start is clamped to K - 8, so reads stay inside the
// row; rows at or past M are clamped to M - 1, and their outputs are discarded by the
// epilogue).
#pragma once

#include "gemm_bf16.h"

namespace pwq {

constexpr int DL_TILE = 256;
constexpr int DL_BK = 32;                                // k per stage
constexpr int DL_NS = 4;                                 // stages
constexpr int DL_STAGE = 2 * DL_TILE * DL_BK;            // bfloat16 elements per stage (A + B)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dl_load16(const uint16_t* g, uint16_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// element offset of row r's logical 16-byte chunk c in a 256 x 32 stage tile
__device__ __forceinline__ int dl_off(int r, int c) { return r * DL_BK + 8 * (c ^ ((r >> 2) & 3)); }

// The segment holding logical k (updated to the offset inside it).  Static indices and
// compares only: a dynamic index into the kernel-argument array would load it from memory
// on every tile, and the wait for that scalar load also waits for the LDS reads in flight.
__device__ __forceinline__ const uint16_t* dl_segment(const uint16_t* const (&seg)[4], int nseg, int64_t kseg,
                                                      int64_t& k) {
    if (nseg == 1) return seg[0];
    const int sg = (int)(k >= kseg) + (int)(k >= 2 * kseg) + (int)(k >= 3 * kseg);
    k -= (int64_t)sg * kseg;
    return sg == 0 ? seg[0] : (sg == 1 ? seg[1] : (sg == 2 ? seg[2] : seg[3]));
}

// Rows of bfloat16 over up to four k segments of kseg each (a multiple of 64): logical k in
// [s kseg, (s+1) kseg) reads seg[s] at k - s kseg.  One segment: kseg is unused.
struct DlRows {
    const uint16_t* seg[4];
    int nseg;
    int64_t ld, M, K, kseg;
    // 256 rows x 32 k of logical k0 into the stage tile S (256 x 32, swizzled): wave w issues
    // the four 16-row groups g = w + 4 q
    __device__ __forceinline__ void load(uint16_t* S, int64_t m0, int64_t k0, int wave, int lane) const {
        int64_t kk = k0;
        const uint16_t* base = dl_segment(seg, nseg, kseg, kk);
        const int pc = lane & 3, rl = lane >> 2;           // position in the row, row in the group
        const int lc = pc ^ ((rl >> 2) & 3);               // logical chunk landing at pc
        int64_t kc = kk + 8 * lc;
        if (kc > K - 8) kc = K - 8;                        // the other operand is 0 there
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r0 = 16 * (wave + 4 * q);
            int64_t row = m0 + r0 + rl;
            if (row > M - 1) row = M - 1;
            dl_load16(base + row * ld + kc, S + r0 * DL_BK);
        }
    }
};

// one 256 x 32 tile-major block (16 KiB in one piece) into the stage tile S, swizzled: wave
// w issues the four 16-row groups g = w + 4 q, lane i carrying row i / 4 and the chunk that
// lands at position i % 4
__device__ __forceinline__ void dl_load_block(const uint16_t* blk, uint16_t* S, int wave, int lane) {
    const int pc = lane & 3, rl = lane >> 2;
    const int lc = pc ^ ((rl >> 2) & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r0 = 16 * (wave + 4 * q);
        dl_load16(blk + (r0 + rl) * DL_BK + 8 * lc, S + r0 * DL_BK);
    }
}

// Rows stored tile-major: the k-tile kt (32 k) of the 256-row panel P is one contiguous
// 256 x 32 block, element (r, k) of a segment at ((r / 256) kpan + k / 32) 8192 +
// (r % 256) 32 + k % 32, kpan = kseg / 32.  A tile's load then reads 16 KiB in one piece
// (each instruction 1 KiB), instead of 256 rows a whole row length apart.  Rows are padded
// to whole panels and k to whole segments (the writer zeroes both), so nothing is clamped.
// Up to four k segments as in DlRows; tile row offsets m0 are multiples of 256.
struct DlTiled {
    const uint16_t* seg[4];
    int nseg;
    int64_t kseg;
    __device__ __forceinline__ void load(uint16_t* S, int64_t m0, int64_t k0, int wave, int lane) const {
        int64_t kk = k0;
        const uint16_t* base = dl_segment(seg, nseg, kseg, kk);
        dl_load_block(base + ((m0 >> 8) * (kseg >> 5) + (kk >> 5)) * (int64_t)(DL_TILE * DL_BK), S, wave, lane);
    }
};

// Rows of a lower-triangular operand stored as whole tile-major panels of growing length:
// panel p (rows 256 p .. 256 p + 255) holds its k-tiles 0 .. KT (p + 1) - 1 of 32 k each,
// panel after panel (panel p starts at k-tile KT p (p + 1) / 2).  Tiles of panel p only read
// k below 32 KT (p + 1).
struct DlTri {
    const uint16_t* p;
    int kt;                                             // KT: k-tiles per 256 columns of the band
    __device__ __forceinline__ void load(uint16_t* S, int64_t m0, int64_t k0, int wave, int lane) const {
        const int64_t pan = m0 >> 8;
        dl_load_block(p + ((int64_t)kt * (pan * (pan + 1) / 2) + (k0 >> 5)) * (int64_t)(DL_TILE * DL_BK), S, wave, lane);
    }
};
// element (r, k) of one segment in the tile-major layout
__host__ __device__ __forceinline__ int64_t dl_tiled_index(int64_t r, int64_t k, int64_t kseg) {
    return ((r >> 8) * (kseg >> 5) + (k >> 5)) * (int64_t)(DL_TILE * DL_BK) + (r & 255) * DL_BK + (k & 31);
}

// s_waitcnt with only the vector-memory count constrained: vmcnt <= N (N < 64)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: __syncthreads() would wait for every
// outstanding load, including the copies of later tiles that are meant to stay in flight.
// The waits that matter are explicit (wait_vmcnt before; a stage's fragment reads are
// consumed by MFMAs before the barrier that frees it); the empty asm keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Issue order of one half tile: MFMA, fragment read, eight times, then the last eight MFMAs.
// With one wave per SIMD the order is what overlaps the reads with the matrix pipe; the
// first MFMA of a half only waits for reads issued during the half before.
__device__ __forceinline__ void dl_interleave() {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
}

template <class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_dl_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, uint16_t* lds) {
    constexpr int FM = 4, FN = 4;
    constexpr int AB = DL_TILE * DL_BK;                  // B's offset inside a stage
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

    const int64_t nk = (t.kend - t.kbeg) / DL_BK;        // host guarantees whole tiles
    // tiles 0 .. 2 into stages 0 .. 2 (eight load instructions per wave and tile)
#pragma unroll
    for (int st = 0; st < DL_NS - 1; ++st)
        if (st < nk) {
            la.load(lds + st * DL_STAGE, t.m0, t.kbeg + st * DL_BK, wave, lane);
            lb.load(lds + st * DL_STAGE + AB, t.n0, t.kbeg + st * DL_BK, wave, lane);
        }
    const int arow = wm * 128 + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    const int half = lane >> 5;
    if (nk > 2) wait_vmcnt<16>();
    else if (nk == 2) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    barrier_nofence();
    bf16x8 a0[FM], b0[FN], a1[FM], b1[FN];               // k halves 0..15 and 16..31 of a tile
#pragma unroll
    for (int i = 0; i < FM; ++i) a0[i] = *(const bf16x8*)(lds + dl_off(arow + 32 * i, half));
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = *(const bf16x8*)(lds + AB + dl_off(brow + 32 * j, half));

    for (int64_t it = 0; it < nk; ++it) {
        const uint16_t* As = lds + (it & 3) * DL_STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) a1[i] = *(const bf16x8*)(As + dl_off(arow + 32 * i, 2 + half));
#pragma unroll
        for (int j = 0; j < FN; ++j) b1[j] = *(const bf16x8*)(As + AB + dl_off(brow + 32 * j, 2 + half));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
        dl_interleave();
        if (it + 1 < nk) {
            // this wave's share of tile it + 1 has landed (tile it + 2 may still fly); past the
            // barrier every wave's has, and every wave is done with tile it - 1
            if (it + 2 < nk) wait_vmcnt<8>();
            else wait_vmcnt<0>();
            barrier_nofence();
            if (it + 3 < nk) {
                uint16_t* Sn = lds + ((it + 3) & 3) * DL_STAGE;
                la.load(Sn, t.m0, t.kbeg + (it + 3) * DL_BK, wave, lane);
                lb.load(Sn + AB, t.n0, t.kbeg + (it + 3) * DL_BK, wave, lane);
            }
        }
        // the next tile's first fragments (after the last tile they read a stage no copy
        // targets any more, and go unused), issued between this half's MFMAs
        const uint16_t* An = lds + ((it + 1) & 3) * DL_STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) a0[i] = *(const bf16x8*)(An + dl_off(arow + 32 * i, half));
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = *(const bf16x8*)(An + AB + dl_off(brow + 32 * j, half));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
        dl_interleave();
        // keep those reads in this iteration (not sunk into the next one's first MFMAs), and
        // their wait after this half's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(a0[i]));
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(b0[j]));
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
    __shared__ __attribute__((aligned(16))) uint16_t lds[DL_NS * DL_STAGE];
    Tile t;
    if (!map.get((int)blockIdx.x, DL_TILE, DL_TILE, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_dl_tile(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

}  // namespace pwq
