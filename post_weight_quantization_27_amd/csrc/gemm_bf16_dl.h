// Large-tile bfloat16 MFMA contraction for gfx950, float32 accumulate:
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k),   A, B row-major with k contiguous.
//
// 256 threads (4 wave64 in 2 x 2) own a 256 x 256 tile; a wave owns 128 x 128 as 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, i.e. 8 operand fragments (16-byte LDS reads) per 16 MFMAs: half
// the LDS read traffic per MFMA of a 64 x 64 wave tile.  An operand tile of 32 k sits in LDS
// as 256 rows of 64 bytes; row r keeps its 16-byte chunk c at position c ^ ((r / 4) % 4), the
// swizzle the fragment reads undo (8 or 16 consecutive rows of one chunk then hit distinct
// banks).  One barrier per k-tile, placed after the first half of the tile's MFMAs, so
// neither the barrier nor the first LDS reads of a tile stand between two tiles' MFMAs.
//
// Two copy paths into that layout:
// * gemm_dl_kernel (rows of any length, DlRows): the load unit copies straight into LDS
//   (global_load_lds_dwordx4, no staging registers): one wave instruction moves 16 rows x
//   64 bytes, lane i carrying row i / 4 and the chunk that lands at position i % 4.  Four
//   LDS stages (128 KiB); past the barrier of tile it, tile it - 1's stage takes the loads
//   three tiles ahead.
// * gemm_rs_kernel (tile-major operands, at the end of this file): loads into VGPRs, then
//   ds_write_b128.  Faster on the Hessian's and the trace product's long k ranges.
//
// Operand requirements of DlRows (checked by the host side): ld % 8 == 0, 16-byte aligned
// bases, k ranges in whole tiles of 32, and for every k at or past an operand's K inside a
// segment the OTHER operand is 0 there (a chunk start is clamped to K - 8, so reads stay
// inside the row; rows at or past M are clamped to M - 1, and their outputs are discarded by
// the epilogue).
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

// Tile-major rows (the operands of the register-staged engine at the end of this file):
// the k-tile kt (32 k) of the 256-row panel P is one contiguous 256 x 32 block, element
// (r, k) of a segment at ((r / 256) kpan + k / 32) 8192 + (r % 256) 32 + k % 32,
// kpan = kseg / 32.  A tile's load then reads 16 KiB in one piece (each instruction 1 KiB),
// instead of 256 rows a whole row length apart.  Rows are padded to whole panels and k to
// whole segments (the writer zeroes both), so nothing is clamped; tile row offsets m0 are
// multiples of 256.

// One k segment
struct DlTiled1 {
    const uint16_t* p;
    int64_t kseg;
    // the 256 x 32 block of rows m0.. and k0..
    __device__ __forceinline__ const uint16_t* block(int64_t m0, int64_t k0) const {
        return p + ((m0 >> 8) * (kseg >> 5) + (k0 >> 5)) * (int64_t)(DL_TILE * DL_BK);
    }
};

// Four k segments of kseg each (logical k in [s kseg, (s+1) kseg) reads seg[s]); the
// segment is picked by selects, so the loop stays one basic block
struct DlTiled4 {
    const uint16_t* seg[4];
    int64_t kseg;
    __device__ __forceinline__ const uint16_t* block(int64_t m0, int64_t k0) const {
        const int sg = (int)(k0 >= kseg) + (int)(k0 >= 2 * kseg) + (int)(k0 >= 3 * kseg);
        const uint16_t* p = sg == 0 ? seg[0] : seg[1];
        p = sg == 2 ? seg[2] : p;
        p = sg == 3 ? seg[3] : p;
        return p + ((m0 >> 8) * (kseg >> 5) + ((k0 - sg * kseg) >> 5)) * (int64_t)(DL_TILE * DL_BK);
    }
};

// Six k segments of kseg each, picked like DlTiled4's.  A float32 product runs on it as the
// six larger terms of its three-piece bfloat16 split (split3_tiled_block below): segment s
// holds the pieces (i, j) of a_i b_j in the order (3,1), (1,3), (2,2), (2,1), (1,2), (1,1),
// the small terms first so they build up before the large ones join the sum.
struct DlTiled6 {
    const uint16_t* seg[6];
    int64_t kseg;
    __device__ __forceinline__ const uint16_t* block(int64_t m0, int64_t k0) const {
        const int sg = (int)(k0 >= kseg) + (int)(k0 >= 2 * kseg) + (int)(k0 >= 3 * kseg) + (int)(k0 >= 4 * kseg) +
                       (int)(k0 >= 5 * kseg);
        const uint16_t* p = sg == 0 ? seg[0] : seg[1];
        p = sg == 2 ? seg[2] : p;
        p = sg == 3 ? seg[3] : p;
        p = sg == 4 ? seg[4] : p;
        p = sg == 5 ? seg[5] : p;
        return p + ((m0 >> 8) * (kseg >> 5) + ((k0 - sg * kseg) >> 5)) * (int64_t)(DL_TILE * DL_BK);
    }
};

// Rows of a lower-triangular operand stored as whole tile-major panels of growing length:
// panel p (rows 256 p .. 256 p + 255) holds its k-tiles 0 .. KT (p + 1) - 1 of 32 k each,
// panel after panel (panel p starts at k-tile KT p (p + 1) / 2).  Tiles of panel p only read
// k below 32 KT (p + 1).
struct DlTri {
    const uint16_t* p;
    int kt;                                             // KT: k-tiles per 256 columns of the band
    __device__ __forceinline__ const uint16_t* block(int64_t m0, int64_t k0) const {
        const int64_t pan = m0 >> 8;
        return p + ((int64_t)kt * (pan * (pan + 1) / 2) + (k0 >> 5)) * (int64_t)(DL_TILE * DL_BK);
    }
};
// rows of a tile-major operand: whole 256-row panels
__host__ __device__ __forceinline__ int64_t dl_panel_pad(int64_t m) { return (m + DL_TILE - 1) / DL_TILE * DL_TILE; }

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

// Issue order of one half tile (16 MFMAs): NV times one MFMA and one global copy, eight
// times one MFMA and one fragment read, then the rest.  With one wave per SIMD the order is
// what overlaps the copies and reads with the matrix pipe; the first MFMA of a half only
// waits for reads issued during the half before.
template <int NV>
__device__ __forceinline__ void dl_interleave() {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (NV < 8) __builtin_amdgcn_sched_group_barrier(0x008, 8 - NV, 0);
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
        dl_interleave<0>();
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
        dl_interleave<0>();
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

// ---------------------------------------------------------------------------------------------
// Register-staged variant for tile-major operands: the same LDS layout and MFMA schedule,
// but each 16 KiB block travels global -> VGPR (four 16-byte loads per lane, every wave
// instruction 1 KiB in one piece) -> LDS (ds_write_b128 to the swizzled position).  Three
// LDS stages and NR register sets: tile j's loads go out NR tiles before its LDS write (set
// j % NR), its LDS write two tiles before its MFMAs.  One barrier per tile, between the
// halves: before it every wave has finished its reads of tile it - 1 and its writes of
// tile it + 1; past it, tile it + 2 goes into tile it - 1's stage.  Every step issues the
// same loads and writes: past the last tile they repeat it, into stages nothing reads any
// more, so the loop has no branch and the compiler can count the loads in flight.  k ranges
// are whole multiples of NR tiles (the host pads them).
constexpr int RS_NS = 3;

typedef unsigned int rs_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const rs_u32x4* rs_gptr_t;

__device__ __forceinline__ void rs_fetch(const uint16_t* blk, rs_u32x4* r, int tid) {
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = *(rs_gptr_t)(blk + (q * 256 + tid) * 8);
}

// chunk q 256 + tid of the block is row q 64 + tid / 4, logical chunk tid % 4
__device__ __forceinline__ void rs_store(uint16_t* S, const rs_u32x4* r, int tid) {
    uint16_t* d = S + dl_off(tid >> 2, tid & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q) *(rs_u32x4*)(d + q * 64 * DL_BK) = r[q];
}

// s_waitcnt with only the LDS / scalar-memory count constrained: lgkmcnt == 0
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int NR, class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_rs_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, uint16_t* lds) {
    constexpr int FM = 4, FN = 4;
    constexpr int AB = DL_TILE * DL_BK;
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

    const int64_t nk = (t.kend - t.kbeg) / DL_BK;
    auto kof = [&](int64_t kt) { return t.kbeg + (kt < nk ? kt : nk - 1) * DL_BK; };
    rs_u32x4 ra[NR][4], rb[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        rs_fetch(la.block(t.m0, kof(r)), ra[r], tid);
        rs_fetch(lb.block(t.n0, kof(r)), rb[r], tid);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        rs_store(lds + r * DL_STAGE, ra[r], tid);
        rs_store(lds + r * DL_STAGE + AB, rb[r], tid);
        rs_fetch(la.block(t.m0, kof(NR + r)), ra[r], tid);
        rs_fetch(lb.block(t.n0, kof(NR + r)), rb[r], tid);
    }
    wait_lgkm0();
    barrier_nofence();

    const int arow = wm * 128 + (lane & 31);
    const int brow = wn * 128 + (lane & 31);
    const int half = lane >> 5;
    bf16x8 a0[FM], b0[FN], a1[FM], b1[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a0[i] = *(const bf16x8*)(lds + dl_off(arow + 32 * i, half));
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = *(const bf16x8*)(lds + AB + dl_off(brow + 32 * j, half));

    int sc = 0, sn = 1, sw = 2;                          // stages of tiles it, it + 1, it + 2
    for (int64_t it0 = 0; it0 < nk; it0 += NR) {
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            const int64_t it = it0 + u;
            const int r = (u + 2) % NR;                  // register set of tile it + 2
            const uint16_t* As = lds + sc * DL_STAGE;
#pragma unroll
            for (int i = 0; i < FM; ++i) a1[i] = *(const bf16x8*)(As + dl_off(arow + 32 * i, 2 + half));
#pragma unroll
            for (int j = 0; j < FN; ++j) b1[j] = *(const bf16x8*)(As + AB + dl_off(brow + 32 * j, 2 + half));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
            dl_interleave<0>();
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkm0();
            barrier_nofence();
            uint16_t* Sw = lds + sw * DL_STAGE;
            rs_store(Sw, ra[r], tid);
            rs_store(Sw + AB, rb[r], tid);
            rs_fetch(la.block(t.m0, kof(it + 2 + NR)), ra[r], tid);
            rs_fetch(lb.block(t.n0, kof(it + 2 + NR)), rb[r], tid);
            const uint16_t* An = lds + sn * DL_STAGE;
#pragma unroll
            for (int i = 0; i < FM; ++i) a0[i] = *(const bf16x8*)(An + dl_off(arow + 32 * i, half));
#pragma unroll
            for (int j = 0; j < FN; ++j) b0[j] = *(const bf16x8*)(An + AB + dl_off(brow + 32 * j, half));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int s0 = sc;
            sc = sn;
            sn = sw;
            sw = s0;
        }
    }
    wait_vmcnt<0>();
    if constexpr (EpiIsFast<EPI>::value) {
        // whole-tile read-modify-write through buffer addressing (the float32 engines' epilogue)
        const int wu = __builtin_amdgcn_readfirstlane(wave);
        epi_rmw_wave<FM, FN>(epi, t, acc, t.m0 + (wu & 1) * 128, t.n0 + (wu >> 1) * 128, lane,
                             epi_whole(epi, t, DL_TILE, DL_TILE));
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t r0 = t.m0 + wm * 128 + i * 32 + 4 * (lane >> 5);
                const int64_t col = t.n0 + wn * 128 + j * 32 + (lane & 31);
                epi_block16(epi, t, acc[i][j], [&](int v) { return r0 + 8 * (v >> 2) + (v & 3); }, col);
            }
    }
}

// One tile task of the register-staged engine, for launches that run two of them
template <int NR, class LA_, class LB_, class MAP_, class EPI_>
struct RsTask {
    LA_ la;
    LB_ lb;
    MAP_ map;
    EPI_ epi;
    __device__ __forceinline__ void run(int bid, uint16_t* lds) {
        Tile t;
        if (!map.get(bid, DL_TILE, DL_TILE, t)) {
            epi.finish(t, threadIdx.x, false);
            return;
        }
        gemm_rs_tile<NR>(la, lb, t, epi, lds);
        epi.finish(t, threadIdx.x, true);
    }
};

// Workgroups [0, n1) run task a, the rest task b; nothing runs while *guard != 0
template <class TA, class TB>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_rs_dual_kernel(TA a, TB b, int n1, const int32_t* guard) {
    if (guard && *guard != 0) return;
    __shared__ __attribute__((aligned(16))) uint16_t lds[RS_NS * DL_STAGE];
    if ((int)blockIdx.x < n1) a.run((int)blockIdx.x, lds);
    else b.run((int)blockIdx.x - n1, lds);
}

// The three bfloat16 pieces of a float32 value: a = p0 + p1 + p2 exactly.  p0 = bf16(a);
// a - p0 is exact in float32 and holds at most 16 significant bits, p1 = bf16(a - p0); the
// rest, at most 8 significant bits, is p2 exactly (bfloat16 shares float32's exponent range,
// and its subnormals hold such a rest whenever |a| >= 2^-110).
__device__ __forceinline__ void split3(float a, uint16_t (&p)[3]) {
    p[0] = f32_to_bf16_bits(a);
    const float r1 = a - bf16_bits_to_f32(p[0]);
    p[1] = f32_to_bf16_bits(r1);
    p[2] = f32_to_bf16_bits(r1 - bf16_bits_to_f32(p[1]));
}

// The pieces of a float32 operand (m, k), m < M, k < K, tile-major for DlTiled6: piece p of
// element (m, k) at out + p pstride + dl_tiled_index(m, k, kseg); zero for m >= M (up to the
// whole 256-row panel) or k >= K (up to kseg, a multiple of 64).  Source element (m, k) at
// src[k ld + m] (KMAJ) or src[m ld + k].  One 64 x 64 block per workgroup through LDS, read
// along the source's contiguous index and written 16 bytes (8 k) at a time: the body of a
// 256-thread kernel with grid (panel-padded M / 64, kseg / 64); each file that launches it
// wraps it in a kernel of its own name.
template <bool KMAJ>
__device__ __forceinline__ void split3_tiled_block(const float* __restrict__ src, int64_t ld, int64_t M, int64_t K,
                                                   uint16_t* __restrict__ out, int64_t kseg, int64_t pstride) {
    __shared__ float tl[64][65];
    const int64_t m0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll 4
    for (int q = ty; q < 64; q += 4) {
        if (KMAJ) {
            const int64_t k = k0 + q, m = m0 + tx;
            tl[tx][q] = (k < K && m < M) ? src[k * ld + m] : 0.f;
        } else {
            const int64_t m = m0 + q, k = k0 + tx;
            tl[q][tx] = (m < M && k < K) ? src[m * ld + k] : 0.f;
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = (int)threadIdx.x + 256 * h;
        const int r = idx >> 3, kc = (idx & 7) * 8;      // row r, k kc .. kc + 7 of the block
        uint32_t w[3][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint16_t lo[3], hi[3];
            split3(tl[r][kc + 2 * j], lo);
            split3(tl[r][kc + 2 * j + 1], hi);
#pragma unroll
            for (int p = 0; p < 3; ++p) w[p][j] = (uint32_t)lo[p] | ((uint32_t)hi[p] << 16);
        }
        const int64_t o = dl_tiled_index(m0 + r, k0 + kc, kseg);
#pragma unroll
        for (int p = 0; p < 3; ++p) *(uint4*)(out + p * pstride + o) = make_uint4(w[p][0], w[p][1], w[p][2], w[p][3]);
    }
}

template <int NR, class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_rs_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    __shared__ __attribute__((aligned(16))) uint16_t lds[RS_NS * DL_STAGE];
    Tile t;
    if (!map.get((int)blockIdx.x, DL_TILE, DL_TILE, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_rs_tile<NR>(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

}  // namespace pwq
