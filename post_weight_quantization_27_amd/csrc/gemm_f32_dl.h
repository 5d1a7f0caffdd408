// Large-tile float32 MFMA contraction for gfx950 with direct global -> LDS loads
// (global_load_lds_dwordx4):
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k)
//
// 256 threads (4 wave64 in 2 x 2) own a 256 x 256 tile; a wave owns 128 x 128 as 4 x 4 blocks
// of v_mfma_f32_32x32x2_f32, all 256 accumulators of a lane in AGPRs.  With no staging
// registers a wave keeps one wave per SIMD busy by itself: per stage of 16 k it issues 128
// MFMAs (64 cycles each) against 8 load instructions, 8 to 16 fragment reads and one barrier.
// Compared with 128 x 128 tiles the operand bytes per flop halve.
//
// Stage tiles hold 256 rows (or columns) of 16 k per operand, 16 KiB each, four stages
// (128 KiB), one barrier per stage as in the bfloat16 engine: past it every wave has its
// share of the next stage in LDS and is done with the one before this, whose buffer then
// takes the loads three stages ahead.
//
// Both operands hand the MFMAs their k values in the same order: in half g of a stage, MFMA
// step q, lane half h supplies k = 8 g + 4 h + q.  A row-major operand (k contiguous) then
// reads its four values of a half with one 16-byte LDS load.
//
// Operand kinds:
//   FdlRows : element (m, k) at p[m * ld + k].  Stage layout [256][16] with row r's 16-byte
//             chunk c at position c ^ ((r / 4) % 4); one load instruction moves 16 rows,
//             lane i carrying row i / 4 and the chunk that lands at position i % 4.
//   FdlCols : element (m, k) at p[k * ld + m].  Stage layout [16][256]; one load
//             instruction moves one k row of 256 values; fragment values are single reads.
// Requirements (checked by the host side): 16-byte aligned bases, ld % 4 == 0, every k range
// a whole number of stages inside [0, K); FdlCols: M % 4 == 0.  Rows (columns) at or past M
// are clamped to the last one; their outputs are discarded by the epilogue's range checks.
#pragma once

#include "gemm_bf16_dl.h"

namespace pwq {

constexpr int FDL_BK = 16;                               // k per stage
constexpr int FDL_NS = 4;                                // stages

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void fdl_load16(const float* g, float* lds_wave_base) {
    __builtin_amdgcn_global_load_lds((const void*)g, (lds_ptr_t)lds_wave_base, 16, 0, 0);
}

// float offset of row r's logical chunk c (four floats) in an FdlRows stage tile
__device__ __forceinline__ int fdl_off(int r, int c) { return r * FDL_BK + 4 * (c ^ ((r >> 2) & 3)); }

// Tiles of T x T (T = 256 or 128): a stage holds T x 16 floats per operand, which T / 16
// load instructions of 1 KiB move, T / 64 per wave.
template <int T>
struct FdlRows {
    static constexpr int kTile = T;
    static constexpr int kReads = 1;                     // LDS reads per fragment
    static constexpr int kLoads = T / 64;                // load instructions per wave and stage
    const float* p;
    int64_t ld, M;
    // rows m0 .. m0 + T - 1, k0 .. k0 + 15 into S: wave w issues the 16-row groups w + 4 q
    __device__ __forceinline__ void load(float* S, int64_t m0, int64_t k0, int wave, int lane) const {
        const int pc = lane & 3, rl = lane >> 2;
        const int lc = pc ^ ((rl >> 2) & 3);               // logical chunk landing at pc
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int r0 = 16 * (wave + 4 * q);
            int64_t row = m0 + r0 + rl;
            if (row > M - 1) row = M - 1;
            fdl_load16(p + row * ld + k0 + 4 * lc, S + r0 * FDL_BK);
        }
    }
    // the four values of half g for row r (tile-relative) and lane half h
    __device__ __forceinline__ f32x4 frag(const float* S, int r, int h, int g) const {
        return *(const f32x4*)(S + fdl_off(r, 2 * g + h));
    }
};

// Stage layout [16][T]: one load instruction moves 256 / T whole k rows (lane l: k row
// l / (T / 4), columns 4 (l % (T / 4)) .. + 3)
template <int T>
struct FdlCols {
    static constexpr int kTile = T;
    static constexpr int kReads = 4;
    static constexpr int kLoads = T / 64;
    static constexpr int RPI = 256 / T;                  // k rows per instruction
    const float* p;
    int64_t ld, M;
    // k rows k0 .. k0 + 15 of columns m0 .. m0 + T - 1 into S: wave w issues the row groups w + 4 q
    __device__ __forceinline__ void load(float* S, int64_t m0, int64_t k0, int wave, int lane) const {
        int64_t col = m0 + 4 * (lane % (T / 4));
        if (col > M - 4) col = M - 4;
        const int kl = lane / (T / 4);
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            const int kr = RPI * (wave + 4 * q);
            fdl_load16(p + (k0 + kr + kl) * ld + col, S + kr * T);
        }
    }
    __device__ __forceinline__ f32x4 frag(const float* S, int r, int h, int g) const {
        const float* c = S + (8 * g + 4 * h) * T + r;
        f32x4 v;
        v[0] = c[0];
        v[1] = c[T];
        v[2] = c[2 * T];
        v[3] = c[3 * T];
        return v;
    }
};

// Issue order of a half stage (MH MFMAs): NV times one MFMA and one global load, NR times one
// MFMA and one LDS read (NR = the half's fragment reads), then the other MFMAs.  Loads and
// reads go out while the matrix pipe is busy; with one wave per SIMD nothing else fills it.
template <int NV, int NR, int MH>
__device__ __forceinline__ void fdl_interleave() {
    static_assert(NV + NR <= MH, "interleave");
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (MH > NV + NR) __builtin_amdgcn_sched_group_barrier(0x008, MH - NV - NR, 0);
}

template <int FM, int FN>
__device__ __forceinline__ void fdl_mfma_half(f32x16 (&acc)[FM][FN], const f32x4 (&a)[FM], const f32x4 (&b)[FN]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][q], b[j][q], acc[i][j], 0, 0, 0);
}

// floats of LDS a launch of T x T tiles takes
template <int T>
constexpr int fdl_lds_floats() { return FDL_NS * 2 * T * FDL_BK; }

template <class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_fdl_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, float* lds) {
    constexpr int T = LA::kTile;
    static_assert(LB::kTile == T, "one tile size");
    constexpr int FM = T / 64, FN = T / 64;                // 32 x 32 blocks per wave (a wave owns T/2 x T/2)
    constexpr int OP = T * FDL_BK, STAGE = 2 * OP;
    constexpr int NV = LA::kLoads + LB::kLoads;          // load instructions per wave and stage
    constexpr int MH = 4 * FM * FN;                      // MFMAs per half stage
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

    // Stage st is copied during iteration st - 3 (the first three before the loop), into buffer
    // st % 4.  Past the last stage the copies repeat the last one into a buffer nothing reads
    // any more, so every iteration issues the same NV loads per wave, with no branch in the
    // loop body; a wave waits for all its copies before it leaves.
    const int64_t nk = (t.kend - t.kbeg) / FDL_BK;       // host guarantees whole stages, nk >= 1
    auto kof = [&](int64_t st) { return t.kbeg + (st < nk ? st : nk - 1) * FDL_BK; };
#pragma unroll
    for (int st = 0; st < FDL_NS - 1; ++st) {
        la.load(lds + st * STAGE, t.m0, kof(st), wave, lane);
        lb.load(lds + st * STAGE + OP, t.n0, kof(st), wave, lane);
    }
    const int ar = wm * (T / 2) + (lane & 31);
    const int br = wn * (T / 2) + (lane & 31);
    const int h = lane >> 5;
    wait_vmcnt<2 * NV>();
    barrier_nofence();
    constexpr int NR = FM * LA::kReads + FN * LB::kReads;
    f32x4 a0[FM], b0[FN], a1[FM], b1[FN];                 // halves g = 0 and g = 1 of a stage
#pragma unroll
    for (int i = 0; i < FM; ++i) a0[i] = la.frag(lds, ar + 32 * i, h, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = lb.frag(lds + OP, br + 32 * j, h, 0);

    for (int64_t it = 0; it < nk; ++it) {
        const float* S = lds + (it & 3) * STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) a1[i] = la.frag(S, ar + 32 * i, h, 1);
#pragma unroll
        for (int j = 0; j < FN; ++j) b1[j] = lb.frag(S + OP, br + 32 * j, h, 1);
        fdl_mfma_half<FM, FN>(acc, a0, b0);
        fdl_interleave<0, NR, MH>();
        // this wave's copy of stage it + 1 has landed (that of it + 2 may still fly); past the
        // barrier every wave's has, and every wave is done with stage it - 1, whose buffer
        // takes stage it + 3
        wait_vmcnt<NV>();
        barrier_nofence();
        float* Sl = lds + ((it + 3) & 3) * STAGE;
        la.load(Sl, t.m0, kof(it + 3), wave, lane);
        lb.load(Sl + OP, t.n0, kof(it + 3), wave, lane);
        // the next stage's first half (after the last stage these read a buffer no copy
        // targets any more, and go unused)
        const float* Sn = lds + ((it + 1) & 3) * STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i) a0[i] = la.frag(Sn, ar + 32 * i, h, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = lb.frag(Sn + OP, br + 32 * j, h, 0);
        fdl_mfma_half<FM, FN>(acc, a1, b1);
        fdl_interleave<NV, NR, MH>();
        // keep those reads in this iteration, and their wait after this half's MFMAs
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(a0[i]));
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(b0[j]));
    }
    wait_vmcnt<0>();

    if constexpr (EpiIsRmw<EPI>::value) {
        const int wu = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform corner for buffer addressing
        epi_rmw_wave<FM, FN>(epi, t, acc, t.m0 + (wu & 1) * (T / 2), t.n0 + (wu >> 1) * (T / 2), lane,
                             epi_whole(epi, t, T, T));
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t r0 = t.m0 + wm * (T / 2) + i * 32 + 4 * (lane >> 5);
                const int64_t col = t.n0 + wn * (T / 2) + j * 32 + (lane & 31);
                epi_block16(epi, t, acc[i][j], [&](int v) { return r0 + 8 * (v >> 2) + (v & 3); }, col);
            }
    }
}

template <class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_fdl_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    constexpr int T = LA::kTile;
    __shared__ __attribute__((aligned(16))) float lds[fdl_lds_floats<T>()];
    Tile t;
    if (!map.get((int)blockIdx.x, T, T, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_fdl_tile(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

// One launch, two independent tile tasks on this engine: blocks [0, n1) run task a, the rest b.
template <class LA_, class LB_, class MAP_, class EPI_>
struct FdlTask {
    static constexpr int kTile = LA_::kTile;
    static constexpr int LDS = fdl_lds_floats<LA_::kTile>();
    LA_ la;
    LB_ lb;
    MAP_ map;
    EPI_ epi;
    __device__ __forceinline__ void run(int bid, float* lds) {
        Tile t;
        if (!map.get(bid, kTile, kTile, t)) {
            epi.finish(t, threadIdx.x, false);
            return;
        }
        gemm_fdl_tile(la, lb, t, epi, lds);
        epi.finish(t, threadIdx.x, true);
    }
};

template <class TA, class TB>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_fdl_dual_kernel(TA a, TB b, int n1, const int32_t* guard) {
    if (guard && *guard != 0) return;
    static_assert(TA::kTile == TB::kTile, "one tile size");
    __shared__ __attribute__((aligned(16))) float lds[fdl_lds_floats<TA::kTile>()];
    if ((int)blockIdx.x < n1) a.run((int)blockIdx.x, lds);
    else b.run((int)blockIdx.x - n1, lds);
}

}  // namespace pwq
