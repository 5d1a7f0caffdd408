// Tiled float32 MFMA contraction engine for gfx950 (v_mfma_f32_32x32x2_f32).
//
//   acc(m, n) = sum_{k in [kbeg, kend)} A(m, k) * B(n, k)
//
// A workgroup of 256 threads (4 wave64s in a 2 x 2 grid) owns a BM x BN output tile;
// each wave owns (BM/2) x (BN/2) as 32 x 32 MFMA blocks.  Operand tiles of BK = 32
// along k are staged through LDS as [k][m] (m contiguous), so every MFMA operand read
// is 32 consecutive floats per half-wave.  The next k-tile is fetched into registers
// while the current one is multiplied.  The operand loaders and the epilogue are
// policy types, so the same engine serves the Hessian build, the Cholesky and
// triangular-inverse updates, the GPTQ trailing update and the error GEMM.
#pragma once

#include "pwq_common.h"

namespace pwq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_BK = 32;

// ---------------------------------------------------------------- element access
// DT: 0 = float32, 1 = float16 bits, 2 = bfloat16 bits.  Values widen exactly to float32.
template <int DT> struct Elem;
template <> struct Elem<0> {
    typedef float T;
    static __device__ __forceinline__ float get(const T* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ float4 get4(const T* p, int64_t i) { return *(const float4*)(p + i); }
};
template <> struct Elem<1> {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(const T* p, int64_t i) { return f16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ float4 get4(const T* p, int64_t i) {
        uint2 u = *(const uint2*)(p + i);
        return make_float4(f16_bits_to_f32((uint16_t)(u.x & 0xffff)), f16_bits_to_f32((uint16_t)(u.x >> 16)),
                           f16_bits_to_f32((uint16_t)(u.y & 0xffff)), f16_bits_to_f32((uint16_t)(u.y >> 16)));
    }
};
template <> struct Elem<2> {
    typedef uint16_t T;
    static __device__ __forceinline__ float get(const T* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ float4 get4(const T* p, int64_t i) {
        uint2 u = *(const uint2*)(p + i);
        return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
                           __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u));
    }
};

// ---------------------------------------------------------------- operand loaders
// Element (m, k) stored at p[k * ld + m]: rows of k, m contiguous.
template <int DT = 0>
struct OpKMajor {
    static constexpr int PAD = 4;
    typedef typename Elem<DT>::T T;
    const T* p;
    int64_t ld, M, K;
    int vec;            // ld % 4 == 0 and p aligned to 4 elements

    template <int BM>
    struct Regs { float4 v[BM * GEMM_BK / (4 * GEMM_THREADS)]; };

    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = BM / 4;
        const bool full = vec && (m0 + BM <= M) && (k0 + GEMM_BK <= K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int idx = tid + i * GEMM_THREADS;
            int kr = idx / PER_ROW, mc = (idx % PER_ROW) * 4;
            int64_t k = k0 + kr, m = m0 + mc;
            if (full) {
                r.v[i] = Elem<DT>::get4(p, k * ld + m);
            } else {
                float t[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) t[c] = (k < K && m + c < M) ? Elem<DT>::get(p, k * ld + m + c) : 0.f;
                r.v[i] = make_float4(t[0], t[1], t[2], t[3]);
            }
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(float* S, const Regs<BM>& r, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = BM / 4;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int idx = tid + i * GEMM_THREADS;
            int kr = idx / PER_ROW, mc = (idx % PER_ROW) * 4;
            *(float4*)(S + kr * (BM + PAD) + mc) = r.v[i];
        }
    }
};

// Element (m, k) stored at p[m * ld + k]: rows of m, k contiguous (transposed into LDS).
template <int DT = 0>
struct OpMMajor {
    static constexpr int PAD = 1;
    typedef typename Elem<DT>::T T;
    const T* p;
    int64_t ld, M, K;
    int vec;

    template <int BM>
    struct Regs { float4 v[BM * GEMM_BK / (4 * GEMM_THREADS)]; };

    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = GEMM_BK / 4;
        const bool full = vec && (m0 + BM <= M) && (k0 + GEMM_BK <= K);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int idx = tid + i * GEMM_THREADS;
            int mr = idx / PER_ROW, kc = (idx % PER_ROW) * 4;
            int64_t m = m0 + mr, k = k0 + kc;
            if (full) {
                r.v[i] = Elem<DT>::get4(p, m * ld + k);
            } else {
                float t[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) t[c] = (m < M && k + c < K) ? Elem<DT>::get(p, m * ld + k + c) : 0.f;
                r.v[i] = make_float4(t[0], t[1], t[2], t[3]);
            }
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(float* S, const Regs<BM>& r, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = GEMM_BK / 4;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int idx = tid + i * GEMM_THREADS;
            int mr = idx / PER_ROW, kc = (idx % PER_ROW) * 4;
            S[(kc + 0) * (BM + PAD) + mr] = r.v[i].x;
            S[(kc + 1) * (BM + PAD) + mr] = r.v[i].y;
            S[(kc + 2) * (BM + PAD) + mr] = r.v[i].z;
            S[(kc + 3) * (BM + PAD) + mr] = r.v[i].w;
        }
    }
};

// ---------------------------------------------------------------- tile maps
struct Tile {
    int64_t m0, n0, kbeg, kend;
    int split, tile;
};

// Rectangular grid of BM x BN tiles over M x N, times `splits` chunks of k.
// tri_k: the k range of a tile starts at its m0 (A upper triangular: A(m, k) = 0, k < m).
// Workgroups run in block order: tiles_m fastest (m-blocks of one n-block run together and
// share that B block), or with nfast set, tiles_n fastest (n-blocks of one m-block share A).
struct RectMap {
    int64_t M, N, K;
    int tiles_m, tiles_n, splits;
    int64_t kchunk;
    int tri_k;
    const int32_t* guard;     // optional: skip all work when *guard != 0
    int nfast;
    __device__ __forceinline__ bool get(int bid, int BM, int BN, Tile& t) const {
        int ntile = tiles_m * tiles_n;
        t.split = bid / ntile;
        t.tile = bid % ntile;
        int ti = nfast ? t.tile / tiles_n : t.tile % tiles_m;
        int tj = nfast ? t.tile % tiles_n : t.tile / tiles_m;
        t.m0 = (int64_t)ti * BM;
        t.n0 = (int64_t)tj * BN;
        t.kbeg = (int64_t)t.split * kchunk;
        t.kend = t.kbeg + kchunk < K ? t.kbeg + kchunk : K;
        if (tri_k && t.kbeg < t.m0) t.kbeg = (t.m0 / GEMM_BK) * GEMM_BK;
        return t.kbeg < t.kend;
    }
};

// Upper-triangular tile pairs (ti <= tj) of an N x N output, times `splits` k chunks.
// Position L of the upper tiles in bands of G tile-rows: within a band, columns left to
// right and the band's rows (at most tj) fastest.  Consecutive positions then share a few
// operand blocks of both kinds.
__device__ __forceinline__ void upper_band_tile(int L, int tiles, int G, int& ti, int& tj) {
    int r0 = 0;
    while (r0 < tiles) {
        const int R = tiles - r0 < G ? tiles - r0 : G;
        const int head = R * (R + 1) / 2;                // columns r0 .. r0 + R - 1: 1 .. R rows
        const int cnt = head + R * (tiles - r0 - R);
        if (L < cnt) {
            if (L < head) {
                int c = 0;
                while ((c + 1) * (c + 2) / 2 <= L) ++c;
                ti = r0 + (L - c * (c + 1) / 2);
                tj = r0 + c;
            } else {
                const int p = L - head;
                tj = r0 + R + p / R;
                ti = r0 + p % R;
            }
            return;
        }
        L -= cnt;
        r0 += R;
    }
    ti = tj = 0;
}

// Upper-triangle tiles (ti <= tj) of an N x N output.  Workgroups [0, full) take tiles
// [0, full) over the whole k range (t.split = -1); the tiles after them are split into
// `splits` k chunks of kchunk, workgroup full + s * (ntile - full) + j taking chunk s of tile
// full + j.  With full = 0 every tile is split.
// xcd: tiles taken in bands of four rows (upper_band_tile); t.tile is then the tile's position
// L in that order (the whole tiles are L < full, the split ones full <= L < ntile).  Workgroup
// b runs on XCD b % 8 and takes the b / 8-th item of that XCD's list: first its share of the
// whole tiles (a contiguous run of ceil(full / 8)), then its share of the split items (chunk
// slowest, a contiguous run of ceil((ntile - full) splits / 8)).  Every XCD then has the same
// work, and the workgroups in flight on one XCD share a few operand blocks (and one k range)
// in its L2.  The grid is 8 (ceil(full / 8) + ceil((ntile - full) splits / 8)); padding
// workgroups have no tile.
struct UpperMap {
    int64_t N, K;
    int tiles, splits;
    int64_t kchunk;
    const int32_t* guard;
    int full;
    int xcd;
    __device__ __forceinline__ bool get(int bid, int BM, int BN, Tile& t) const {
        const int ntile = tiles * (tiles + 1) / 2;
        int ti = 0, tj = 0;
        if (xcd) {
            const int ntail = ntile - full, nsplit = ntail > 0 ? ntail * splits : 0;
            const int wpx = (full + 7) / 8, x = bid % 8, p = bid / 8;
            int L;
            if (p < wpx) {
                L = x * wpx + p;
                t.split = -1;
                if (L >= full) L = -1;
            } else {
                const int j = x * ((nsplit + 7) / 8) + (p - wpx);
                t.split = j / (ntail > 0 ? ntail : 1);
                L = j < nsplit ? full + j % ntail : -1;
            }
            if (L < 0) {
                t.split = -1;
                t.tile = 0;
                t.kbeg = t.kend = 0;
                return false;
            }
            upper_band_tile(L, tiles, 4, ti, tj);
            t.tile = L;
        } else {
            if (bid < full) {
                t.split = -1;
                t.tile = bid;
            } else {
                const int nt = ntile - full, b = bid - full;
                t.split = b / nt;
                t.tile = full + b % nt;
            }
            int r = t.tile;
            while (r >= tiles - ti) { r -= tiles - ti; ++ti; }
            tj = ti + r;
        }
        t.m0 = (int64_t)ti * BM;
        t.n0 = (int64_t)tj * BN;
        if (t.split < 0) {
            t.kbeg = 0;
            t.kend = K;
        } else {
            t.kbeg = (int64_t)t.split * kchunk;
            t.kend = t.kbeg + kchunk < K ? t.kbeg + kchunk : K;
        }
        return t.kbeg < t.kend;
    }
};

// Rectangular grid of BM x BN tiles over M x N, whole k range [0, K), in the per-XCD order
// of UpperMap's xcd mode: tiles in bands of four tile-rows, within a band columns left to
// right and the band's rows fastest; workgroup b runs on XCD b % 8 and takes position
// (b % 8) ceil(ntile / 8) + b / 8 of that order.  The workgroups in flight on one XCD then
// hold about four row blocks and eight column blocks of operands in its L2 (with the plain
// order and many row blocks, nearly every workgroup of an XCD reads its own row block).
// Grid: 8 ceil(ntile / 8); padding workgroups have no tile.
struct XcdRectMap {
    int64_t M, N, K;
    int tiles_m, tiles_n;
    const int32_t* guard;
    __device__ __forceinline__ bool get(int bid, int BM, int BN, Tile& t) const {
        const int ntile = tiles_m * tiles_n;
        const int per = (ntile + 7) / 8;
        const int L = (bid % 8) * per + bid / 8;
        t.split = 0;
        t.tile = L;
        t.kbeg = 0;
        if (L >= ntile) {
            t.m0 = t.n0 = 0;
            t.kend = 0;
            return false;
        }
        const int band = L / (4 * tiles_n);              // whole bands of 4 rows before it
        const int r0 = band * 4;
        const int R = tiles_m - r0 < 4 ? tiles_m - r0 : 4;
        const int p = L - band * 4 * tiles_n;
        t.m0 = (int64_t)(r0 + p % R) * BM;
        t.n0 = (int64_t)(p / R) * BN;
        t.kend = K;
        return true;
    }
};
inline int xcd_grid(int ntile) { return 8 * ((ntile + 7) / 8); }

// ---------------------------------------------------------------- epilogue protocol
// Plain epilogues take element(t, row, col, v) for every output.  Epilogues that read the
// output before writing it declare `static constexpr bool kRmw = true` and give
// old(t, row, col) (the value read; 0 when out of range or not needed) and
// put(t, row, col, v, old).  The engines read the 16 values of an accumulator block before
// writing any of them: the compiler cannot prove that one element's write does not alias
// the next element's read, so element-wise read-modify-writes would wait one memory latency
// each.
template <class EPI, class = void>
struct EpiIsRmw { static constexpr bool value = false; };
template <class EPI>
struct EpiIsRmw<EPI, decltype((void)EPI::kRmw)> { static constexpr bool value = EPI::kRmw; };

template <class EPI, class ROW>
__device__ __forceinline__ void epi_block16(EPI& epi, const Tile& t, const f32x16& acc, ROW row_of, int64_t col) {
    if constexpr (EpiIsRmw<EPI>::value) {
        float old[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) old[v] = epi.old(t, row_of(v), col);
#pragma unroll
        for (int v = 0; v < 16; ++v) epi.put(t, row_of(v), col, acc[v], old[v]);
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) epi.element(t, row_of(v), col, acc[v]);
    }
}

// Read-modify-write epilogues may also declare `static constexpr bool kFast = true` and give
//   bool whole(const Tile&, int BM, int BN) const : every element of the BM x BN tile is
//       written, with no range or triangle test
//   float* at(int64_t row, int64_t col) const     : an output element's address (row stride ld)
//   float combine(float old, float v) const       : the value written over old
template <class EPI, class = void>
struct EpiIsFast { static constexpr bool value = false; };
template <class EPI>
struct EpiIsFast<EPI, decltype((void)EPI::kFast)> { static constexpr bool value = EPI::kFast; };

// Raw buffer resource over a wave-uniform base, no range limit (gfx9 descriptor word 3)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const float* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, -1, 0x00020000);
}

// Read-modify-write epilogue of one wave's FM x FN accumulator blocks (32 x 32 MFMA layout:
// lane l holds column c0 + 32 j + l % 32 and rows r0 + 32 i + 4 (l / 32) + 8 (v / 4) + v % 4),
// r0 and c0 wave-uniform.  A whole tile of a fast epilogue goes through buffer loads and
// stores off the wave's corner (per element one scalar row offset and an immediate column
// offset, no 64-bit address arithmetic) and loads the old values of the next row of blocks
// before it writes the current one (two buffers of FN x 16 registers): one memory latency
// is exposed per tile, and nothing is tested per element.  Otherwise each row of blocks
// reads all its old values before writing any: FM latencies per tile instead of FM * FN.
template <int FM, int FN, class EPI>
__device__ __forceinline__ void epi_rmw_wave(EPI& epi, const Tile& t, const f32x16 (&acc)[FM][FN], int64_t r0, int64_t c0,
                                             int lane, bool whole) {
    if constexpr (EpiIsFast<EPI>::value) {
        if (whole) {
            // element (i, j, v): lane offset vq[v % 4], scalar row offset (32 i + 8 (v / 4)) ld,
            // immediate column offset 32 j
            const int ld4 = (int)epi.ld * 4;
            const __amdgpu_buffer_rsrc_t rs = wave_rsrc(epi.at(r0, c0));
            const int vo = 4 * (lane >> 5) * ld4 + 4 * (lane & 31);
            int vq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) vq[q] = vo + q * ld4;
            float old[2][FN][16];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    old[0][j][v] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rs, vq[v & 3] + 128 * j, 8 * (v >> 2) * ld4, 0));
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (i + 1 < FM) {
#pragma unroll
                    for (int j = 0; j < FN; ++j)
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            old[(i + 1) & 1][j][v] = __builtin_bit_cast(
                                float, __builtin_amdgcn_raw_buffer_load_b32(rs, vq[v & 3] + 128 * j,
                                                                            (32 * (i + 1) + 8 * (v >> 2)) * ld4, 0));
                }
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __builtin_bit_cast(uint32_t, epi.combine(old[i & 1][j][v], acc[i][j][v])), rs,
                            vq[v & 3] + 128 * j, (32 * i + 8 * (v >> 2)) * ld4, 0);
            }
            return;
        }
    }
    const int64_t rl = r0 + 4 * (lane >> 5), cl = c0 + (lane & 31);
    if constexpr (EpiIsFast<EPI>::value) {
        // edge tiles of a fast epilogue: block by block, few registers
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                epi_block16(epi, t, acc[i][j], [&](int v) { return rl + 32 * i + 8 * (v >> 2) + (v & 3); }, cl + 32 * j);
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int64_t rb = rl + 32 * i;
            float old[FN][16];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) old[j][v] = epi.old(t, rb + 8 * (v >> 2) + (v & 3), cl + 32 * j);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    epi.put(t, rb + 8 * (v >> 2) + (v & 3), cl + 32 * j, acc[i][j][v], old[j][v]);
        }
    }
}

template <class EPI>
__device__ __forceinline__ bool epi_whole(const EPI& epi, const Tile& t, int bm, int bn) {
    if constexpr (EpiIsFast<EPI>::value) return epi.whole(t, bm, bn);
    else return false;
}


// ---------------------------------------------------------------- the tile engine
// Epilogue interface:
//   __device__ void element(const Tile&, int64_t row, int64_t col, float v)  for every
//       output element of the tile (row < m-extent and col < n-extent checked by the epilogue)
//   __device__ void finish(const Tile&, int tid, bool valid)  once per thread at the end
//       (valid = false: the tile had an empty k range and no element() calls were made).
// Host side guarantees: kchunk and every kbeg are multiples of GEMM_BK.
template <int BM, int BN, class LA, class LB>
struct GemmLds {
    static constexpr int A_FLOATS = GEMM_BK * (BM + LA::PAD);
    static constexpr int B_FLOATS = GEMM_BK * (BN + LB::PAD);
    static constexpr int FLOATS = A_FLOATS + B_FLOATS;
};

// one k-tile of MFMAs from the operand tiles in LDS
template <int BM, int BN, class LA, class LB>
__device__ __forceinline__ void gemm_ktile(const float* As, const float* Bs, f32x16 (&acc)[BM / 64][BN / 64], int lane,
                                           int wm, int wn) {
    constexpr int FM = BM / 64, FN = BN / 64;
#pragma unroll 4
    for (int kk = 0; kk < GEMM_BK; kk += 2) {
        float a[FM], b[FN];
        const int kr = kk + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = As[kr * (BM + LA::PAD) + wm * (BM / 2) + i * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = Bs[kr * (BN + LB::PAD) + wn * (BN / 2) + j * 32 + (lane & 31)];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Short k ranges (at most SHORT_KT k-tiles, e.g. the depth-128 updates of the factor and of
// the GPTQ loop) on small tiles: every k-tile's global loads are issued at the start, so the
// tile waits for one memory latency instead of one per k-tile.
constexpr int SHORT_KT = 4;

template <int BM, int BN, class LA, class LB, class EPI>
__device__ __forceinline__ void gemm_tile(const LA& la, const LB& lb, const Tile& t, EPI& epi, float* lds) {
    constexpr int FM = BM / 64, FN = BN / 64;
    float* As = lds;
    float* Bs = lds + GemmLds<BM, BN, LA, LB>::A_FLOATS;

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

    // kbeg and every split boundary are multiples of GEMM_BK, so a k-tile never reaches into
    // the next chunk; past K both operands are zero-filled.
    bool done = false;
    if constexpr (BM * BN <= 64 * 64) {
        const int nk = (int)((t.kend - t.kbeg + GEMM_BK - 1) / GEMM_BK);
        if (nk <= SHORT_KT) {
            typename LA::template Regs<BM> ra[SHORT_KT];
            typename LB::template Regs<BN> rb[SHORT_KT];
#pragma unroll
            for (int i = 0; i < SHORT_KT; ++i) {
                if (i < nk) {
                    la.template load<BM>(ra[i], t.m0, t.kbeg + i * GEMM_BK, tid);
                    lb.template load<BN>(rb[i], t.n0, t.kbeg + i * GEMM_BK, tid);
                }
            }
#pragma unroll
            for (int i = 0; i < SHORT_KT; ++i) {
                if (i < nk) {
                    __syncthreads();
                    la.template store<BM>(As, ra[i], tid);
                    lb.template store<BN>(Bs, rb[i], tid);
                    __syncthreads();
                    gemm_ktile<BM, BN, LA, LB>(As, Bs, acc, lane, wm, wn);
                }
            }
            done = true;
        }
    }
    if (!done) {
        typename LA::template Regs<BM> ra;
        typename LB::template Regs<BN> rb;
        la.template load<BM>(ra, t.m0, t.kbeg, tid);
        lb.template load<BN>(rb, t.n0, t.kbeg, tid);
        for (int64_t k0 = t.kbeg; k0 < t.kend; k0 += GEMM_BK) {
            __syncthreads();
            la.template store<BM>(As, ra, tid);
            lb.template store<BN>(Bs, rb, tid);
            __syncthreads();
            if (k0 + GEMM_BK < t.kend) {
                la.template load<BM>(ra, t.m0, k0 + GEMM_BK, tid);
                lb.template load<BN>(rb, t.n0, k0 + GEMM_BK, tid);
            }
            gemm_ktile<BM, BN, LA, LB>(As, Bs, acc, lane, wm, wn);
        }
    }

    if constexpr (EpiIsRmw<EPI>::value) {
        const int wu = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform corner for buffer addressing
        epi_rmw_wave<FM, FN>(epi, t, acc, t.m0 + (wu & 1) * (BM / 2), t.n0 + (wu >> 1) * (BN / 2), lane,
                             epi_whole(epi, t, BM, BN));
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t r0 = t.m0 + wm * (BM / 2) + i * 32 + 4 * (lane >> 5);
                const int64_t col = t.n0 + wn * (BN / 2) + j * 32 + (lane & 31);
                epi_block16(epi, t, acc[i][j], [&](int v) { return r0 + 8 * (v >> 2) + (v & 3); }, col);
            }
    }
}

template <int BM, int BN, class LA, class LB, class MAP, class EPI>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_f32_kernel(LA la, LB lb, MAP map, EPI epi) {
    if (map.guard && *map.guard != 0) return;
    __shared__ __attribute__((aligned(16))) float lds[GemmLds<BM, BN, LA, LB>::FLOATS];
    Tile t;
    if (!map.get((int)blockIdx.x, BM, BN, t)) {
        epi.finish(t, threadIdx.x, false);
        return;
    }
    gemm_tile<BM, BN>(la, lb, t, epi, lds);
    epi.finish(t, threadIdx.x, true);
}

// One launch, two independent tile tasks: blocks [0, n1) run task a, the rest task b.
template <int BM_, int BN_, class LA_, class LB_, class MAP_, class EPI_>
struct GemmTask {
    static constexpr int BM = BM_, BN = BN_;
    typedef LA_ LA;
    typedef LB_ LB;
    LA_ la;
    LB_ lb;
    MAP_ map;
    EPI_ epi;
    static constexpr int LDS = GemmLds<BM_, BN_, LA_, LB_>::FLOATS;
    __device__ __forceinline__ void run(int bid, float* lds) {
        Tile t;
        if (!map.get(bid, BM, BN, t)) {
            epi.finish(t, threadIdx.x, false);
            return;
        }
        gemm_tile<BM, BN>(la, lb, t, epi, lds);
        epi.finish(t, threadIdx.x, true);
    }
};

// Trace epilogue for acc = A B with A = dW (element (row, k) at dW[row * ld + k], M x N):
// part[workgroup] = sum over its tile of (acc[row][col] - shift * dW[row][col]) * dW[row][col]
// in float64, so the parts sum to tr(dW (B - shift I) dW^T); shift is a device float
// (NULL: 0) read by the kernel.
struct EpiTrace {
    static constexpr bool kRmw = true;
    const float* dW;
    int64_t ld, M, N;
    double* part;
    const float* shift;
    float acc;
    __device__ __forceinline__ float old(const Tile&, int64_t row, int64_t col) const {
        return (row < M && col < N) ? dW[row * ld + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile&, int64_t, int64_t, float v, float o) {
        const float lam = shift ? *shift : 0.f;
        acc = fmaf(fmaf(-lam, o, v), o, acc);
    }
    __device__ __forceinline__ void finish(const Tile&, int tid, bool) {
        __shared__ double red[GEMM_THREADS / 64];
        const double d = wave_sum_d((double)acc);
        if ((tid & 63) == 0) red[tid >> 6] = d;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < GEMM_THREADS / 64; ++w) s += red[w];
            part[blockIdx.x] = s;
        }
    }
};

template <class TA, class TB>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_f32_dual_kernel(TA a, TB b, int n1, const int32_t* guard) {
    if (guard && *guard != 0) return;
    constexpr int L = TA::LDS > TB::LDS ? TA::LDS : TB::LDS;
    __shared__ __attribute__((aligned(16))) float lds[L];
    if ((int)blockIdx.x < n1) a.run((int)blockIdx.x, lds);
    else b.run((int)blockIdx.x - n1, lds);
}

}  // namespace pwq
