// Hessian of the layer objective, H = 2 X^T X summed over calibration tokens
// ("GPTQ: Post-Training INT4", section "Hessian-Based Weight Update"), its damping by
// damp * mean(diag H) and the act-order permutation (desc_act of the same page,
// section "Running GPTQ with AutoGPTQ").
//
// The contraction runs over the upper-triangular tiles of H only, accumulating in float32.
// bfloat16 X: bfloat16 MFMA (products exact), large problems on the 256 x 256 engine
// through a transposed, tile-major copy (operand tiles staged global -> VGPR -> LDS).
// float32 X: small problems on the float32 MFMA engine; larger ones as the four products of
// a bfloat16 pair X = XH + XL on the same 256 x 256 engine (each product exact; only X's
// residual below 2^-17 relative is dropped).  Small d_in gives few tiles, so the token
// range is cut into chunks whose partial tiles land in a workspace and are summed in a
// fixed order (bit-reproducible, no atomics).  A last pass copies the upper triangle onto
// the lower one.
#include "gemm_bf16_dl.h"
#include "../../include/pwq.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// split > 1: partial tile of chunk `split` -> ws[split][tile][BM*BN]
// split == 1: H[row][col] += 2 * acc directly (upper tiles only; diagonal tiles whole)
struct EpiHess {
    static constexpr bool kRmw = true;
    float* H;
    float* part;
    int64_t n;
    int full, ntail, bm;       // whole-k tiles [0, full) add into H; split tiles write partials
    __device__ __forceinline__ float old(const Tile& t, int64_t row, int64_t col) const {
        return (t.split < 0 && row < n && col < n) ? H[row * n + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile& t, int64_t row, int64_t col, float v, float o) {
        if (t.split < 0) {
            if (row < n && col < n) H[row * n + col] = o + 2.f * v;
        } else {
            int64_t lr = row - t.m0, lc = col - t.n0;
            part[((int64_t)t.split * ntail + (t.tile - full)) * (int64_t)(bm * bm) + lr * bm + lc] = v;
        }
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

// H[tile] += 2 * sum_s part[s][tile - full] over the split tiles, s in increasing order;
// tile numbers in the plain order, or (band) in the band order of upper_band_tile.
// grid: x = 1024-element chunk of a tile, y = split tile index (tile - full)
__global__ __launch_bounds__(256) void hess_reduce_kernel(const float* __restrict__ part, float* __restrict__ H,
                                                          int64_t n, int tiles, int full, int splits, int bm, int band) {
    const int ntail = tiles * (tiles + 1) / 2 - full;
    const int tile = full + (int)blockIdx.y;
    int ti = 0, tj = 0;
    if (band) {
        upper_band_tile(tile, tiles, 4, ti, tj);
    } else {
        int r = tile;
        while (r >= tiles - ti) { r -= tiles - ti; ++ti; }
        tj = ti + r;
    }
    const int64_t per_tile = (int64_t)bm * bm;
    const int64_t le = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
    if (le >= per_tile) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < splits; ++sp) {
        const float4 v = *(const float4*)(part + ((int64_t)sp * ntail + blockIdx.y) * per_tile + le);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const int64_t row = (int64_t)ti * bm + le / bm, col = (int64_t)tj * bm + le % bm;
    if (row >= n) return;
    const float a[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (col + c < n) H[row * n + col + c] += 2.f * a[c];
}

// lower triangle := upper triangle, 64 x 64 blocks through LDS (coalesced both ways); grid
// (column block bj, row block bi), blocks below the diagonal return at once
__global__ __launch_bounds__(256) void mirror_upper_kernel(float* __restrict__ H, int64_t n) {
    const int64_t bi = blockIdx.y, bj = blockIdx.x;
    if (bi > bj) return;
    __shared__ float tile[64][65];
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
#pragma unroll 4
    for (int k = ty; k < 64; k += 4) {
        const int64_t i = bi * 64 + k, j = bj * 64 + tx;
        tile[k][tx] = (i < n && j < n) ? H[i * n + j] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = ty; k < 64; k += 4) {
        const int64_t i = bj * 64 + k, j = bi * 64 + tx;      // target H[i][j] = H[j][i], i > j
        if (i < n && j < n && i > j) H[i * n + j] = tile[tx][k];
    }
}

__global__ __launch_bounds__(256) void damp_kernel(float* __restrict__ H, int64_t n, float damp, float* lambda_out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)H[i * n + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    const float lam = (float)((double)damp * (red[0] / (double)n));
    for (int64_t i = threadIdx.x; i < n; i += 256) H[i * n + i] += lam;
    if (threadIdx.x == 0 && lambda_out) *lambda_out = lam;
}

// rank of column i in the descending order of diag H, ties by lower index: a stable,
// comparison-count sort (each rank is unique, so perm[rank] = i fills perm exactly).
__global__ __launch_bounds__(256) void act_order_kernel(const float* __restrict__ H, int64_t n, int32_t* __restrict__ perm) {
    __shared__ float d[1024];
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const float di = i < n ? H[i * n + i] : 0.f;
    int64_t rank = 0;
    for (int64_t j0 = 0; j0 < n; j0 += 1024) {
        __syncthreads();
        for (int t = threadIdx.x; t < 1024; t += 256) d[t] = (j0 + t < n) ? H[(j0 + t) * n + (j0 + t)] : 0.f;
        __syncthreads();
        const int lim = (int)((n - j0) < 1024 ? (n - j0) : 1024);
        for (int t = 0; t < lim; ++t) {
            const float dj = d[t];
            rank += (dj > di) || (dj == di && (j0 + t) < i);
        }
    }
    if (i < n) perm[rank] = (int32_t)i;
}

// The same ranks for n <= PERM_MAX_N: every workgroup stages the whole diagonal in LDS once
// (so one workgroup fits a CU, and it takes 16 waves), and four threads count for each
// column, thread q of the four over the float4 chunks q, q + 4, q + 8, ... (the four
// addresses a wave reads at once fall in different banks); the quad's counts are summed
// with two lane exchanges.  256 columns per workgroup.
__global__ __launch_bounds__(1024) void act_order_lds_kernel(const float* __restrict__ H, int64_t n,
                                                             int32_t* __restrict__ perm) {
    __shared__ __attribute__((aligned(16))) float d[PERM_MAX_N];
    constexpr int NT = 1024, UR = 8;                     // strided loads in batches of eight per thread
    for (int64_t j0 = 0; j0 < n; j0 += NT * UR) {
        float v[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = j0 + u * NT + threadIdx.x;
            v[u] = j < n ? H[j * n + j] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = j0 + u * NT + threadIdx.x;
            if (j < n) d[j] = v[u];
        }
    }
    __syncthreads();
    const int q = (int)(threadIdx.x & 3);
    const int64_t i64 = (int64_t)blockIdx.x * 256 + (threadIdx.x >> 2);
    const bool live = i64 < n;                           // every lane takes part in the exchanges
    const int i = live ? (int)i64 : 0, nn = (int)n;
    const float di = d[i];
    int rank = 0;
    const int n4 = nn / 4;
    for (int t = q; t < n4; t += 4) {
        const float4 c = ((const float4*)d)[t];
        const int j = 4 * t;
        rank += (c.x > di) || (c.x == di && j < i);
        rank += (c.y > di) || (c.y == di && j + 1 < i);
        rank += (c.z > di) || (c.z == di && j + 2 < i);
        rank += (c.w > di) || (c.w == di && j + 3 < i);
    }
    if (q == 0)
        for (int j = 4 * n4; j < nn; ++j) rank += (d[j] > di) || (d[j] == di && j < i);
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    if (live && q == 0) perm[rank] = i;
}

// bfloat16 X: native bf16 MFMA (products exact in float32), 128 x 128 upper tiles; the two
// operand loaders split the 256 threads (each tile operand has 128 transposing blocks)
hipError_t hess_gemm_bf16(const void* X, int64_t n_tok, int64_t n, int64_t ldx, float* H, float* part, const HessPlan& pl,
                          hipStream_t s) {
    const int vec = (ldx % 8 == 0) && aligned(X, 16);
    Bf16Cols a{(const uint16_t*)X, ldx, n, n_tok, vec, 0};
    Bf16Cols b{(const uint16_t*)X, ldx, n, n_tok, vec, GEMM_THREADS / 2};
    UpperMap map{n, n_tok, pl.tiles, pl.splits, pl.kchunk, nullptr, pl.full};
    const int ntile = pl.tiles * (pl.tiles + 1) / 2;
    EpiHess epi{H, part, n, pl.full, ntile - pl.full, 128};
    prof_begin(PWQ_PROF_XTX, s);
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, Bf16Cols, Bf16Cols, UpperMap, EpiHess>),
                       dim3(pl.full + (ntile - pl.full) * pl.splits), dim3(GEMM_THREADS), 0, s, a, b, map, epi);
    prof_end(PWQ_PROF_XTX, s, (double)n_tok * n * (n + 1));
    return hipGetLastError();
}

// XT[c][t] = X[t][c] for t < n_tok, 0 for n_tok <= t < npad: 64 tokens x 64 columns per
// workgroup through LDS, 16-byte reads and writes (bfloat16 bits are moved, not converted)
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ X, int64_t n_tok, int64_t n,
                                                             int64_t ldx, int vec, uint16_t* __restrict__ XT,
                                                             int64_t npad) {
    __shared__ uint16_t tile[64][64 + 8];
    const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = tid + 256 * h;
        const int r = idx >> 3, ch = (idx & 7) * 8;        // token row r, columns ch .. ch+7
        const int64_t t = t0 + r, c = c0 + ch;
        uint16_t v[8];
        if (vec && t < n_tok && c + 8 <= n) {
            const uint4 q = *(const uint4*)(X + t * ldx + c);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) { v[2 * k] = (uint16_t)(w[k] & 0xffff); v[2 * k + 1] = (uint16_t)(w[k] >> 16); }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = (t < n_tok && c + k < n) ? X[t * ldx + c + k] : (uint16_t)0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) tile[r][ch + k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = tid + 256 * h;
        const int cr = idx >> 3, tch = (idx & 7) * 8;      // output row = column cr, tokens tch .. +7
        const int64_t c = c0 + cr;                         // rows past n (panel padding) get zeros
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = c < n ? ((uint32_t)tile[tch + 2 * k][cr] | ((uint32_t)tile[tch + 2 * k + 1][cr] << 16)) : 0u;
        *(uint4*)(XT + dl_tiled_index(c, t0 + tch, npad)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// float32 X split into a bfloat16 pair, transposed: XH[c][t] = bf16(X[t][c]), XL[c][t] =
// bf16(X[t][c] - XH[c][t]), zero for n_tok <= t < npad (64 x 64 per workgroup through LDS)
__global__ __launch_bounds__(256) void transpose_split_f32_kernel(const float* __restrict__ X, int64_t n_tok, int64_t n,
                                                                  int64_t ldx, int vec, uint16_t* __restrict__ XH,
                                                                  uint16_t* __restrict__ XL, int64_t npad) {
    __shared__ uint16_t th[64][64 + 8];
    __shared__ uint16_t tl[64][64 + 8];
    const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int idx = tid + 256 * h;
        const int r = idx >> 4, ch = (idx & 15) * 4;       // token row r, columns ch .. ch+3
        const int64_t t = t0 + r, c = c0 + ch;
        float v[4];
        if (vec && t < n_tok && c + 4 <= n) {
            const float4 q = *(const float4*)(X + t * ldx + c);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) v[k] = (t < n_tok && c + k < n) ? X[t * ldx + c + k] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint16_t hb = f32_to_bf16_bits(v[k]);
            th[r][ch + k] = hb;
            tl[r][ch + k] = f32_to_bf16_bits(v[k] - bf16_bits_to_f32(hb));
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = tid + 256 * h;
        const int cr = idx >> 3, tch = (idx & 7) * 8;
        const int64_t c = c0 + cr;                         // rows past n (panel padding) get zeros
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            wh[k] = c < n ? ((uint32_t)th[tch + 2 * k][cr] | ((uint32_t)th[tch + 2 * k + 1][cr] << 16)) : 0u;
            wl[k] = c < n ? ((uint32_t)tl[tch + 2 * k][cr] | ((uint32_t)tl[tch + 2 * k + 1][cr] << 16)) : 0u;
        }
        const int64_t o = dl_tiled_index(c, t0 + tch, npad);
        *(uint4*)(XH + o) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        *(uint4*)(XL + o) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
}

// workgroups of the 256 x 256 Hessian in the per-XCD order of UpperMap (xcd set)
int hess_dl_grid(const HessPlan& pl, int ntile) {
    const int nsplit = pl.full < ntile ? (ntile - pl.full) * pl.splits : 0;
    return 8 * ((pl.full + 7) / 8 + (nsplit + 7) / 8);
}

// bfloat16 X on the 256 x 256 engine: both operands are rows of the transposed copy
// (stored tile-major, zero past n_tok and past n), 256 x 256 upper tiles
hipError_t hess_gemm_dl(const void* X, int64_t n_tok, int64_t n, int64_t ldx, float* H, uint16_t* XT, float* part,
                        const HessPlan& pl, hipStream_t s) {
    const int vec = (ldx % 8 == 0) && aligned(X, 16);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(pl.npad / 64), (unsigned)(cdiv(n, DL_TILE) * (DL_TILE / 64))),
                       dim3(256), 0, s, (const uint16_t*)X, n_tok, n, ldx, vec, XT, pl.npad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DlTiled1 op{XT, pl.npad};
    const int ntile = pl.tiles * (pl.tiles + 1) / 2;
    // work items in L2-friendly bands, an equal share per XCD
    UpperMap map{n, pl.npad, pl.tiles, pl.splits, pl.kchunk, nullptr, pl.full, 1};
    EpiHess epi{H, part, n, pl.full, ntile - pl.full, DL_TILE};
    const int nwg = hess_dl_grid(pl, ntile);
    prof_begin(PWQ_PROF_XTX, s);
    // register-staged loads, two tiles per unrolled step: k ranges are whole multiples of
    // 64 (npad and kchunk are)
    static_assert(BK16 % (2 * DL_BK) == 0, "k chunks must hold whole pairs of k-tiles");
    hipLaunchKernelGGL((gemm_rs_kernel<2, DlTiled1, DlTiled1, UpperMap, EpiHess>), dim3(nwg), dim3(GEMM_THREADS),
                       0, s, op, op, map, epi);
    prof_end(PWQ_PROF_XTX, s, (double)n_tok * n * (n + 1));
    return hipGetLastError();
}

// float32 X on the 256 x 256 engine: X = XH + XL (+ a residual below 2^-17 |x|), and
// X^T X = XH XH^T + XH XL^T + XL XH^T + XL XL^T, all four products exact in float32, summed
// by one contraction over four k segments (A: XH XH XL XL, B: XH XL XH XL)
hipError_t hess_gemm_dl4(const void* X, int64_t n_tok, int64_t n, int64_t ldx, float* H, uint16_t* XH, float* part,
                         const HessPlan& pl, hipStream_t s) {
    uint16_t* XL = XH + cdiv(n, DL_TILE) * DL_TILE * pl.npad;
    const int vec = (ldx % 4 == 0) && aligned(X, 16);
    hipLaunchKernelGGL(transpose_split_f32_kernel, dim3((unsigned)(pl.npad / 64), (unsigned)(cdiv(n, DL_TILE) * (DL_TILE / 64))),
                       dim3(256), 0, s, (const float*)X, n_tok, n, ldx, vec, XH, XL, pl.npad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DlTiled4 a{{XH, XH, XL, XL}, pl.npad};
    DlTiled4 b{{XH, XL, XH, XL}, pl.npad};
    const int ntile = pl.tiles * (pl.tiles + 1) / 2;
    // work items in L2-friendly bands, an equal share per XCD
    UpperMap map{n, 4 * pl.npad, pl.tiles, pl.splits, pl.kchunk, nullptr, pl.full, 1};
    EpiHess epi{H, part, n, pl.full, ntile - pl.full, DL_TILE};
    const int nwg = hess_dl_grid(pl, ntile);
    prof_begin(PWQ_PROF_XTX, s);
    hipLaunchKernelGGL((gemm_rs_kernel<2, DlTiled4, DlTiled4, UpperMap, EpiHess>), dim3(nwg), dim3(GEMM_THREADS),
                       0, s, a, b, map, epi);
    prof_end(PWQ_PROF_XTX, s, (double)n_tok * n * (n + 1));
    return hipGetLastError();
}

template <int BM, int DT>
hipError_t hess_gemm(const void* X, int64_t n_tok, int64_t n, int64_t ldx, float* H, float* part, const HessPlan& pl,
                     hipStream_t s) {
    typedef typename Elem<DT>::T T;
    OpKMajor<DT> op{(const T*)X, ldx, n, n_tok, (int)((ldx % 4 == 0) && aligned(X, 4 * sizeof(T)))};
    UpperMap map{n, n_tok, pl.tiles, pl.splits, pl.kchunk, nullptr, pl.full};
    const int ntile = pl.tiles * (pl.tiles + 1) / 2;
    EpiHess epi{H, part, n, pl.full, ntile - pl.full, BM};
    prof_begin(PWQ_PROF_XTX, s);
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BM, OpKMajor<DT>, OpKMajor<DT>, UpperMap, EpiHess>),
                       dim3(pl.full + (ntile - pl.full) * pl.splits), dim3(GEMM_THREADS), 0, s, op, op, map, epi);
    prof_end(PWQ_PROF_XTX, s, (double)n_tok * n * (n + 1));
    return hipGetLastError();
}

}  // namespace

HessPlan hessian_plan(int64_t n_tok, int64_t d_in, int x_dtype) {
    HessPlan p{};
    const bool bf = x_dtype == 2;
    // bfloat16 X with enough 256-wide tiles (and tokens) goes through a transposed copy;
    // float32 X through a transposed bfloat16 pair (four products), once there are enough
    // tokens for the split to pay
    p.dl = (bf && d_in >= 1024 && n_tok >= 256) ? 1 : ((!bf && d_in >= 256 && n_tok >= 1024) ? 4 : 0);
    p.bm = p.dl ? DL_TILE : ((!bf && d_in <= 1024) ? 64 : 128);
    p.tiles = (int)cdiv(d_in, p.bm);
    const int ntile = p.tiles * (p.tiles + 1) / 2;
    const int kq = (bf || p.dl) ? BK16 : GEMM_BK;       // chunk boundaries on whole k-tiles
    p.npad = p.dl ? cdiv(n_tok, 64) * 64 : n_tok;
    const int64_t ksteps = cdiv(p.npad * (p.dl == 4 ? 4 : 1), kq);
    // one 256-wide workgroup per CU (LDS), else >= 4 workgroups per CU of 256
    // Workgroups resident at once: one 256-wide tile per CU (LDS), else about four per CU.
    // Whole rounds of tiles run over all tokens; the tiles left over (all of them when there
    // are fewer than a round) are split into token chunks so that the last round is not a
    // handful of full-length workgroups on an idle chip.  The split count minimises rounds x
    // workgroup length (a fixed cost of about four k tiles each), preferring fewer chunks
    // unless more are at least 2 % faster; a chunk holds at least 8 k tiles.  Splitting
    // (partial tiles in the workspace, one more pass) must save 3 % of the whole call.
    const int conc = p.dl ? 256 : 1024;
    int full = (ntile / conc) * conc;
    const int tail = ntile - full;
    const int64_t max_splits = ksteps / 8 > 1 ? ksteps / 8 : 1;
    int64_t splits = 1;
    if (tail > 0) {
        double best = 0.0, whole = 0.0;
        for (int64_t sp = 1; sp <= max_splits; ++sp) {
            const double cost = (double)cdiv(tail * sp, conc) * (double)(cdiv(ksteps, sp) + 4);
            if (sp == 1) whole = cost;
            if (sp == 1 || cost < 0.98 * best) {
                best = cost;
                splits = sp;
            }
        }
        const double rounds_full = (double)(full / conc) * (double)(ksteps + 4);
        if (rounds_full + best > 0.97 * (rounds_full + whole)) splits = 1;
    }
    p.kchunk = cdiv(ksteps, splits) * kq;
    p.splits = (int)cdiv(p.npad * (p.dl == 4 ? 4 : 1), p.kchunk);
    if (p.splits <= 1) {
        p.splits = 1;
        full = ntile;                                    // nothing split: every tile adds into H
    }
    p.full = full;
    const int copies = p.dl == 4 ? 2 : (p.dl ? 1 : 0);   // transposed X, or its bfloat16 pair
    // the transposed copy is tile-major, rows padded to whole 256-row panels
    p.xt_bytes = align_up((size_t)copies * cdiv(d_in, DL_TILE) * DL_TILE * p.npad * sizeof(uint16_t), 256);
    const size_t parts = p.splits > 1 ? (size_t)p.splits * (ntile - full) * p.bm * p.bm * sizeof(float) : 0;
    p.ws_bytes = p.xt_bytes + parts;
    return p;
}

hipError_t hessian_launch(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, float* H, void* ws,
                          hipStream_t s) {
    if (n_tok == 0 || d_in == 0) return hipSuccess;
    const HessPlan pl = hessian_plan(n_tok, d_in, x_dtype);
    float* part = (float*)((char*)ws + pl.xt_bytes);
    hipError_t e;
    if (pl.dl == 4) {
        e = hess_gemm_dl4(X, n_tok, d_in, ldx, H, (uint16_t*)ws, part, pl, s);
    } else if (x_dtype == 0) {
        e = pl.bm == 64 ? hess_gemm<64, 0>(X, n_tok, d_in, ldx, H, part, pl, s) : hess_gemm<128, 0>(X, n_tok, d_in, ldx, H, part, pl, s);
    } else if (pl.dl) {
        e = hess_gemm_dl(X, n_tok, d_in, ldx, H, (uint16_t*)ws, part, pl, s);
    } else {
        e = hess_gemm_bf16(X, n_tok, d_in, ldx, H, part, pl, s);
    }
    if (e != hipSuccess) return e;
    if (pl.splits > 1) {
        const int ntail = pl.tiles * (pl.tiles + 1) / 2 - pl.full;
        const unsigned chunks = (unsigned)cdiv((int64_t)pl.bm * pl.bm, 1024);
        hipLaunchKernelGGL(hess_reduce_kernel, dim3(chunks, (unsigned)ntail), dim3(256), 0, s, part, H, d_in, pl.tiles,
                           pl.full, pl.splits, pl.bm, pl.dl ? 1 : 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const unsigned nb = (unsigned)cdiv(d_in, 64);
    hipLaunchKernelGGL(mirror_upper_kernel, dim3(nb, nb), dim3(256), 0, s, H, d_in);
    return hipGetLastError();
}

hipError_t damp_launch(float* H, int64_t n, float damp, float* lambda_out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, s, H, n, damp, lambda_out);
    return hipGetLastError();
}

hipError_t act_order_launch(const float* H, int64_t n, int32_t* perm, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (n <= PERM_MAX_N) hipLaunchKernelGGL(act_order_lds_kernel, dim3((unsigned)cdiv(n, 256)), dim3(1024), 0, s, H, n, perm);
    else hipLaunchKernelGGL(act_order_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, H, n, perm);
    return hipGetLastError();
}

}  // namespace pwq
