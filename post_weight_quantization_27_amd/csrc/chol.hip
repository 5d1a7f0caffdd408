// Upper Cholesky factor of the inverse Hessian, U with H^-1 = U^T U ("Model Quantization
// Mechanics", section 2.1: GPTQ uses a Cholesky decomposition of H^-1 for its updates).
//
// Route: H = V V^T with V upper triangular (a Cholesky that eliminates from the last
// column to the first), and U = V^-1.  Indeed H^-1 = V^-T V^-1 = U^T U with U upper and
// U_jj = 1 / V_jj > 0, and that factor is unique.  H^-1 itself is never formed.
//
// Blocked with NB = 128, bottom-right to top-left, everything in place in U:
//   top-left  (rows, cols < k0): the trailing matrix A still being factored (upper part)
//   top-right (rows < k0, cols >= k0): R = sum_l V_{., l} U_{l, .} over finished blocks l
//   bottom    (rows >= k0): finished rows of U
// Step k (block rows/cols [k0, k0 + bs)):
//   diag     : A_kk = V_kk V_kk^T and Z_kk = V_kk^-1 in registers of one workgroup;
//              Z_kk is also U's diagonal block
//   trsm     : P = V_{<k, k} = A_{<k, k} Z_kk^T                       (panel workspace)
//   finalize : U_{k, >k} = -Z_kk R_{k, >k}          (from V U = I: V_kk U_kj = -sum_l V_kl U_lj)
//   syrk     : A_{<k, <k} -= P P^T                                    (upper tiles)
//   push     : R_{<k, >=k} += P U_{k, >=k}   (overwrite for the block column k itself)
// trsm + finalize share one launch, syrk + push another: three launches per block.
// Every kernel reads `info` first and does nothing once a pivot has failed.
#include "gemm_f32.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// U[i][j] = H[i][j] for j >= i, 0 below the diagonal; grid (column chunks of 1024, rows)
__global__ __launch_bounds__(256) void copy_upper_kernel(const float* __restrict__ H, float* __restrict__ U, int64_t n) {
    const int64_t i = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * 1024 + threadIdx.x * 4;
    const float* src = H + i * n;
    float* dst = U + i * n;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t j = j0 + c;
        if (j < n) dst[j] = j >= i ? src[j] : 0.f;
    }
}

__global__ void set_int_kernel(int32_t* p, int32_t v) { *p = v; }

// U[i][j] = H[perm[i]][perm[j]] for j >= i, 0 below: row perm[i] of the full symmetric H is
// staged in LDS, so both the read and the write are coalesced.  One workgroup per row.
__global__ __launch_bounds__(256) void copy_perm_kernel(const float* __restrict__ H, const int32_t* __restrict__ perm,
                                                        float* __restrict__ U, int64_t n) {
    __shared__ float row[PERM_MAX_N];
    const int64_t i = blockIdx.x;
    const float* src = H + (int64_t)perm[i] * n;
    for (int64_t j = threadIdx.x; j < n; j += 256) row[j] = src[j];
    __syncthreads();
    float* dst = U + i * n;
    for (int64_t j = threadIdx.x; j < n; j += 256) dst[j] = j >= i ? row[perm[j]] : 0.f;
}

// ------------------------------------------------------------------ diagonal block
// 256 threads as 16 x 16 (tr, tc); thread (tr, tc) holds the 8 x 8 register tile of rows
// tr + 16 ii and columns tc + 16 jj (cyclic), so the active part [0, c) x [0, c) shrinks
// evenly over all threads as pivots retire.  Per pivot, the pivot column (factor) or the
// pivot row and column (inverse) travel through LDS in a permuted layout ([lane % 16][i / 16],
// two 16-byte reads per thread), zero outside the active range so the rank-1 update needs
// no predicates; double buffered, one barrier per pivot.  A ragged block (bs < 128) is
// padded with the identity, which leaves the real part unchanged.
__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ U, int64_t n, int64_t k0, int bs,
                                                        int32_t* __restrict__ info) {
    if (*info) return;
    __shared__ __attribute__((aligned(16))) float colb[2][16][8];
    __shared__ __attribute__((aligned(16))) float rowb[2][16][8];
    __shared__ float pivb[2];
    const int tid = threadIdx.x;
    const int tr = tid >> 4, tc = tid & 15;

    float a[8][8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int i = tr + 16 * ii, j = tc + 16 * jj;
            float v;
            if (i < bs && j < bs) v = i <= j ? U[(k0 + i) * n + k0 + j] : U[(k0 + j) * n + k0 + i];
            else v = i == j ? 1.f : 0.f;
            a[ii][jj] = v;
        }

    // ---- factor: for c = 127..0: V_cc = sqrt(a_cc); V_ic = a_ic / V_cc; a_ij -= V_ic V_jc (i, j < c)
#pragma unroll
    for (int jb = 7; jb >= 0; --jb) {
        for (int cr = 15; cr >= 0; --cr) {
            const int c = 16 * jb + cr;
            const int buf = c & 1;
            if (tc == cr) {                                   // owners of column c
                float t[8];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) t[ii] = (tr + 16 * ii < c) ? a[ii][jb] : 0.f;
                *(float4*)&colb[buf][tr][0] = make_float4(t[0], t[1], t[2], t[3]);
                *(float4*)&colb[buf][tr][4] = make_float4(t[4], t[5], t[6], t[7]);
                if (tr == cr) pivb[buf] = a[jb][jb];
            }
            __syncthreads();
            const float d = pivb[buf];
            if (!(d > 0.f)) {                                 // same value in every thread
                if (tid == 0) *info = (int32_t)(k0 + c + 1);
                return;
            }
            const float r = sqrtf(d);
            const float inv = 1.0f / r;
            const float inv2 = inv * inv;
            const float4 r0 = *(const float4*)&colb[buf][tr][0], r1 = *(const float4*)&colb[buf][tr][4];
            const float4 c0 = *(const float4*)&colb[buf][tc][0], c1 = *(const float4*)&colb[buf][tc][4];
            const float vr[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
            const float vc[8] = {c0.x * inv2, c0.y * inv2, c0.z * inv2, c0.w * inv2,
                                 c1.x * inv2, c1.y * inv2, c1.z * inv2, c1.w * inv2};
#pragma unroll
            for (int ii = 0; ii < 8; ++ii)
                if (tr + 16 * ii < c) {
#pragma unroll
                    for (int jj = 0; jj < jb + 1; ++jj) a[ii][jj] = fmaf(-vr[ii], vc[jj], a[ii][jj]);
                }
            if (tc == cr) {
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) {
                    const int i = tr + 16 * ii;
                    a[ii][jb] = i < c ? vr[ii] * inv : (i == c ? r : 0.f);
                }
            }
        }
    }

    // ---- inverse Z = V^-1 by rows from the bottom: with R = I initially, for i = 127..0:
    //      Z_i. = R_i. / V_ii and R_r. -= V_ri Z_i. = (V_ri / V_ii) R_i. for r < i
    float z[8][8];
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) z[ii][jj] = (tr + 16 * ii == tc + 16 * jj) ? 1.f : 0.f;

#pragma unroll
    for (int ib = 7; ib >= 0; --ib) {
        for (int ir = 15; ir >= 0; --ir) {
            const int i = 16 * ib + ir;
            const int buf = i & 1;
            if (tc == ir) {                                   // column i of V, rows < i
                float t[8];
#pragma unroll
                for (int ii = 0; ii < 8; ++ii) t[ii] = (tr + 16 * ii < i) ? a[ii][ib] : 0.f;
                *(float4*)&colb[buf][tr][0] = make_float4(t[0], t[1], t[2], t[3]);
                *(float4*)&colb[buf][tr][4] = make_float4(t[4], t[5], t[6], t[7]);
                if (tr == ir) pivb[buf] = a[ib][ib];
            }
            if (tr == ir) {                                   // row i of R (columns >= i)
                *(float4*)&rowb[buf][tc][0] = make_float4(z[ib][0], z[ib][1], z[ib][2], z[ib][3]);
                *(float4*)&rowb[buf][tc][4] = make_float4(z[ib][4], z[ib][5], z[ib][6], z[ib][7]);
            }
            __syncthreads();
            const float inv = 1.0f / pivb[buf];
            const float4 v0 = *(const float4*)&colb[buf][tr][0], v1 = *(const float4*)&colb[buf][tr][4];
            const float4 w0 = *(const float4*)&rowb[buf][tc][0], w1 = *(const float4*)&rowb[buf][tc][4];
            const float vr[8] = {v0.x * inv, v0.y * inv, v0.z * inv, v0.w * inv, v1.x * inv, v1.y * inv, v1.z * inv, v1.w * inv};
            const float rz[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int ii = 0; ii < 8; ++ii)
                if (tr + 16 * ii < i) {
#pragma unroll
                    for (int jj = ib; jj < 8; ++jj) z[ii][jj] = fmaf(-vr[ii], rz[jj], z[ii][jj]);
                }
            if (tr == ir) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) z[ib][jj] *= inv;
            }
        }
    }

#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int i = tr + 16 * ii, j = tc + 16 * jj;
            if (i < bs && j < bs) U[(k0 + i) * n + k0 + j] = j >= i ? z[ii][jj] : 0.f;
        }
}

// ------------------------------------------------------------------ epilogues
struct EpiStore {                 // out[row][col] = alpha * acc
    float* out;
    int64_t ld, M, N;
    float alpha;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row < M && col < N) out[row * ld + col] = alpha * v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

struct EpiSyrk {                  // A[row][col] -= acc on the upper triangle of the leading N x N
    float* U;
    int64_t ld, N;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row <= col && col < N) U[row * ld + col] -= v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

struct EpiPush {                  // R[row][col] (+)= acc; the first `fresh` columns are overwritten
    float* out;
    int64_t ld, M, N, fresh;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row < M && col < N) {
            float* p = out + row * ld + col;
            *p = col < fresh ? v : *p + v;
        }
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

RectMap rect(int bm, int bn, int64_t M, int64_t N, int64_t K) {
    RectMap m{};
    m.M = M; m.N = N; m.K = K;
    m.tiles_m = (int)cdiv(M, bm);
    m.tiles_n = (int)cdiv(N, bn);
    m.splits = 1;
    m.kchunk = cdiv(K, GEMM_BK) * GEMM_BK;
    m.tri_k = 0;
    m.guard = nullptr;
    return m;
}

inline int vec_ok(const float* p, int64_t ld) { return (ld % 4 == 0) && aligned(p, 16); }

typedef GemmTask<64, 64, OpMMajor<0>, OpMMajor<0>, RectMap, EpiStore> TrsmTask;
typedef GemmTask<128, 64, OpMMajor<0>, OpKMajor<0>, RectMap, EpiStore> FinalizeTask;
template <int T>
using SyrkTask = GemmTask<T, T, OpMMajor<0>, OpMMajor<0>, UpperMap, EpiSyrk>;
template <int T>
using PushTask = GemmTask<T, T, OpMMajor<0>, OpKMajor<0>, RectMap, EpiPush>;

int ntiles(const RectMap& m) { return m.tiles_m * m.tiles_n; }
int ntiles(const UpperMap& m) { return m.tiles * (m.tiles + 1) / 2; }

template <int T>
hipError_t launch_update(float* U, float* P, int64_t n, int64_t k0, int bs, int32_t* info, int vu, hipStream_t s) {
    SyrkTask<T> sy{};
    sy.la = OpMMajor<0>{P, CHOL_NB, k0, bs, 1};
    sy.lb = sy.la;
    sy.map = UpperMap{k0, bs, (int)cdiv(k0, T), 1, cdiv(bs, GEMM_BK) * GEMM_BK, nullptr};
    sy.epi = EpiSyrk{U, n, k0};
    PushTask<T> pu{};
    pu.la = OpMMajor<0>{P, CHOL_NB, k0, bs, 1};
    pu.lb = OpKMajor<0>{U + k0 * n + k0, n, n - k0, bs, vu && (k0 % 4 == 0)};
    pu.map = rect(T, T, k0, n - k0, bs);
    pu.epi = EpiPush{U + k0, n, k0, n - k0, bs};
    const int n1 = ntiles(sy.map), n2 = ntiles(pu.map);
    hipLaunchKernelGGL((gemm_f32_dual_kernel<SyrkTask<T>, PushTask<T>>), dim3(n1 + n2), dim3(GEMM_THREADS), 0, s, sy, pu, n1,
                       info);
    return hipGetLastError();
}

}  // namespace

size_t chol_ws_bytes(int64_t n) { return (size_t)n * CHOL_NB * sizeof(float); }

hipError_t chol_launch(const float* H, int64_t n, const int32_t* perm, float* U, int32_t* info, void* ws, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipError_t e;
    // a fill kernel, not a memset node, so the sequence can be captured in a graph
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, info, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (perm) hipLaunchKernelGGL(copy_perm_kernel, dim3((unsigned)n), dim3(256), 0, s, H, perm, U, n);
    else hipLaunchKernelGGL(copy_upper_kernel, dim3((unsigned)cdiv(n, 1024), (unsigned)n), dim3(256), 0, s, H, U, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    float* P = (float*)ws;     // n x CHOL_NB panel
    const int nt = (int)cdiv(n, CHOL_NB);
    const int vu = vec_ok(U, n);
    for (int kb = nt - 1; kb >= 0; --kb) {
        const int64_t k0 = (int64_t)kb * CHOL_NB;
        const int bs = (int)((n - k0) < CHOL_NB ? (n - k0) : CHOL_NB);
        const int64_t r = n - k0 - bs;
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, U, n, k0, bs, info);
        if ((e = hipGetLastError()) != hipSuccess) return e;

        // trsm (rows above) + finalize (block row k of U, right of the diagonal)
        TrsmTask tt{};
        tt.la = OpMMajor<0>{U + k0, n, k0, bs, vu && (k0 % 4 == 0)};
        tt.lb = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
        tt.map = rect(64, 64, k0, bs, bs);
        tt.epi = EpiStore{P, CHOL_NB, k0, bs, 1.f};
        FinalizeTask ft{};
        ft.la = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
        ft.lb = OpKMajor<0>{U + k0 * n + k0 + bs, n, r, bs, vu && ((k0 + bs) % 4 == 0)};
        ft.map = rect(128, 64, bs, r, bs);
        ft.epi = EpiStore{U + k0 * n + k0 + bs, n, bs, r, -1.f};
        const int n1 = k0 > 0 ? ntiles(tt.map) : 0;
        const int n2 = r > 0 ? ntiles(ft.map) : 0;
        if (n1 + n2 > 0) {
            hipLaunchKernelGGL((gemm_f32_dual_kernel<TrsmTask, FinalizeTask>), dim3(n1 + n2), dim3(GEMM_THREADS), 0, s, tt, ft,
                               n1, info);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (k0 == 0) break;
        // syrk (top-left, upper) + push (top-right R)
        const int64_t big = cdiv(k0, 128) * cdiv(n, 128);
        e = big >= 512 ? launch_update<128>(U, P, n, k0, bs, info, vu, s) : launch_update<64>(U, P, n, k0, bs, info, vu, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pwq
