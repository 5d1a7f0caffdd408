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
// trsm + finalize share one launch, syrk + push another: three launches per block.  Below
// n = 4096 the diagonal factor of block k - 1 joins block k's syrk + push launch: two
// launches per block, and the serial factor overlaps the update.  Block k's update of that
// diagonal block is then done ahead, in block k's trsm + finalize launch: ten workgroups,
// one per upper 32 x 32 tile, each forming the rows of P it needs from A and Z_kk.  From
// n = 4096 on, updates are batched per super-block, and the same overlap holds inside a
// super-block (the diagonal factor joins the launch of the products the super-block's later
// blocks need now); the first block past a super-block waits for its far products.
// Every kernel reads `info` first and does nothing once a pivot has failed.
#include "gemm_f32_dl.h"
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
// staged in LDS, so both the read and the write are coalesced.  One workgroup per row; each
// thread issues its loads (of the row, then of perm) in batches of four, so the workgroup
// waits for one memory latency per batch rather than per element.  The row's LDS allows one
// workgroup per CU, so it takes 16 waves, and 16-byte loads where rows are aligned, to keep
// enough bytes in flight to stream the row.
__global__ __launch_bounds__(1024) void copy_perm_kernel(const float* __restrict__ H, const int32_t* __restrict__ perm,
                                                         float* __restrict__ U, int64_t n) {
    __shared__ __attribute__((aligned(16))) float row[PERM_MAX_N];
    constexpr int NT = 1024, UR = 4;
    const int64_t i = blockIdx.x;
    const int tid = threadIdx.x;
    const float* src = H + (int64_t)perm[i] * n;
    if (n % 4 == 0 && ((uintptr_t)H & 15) == 0) {
        const int64_t nv = n / 4;
        for (int64_t j0 = 0; j0 < nv; j0 += NT * UR) {
            float4 v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + tid;
                v[u] = j < nv ? *(const float4*)(src + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + tid;
                if (j < nv) *(float4*)(row + 4 * j) = v[u];
            }
        }
    } else {
        for (int64_t j0 = 0; j0 < n; j0 += NT * UR) {
            float v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + tid;
                v[u] = j < n ? src[j] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + tid;
                if (j < n) row[j] = v[u];
            }
        }
    }
    __syncthreads();
    float* dst = U + i * n;
    for (int64_t j0 = 0; j0 < n; j0 += NT * UR) {
        int32_t pj[UR];
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = j0 + u * NT + tid;
            pj[u] = (j < n && j >= i) ? perm[j] : 0;
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = j0 + u * NT + tid;
            if (j < n) dst[j] = j >= i ? row[pj[u]] : 0.f;
        }
    }
}

// ------------------------------------------------------------------ diagonal block
// One workgroup of 256 threads factors the 128 x 128 diagonal block A = V V^T (V upper) and
// inverts V, everything in one 128 x 129 LDS matrix (66 KB, so that two workgroups of the
// update launch it shares fit on a CU):
//   factor, 32-column panels from the right: one wave holds the panel region (rows above
//     and inside the panel) in registers and runs its 32 pivots with readlane broadcasts;
//     after the panel, the rows and columns left of it get one rank-32 update on MFMA
//     (32 x 32 output tiles spread over the four waves).
//   inverse Z = V^-1, in place: each 32 x 32 diagonal block by one wave as soon as its panel
//     is done (no barriers: a wave's own LDS accesses are in order), most of the products
//     that join them on the waves the last two panels leave free; after the last panel,
//     the last leaf and one round of MFMA products.
// A ragged block (bs < 128) is padded with the identity, which leaves the real part unchanged.
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int LP = CHOL_NB + 1;    // padded LDS row

// Empty asm statements that fix where a value is computed: pin(x) needs x computed before
// it, pass(x) makes later uses of x wait for it.  Volatile asm keeps its order, so together
// they keep arithmetic from being moved past one another.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pass(float& x) { asm volatile("" : "+v"(x)); }

// v's value in lane l (l a constant), broadcast through an SGPR
__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// 32 x 32 tile of A B^T on MFMA: A rows [ra, ra+32) of the LDS matrix MA, B rows [rb, rb+32)
// of MB, k over [k0, k0 + kn) (kn even)
__device__ __forceinline__ f32x16 mfma_tile_abT2(const float (*MA)[LP], int ra, const float (*MB)[LP], int rb, int k0,
                                                 int kn, int lane) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll 4
    for (int kp = 0; kp < kn; kp += 2) {
        const float av = MA[ra + (lane & 31)][k0 + kp + (lane >> 5)];
        const float bv = MB[rb + (lane & 31)][k0 + kp + (lane >> 5)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    return acc;
}
// the same with both operands in one LDS matrix M
__device__ __forceinline__ f32x16 mfma_tile_abT(const float (*M)[LP], int ra, int rb, int k0, int kn, int lane) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    for (int kp = 0; kp < kn; kp += 2) {
        const float av = M[ra + (lane & 31)][k0 + kp + (lane >> 5)];
        const float bv = M[rb + (lane & 31)][k0 + kp + (lane >> 5)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    return acc;
}
// acc = A[ra.., ka + k] * B[kb + k][cb..], A from MA (row-major [i][k]), B from MB ([k][j])
__device__ __forceinline__ f32x16 mfma_tile_ab(const float (*MA)[LP], int ra, int ka, const float (*MB)[LP], int kb,
                                               int cb, int kn, int lane) {
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    for (int kp = 0; kp < kn; kp += 2) {
        const float av = MA[ra + (lane & 31)][ka + kp + (lane >> 5)];
        const float bv = MB[kb + kp + (lane >> 5)][cb + (lane & 31)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    return acc;
}
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

// Z = V^-1 of the 32 x 32 diagonal block o = 32 w, in place, by one wave: lane j owns column
// j of Z and back-substitutes it from the broadcast columns of V (no cross-lane traffic).
// Right-looking: once z_l is known, it leaves the pending sums s_i (i < l) as independent
// FMAs, so the dependent chain is two operations per row.  The block (zeros below its
// diagonal) is written over V's, which only this wave reads.
__device__ __forceinline__ void leaf_inverse(float (*A)[LP], int o, int lane) {
    const int j = lane & 31;
    float s[32], z[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) s[i] = i == j ? 1.f : 0.f;
#pragma unroll
    for (int l = 31; l >= 0; --l) {
        z[l] = s[l] * __builtin_amdgcn_rcpf(A[o + l][o + l]);
#pragma unroll
        for (int i = 0; i < l; ++i) s[i] = fmaf(-A[o + i][o + l], z[l], s[i]);
    }
    if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 32; ++i) A[o + i][o + j] = z[i];
    }
}

// 32 x 32 result of mfma_tile_ab stored at (r0, c0), times s
__device__ __forceinline__ void put_tile(float (*A)[LP], int r0, int c0, const f32x16& t, float s, int lane) {
#pragma unroll
    for (int v = 0; v < 16; ++v) A[r0 + acc_row(v, lane)][c0 + (lane & 31)] = s * t[v];
}

// Z = V^-1 of the 128 x 128 block, in place, in 32 x 32 blocks (V_ij, Z_ij; A = blocks 0-1,
// B = blocks 2-3), from the blocks inverted:
//   Z_23 = -Z_22 T23,  T23 = V_23 Z_33;     Z_01 = -Z_00 T01,  T01 = V_01 Z_11
//   Z_AB = -Z_AA T_AB, T_AB = V_AB Z_BB, so with W(tj) = T_AB(0, tj) - T01 T_AB(1, tj):
//   Z_AB(1, tj) = -Z_11 T_AB(1, tj),  Z_AB(0, tj) = -Z_00 W(tj).
// The intermediates live below the diagonal, where Z and V are zero and never stored:
// T_AB (then W) in rows 64.., columns ..63, T01 in rows 96.., columns 64..95 (after T_AB
// has been formed: T_AB(., 0) takes k over Z_22's rows only, so it never reads that zero
// block), T23 in rows 96.., columns 32..63 before T_AB(1, 1) goes there.  Z_22 and Z_33
// are inverted during panel 1's factor; during panel 0's, the waves it leaves free do this:
//   wave 1: Z_11, then T01;  wave 2: T23, Z_23, then T_AB(., 1);  wave 3: T_AB(., 0).
__device__ __forceinline__ void inverse_early(float (*A)[LP], int wave, int lane) {
    if (wave == 1) {
        leaf_inverse(A, 32, lane);
        put_tile(A, 96, 64, mfma_tile_ab(A, 0, 32, A, 32, 32, 32, lane), 1.f, lane);
    } else if (wave == 2) {
        put_tile(A, 96, 32, mfma_tile_ab(A, 64, 96, A, 96, 96, 32, lane), 1.f, lane);
        put_tile(A, 64, 96, mfma_tile_ab(A, 64, 64, A, 96, 32, 32, lane), -1.f, lane);
        const f32x16 t0 = mfma_tile_ab(A, 0, 64, A, 64, 96, 64, lane);
        const f32x16 t1 = mfma_tile_ab(A, 32, 64, A, 64, 96, 64, lane);
        put_tile(A, 64, 32, t0, 1.f, lane);
        put_tile(A, 96, 32, t1, 1.f, lane);
    } else if (wave == 3) {
        put_tile(A, 64, 0, mfma_tile_ab(A, 0, 64, A, 64, 64, 32, lane), 1.f, lane);
        put_tile(A, 96, 0, mfma_tile_ab(A, 32, 64, A, 64, 64, 32, lane), 1.f, lane);
    }
}

constexpr int DIAG_FLOATS = CHOL_NB * LP + 4;           // A (then Z in its place), the failed-pivot word

// The diagonal block [k0, k0 + bs) in one workgroup, in the LDS buffer smem (DIAG_FLOATS
// floats).
__device__ __forceinline__ void diag_block(float* __restrict__ U, int64_t n, int64_t k0, int bs,
                                           int32_t* __restrict__ info, float* smem) {
    float (*A)[LP] = (float (*)[LP])smem;
    int& fail = *(int*)(smem + CHOL_NB * LP);           // failed pivot + 1 of the current panel
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---------------- load: thread = (row, 64-column half), all loads in flight.  Below the
    // diagonal, U holds zeros (every writer of U keeps it so); nothing here reads those
    // entries as factors anyway: the panels carry them along as meaningless values and
    // write them back as zeros, the inverse reads only blocks on or above the diagonal.
    {
        const int i = tid >> 1, c0 = 64 * (tid & 1);
        const float* src = U + (k0 + i) * n + k0 + c0;
        float v[64];
        if (bs == CHOL_NB && (n % 4) == 0) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const float4 t = *(const float4*)(src + 4 * q);
                v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 64; ++q) {
                const int j = c0 + q;
                v[q] = (i < bs && j < bs) ? src[q] : (i == j ? 1.f : 0.f);
            }
        }
#pragma unroll
        for (int q = 0; q < 64; ++q) A[i][c0 + q] = v[q];
    }
    __syncthreads();

    // ---------------- factor: 32-column panels from the right.  The waves holding rows at or
    // above the panel's diagonal factor it in registers (32 rows each, plus a copy of the
    // panel's rows): the pivot and the pivot column's entries of the panel rows reach every
    // lane by readlane, so a pivot costs no LDS round trip and no barrier.  Entries below the diagonal pick up meaningless
    // values on the way (they only ever feed other entries below the diagonal) and are
    // written back as 0.  The panel's rank-32 update of the rows and columns left of it runs
    // on MFMA in two parts: the next panel's column block at once (all four waves), the rest
    // on the waves that hold no rows of that next panel while the others factor it.
    // unrolled over the four panels, so every readlane lane index is a constant.  A pivot's
    // broadcasts all go out before its FMAs (each into its own SGPR, fenced by a scheduling
    // barrier): interleaved, every FMA pair would wait out the latency of its own readlane.
    // Waves whose rows all lie below the panel's diagonal take no part in its factor.
#pragma unroll
    for (int p = 3; p >= 0; --p) {
        const int c0 = 32 * p;
        if (wave <= p) {
            // waves 0..p factor the panel together, each on its own 32 rows (lanes 0..31: row
            // 32 wave + lane) and a private copy of the panel's 32 rows (lanes 32..63: row
            // c0 + lane - 32), so every broadcast comes from its own lanes; all waves take the
            // same pivots
            const int row = lane < 32 ? 32 * wave + lane : c0 + lane - 32;
            float a[32];
#pragma unroll
            for (int kk = 0; kk < 32; ++kk) a[kk] = A[row][c0 + kk];
            int bad = -1;                                // first failed pivot (uniform)
            {
                const float d = lane_f(a[31], 63);
                if (!(d > 0.f)) bad = 31;
                a[31] *= __builtin_amdgcn_rsqf(d);       // column 31 of V (the pivot row gets d r)
            }
            __builtin_amdgcn_sched_barrier(0);
            // Pivot kk's column is scaled when its turn comes.  Its broadcasts go out first,
            // the next pivot's entry first; then the FMA into the next pivot's column, and the
            // next pivot's readlane, rsq and scaling are spread between this pivot's other FMAs,
            // so their latencies overlap them.  Scheduling barriers keep that order.
#pragma unroll
            for (int kk = 31; kk >= 0; --kk) {
                float vj[32];
#pragma unroll
                for (int jj = kk - 1; jj >= 0; --jj) vj[jj] = lane_f(a[kk], 32 + jj);
                __builtin_amdgcn_sched_barrier(0);
                if (kk > 0) {
                    constexpr int G = 3;                 // FMAs between the next pivot's steps
                    a[kk - 1] = fmaf(-a[kk], vj[kk - 1], a[kk - 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    const float dn = lane_f(a[kk - 1], 32 + kk - 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = kk - 2; jj >= 0 && jj > kk - 2 - G; --jj) {
                        a[jj] = fmaf(-a[kk], vj[jj], a[jj]);
                        pin(a[jj]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    bad = max(bad, dn > 0.f ? -1 : kk - 1);  // pivots run downwards: the first is the largest
                    float rn = __builtin_amdgcn_rsqf(dn);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = kk - 2 - G; jj >= 0 && jj > kk - 2 - 2 * G; --jj) {
                        a[jj] = fmaf(-a[kk], vj[jj], a[jj]);
                        pin(a[jj]);
                    }
                    pass(rn);
                    __builtin_amdgcn_sched_barrier(0);
                    a[kk - 1] *= rn;
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = kk - 2 - 2 * G; jj >= 0; --jj) a[jj] = fmaf(-a[kk], vj[jj], a[jj]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (lane < 32) {
#pragma unroll
                for (int kk = 0; kk < 32; ++kk) A[row][c0 + kk] = row <= c0 + kk ? a[kk] : 0.f;
            }
            if (wave == 0 && lane == 0) fail = bad >= 0 ? (int)(k0 + c0 + bad + 1) : 0;
        } else if (p < 3) {
            // the rest of panel p + 1's update (column blocks left of this panel), on the waves
            // p + 1 .. 3 while the others factor panel p: disjoint columns
            const int cp = 32 * (p + 1);
            const int nd = p * (p + 1) / 2;
            for (int t = wave - (p + 1); t < nd; t += 3 - p) {
                int ti = 0, r = t;
                while (r >= p - ti) { r -= p - ti; ++ti; }
                const int tj = ti + r;
                const f32x16 acc = mfma_tile_abT(A, 32 * ti, 32 * tj, cp, 32, lane);
#pragma unroll
                for (int v = 0; v < 16; ++v) A[32 * ti + acc_row(v, lane)][32 * tj + (lane & 31)] -= acc[v];
            }
            // the inverse, as far as the finished blocks allow (see below)
            if (p == 1) leaf_inverse(A, 32 * wave, lane);          // Z_22, Z_33
            if (p == 0) inverse_early(A, wave, lane);
        }
        __syncthreads();
        if (fail) {                                      // same decision in every thread
            if (tid == 0) *info = fail;
            return;
        }
        if (p > 0) {
            // A[0:c0, 0:c0] -= P P^T, P = V[0:c0, panel]: now only the next panel's column
            // block (its tiles (ti, p - 1)); the rest runs beside that panel's factor
            for (int t = wave; t < p; t += 4) {
                const f32x16 acc = mfma_tile_abT(A, 32 * t, 32 * (p - 1), c0, 32, lane);
#pragma unroll
                for (int v = 0; v < 16; ++v) A[32 * t + acc_row(v, lane)][32 * (p - 1) + (lane & 31)] -= acc[v];
            }
            __syncthreads();
        }
    }

    // ---------------- inverse, rest: Z_00 (wave 0); meanwhile, per column block tj of the
    // upper right (wave 3 - tj): Z_AB(1, tj) = -Z_11 T_AB(1, tj) and
    // W(tj) = T_AB(0, tj) - T01 T_AB(1, tj) over T_AB(0, tj); then everything left of Z's top
    // row block is -Z_00 [T01 | W(0) | W(1)].
    if (wave == 0) {
        leaf_inverse(A, 0, lane);
    } else if (wave >= 2) {
        const int tj = 3 - wave;
        put_tile(A, 32, 64 + 32 * tj, mfma_tile_ab(A, 32, 32, A, 96, 32 * tj, 32, lane), -1.f, lane);
        const f32x16 pr = mfma_tile_ab(A, 96, 64, A, 96, 32 * tj, 32, lane);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float& w = A[64 + acc_row(v, lane)][32 * tj + (lane & 31)];
            w = w - pr[v];
        }
    }
    __syncthreads();
    if (wave < 3) {
        // wave 0: Z_01 from T01 (rows 96.., columns 64..); waves 1, 2: Z_AB(0, wave - 1)
        const int sr = wave == 0 ? 96 : 64, sc = wave == 0 ? 64 : 32 * (wave - 1);
        put_tile(A, 0, 32 + 32 * wave, mfma_tile_ab(A, 0, 0, A, sr, sc, 32, lane), -1.f, lane);
    }
    __syncthreads();

    // ---------------- store: thread = (row, 64-column half).  Below the diagonal the block
    // holds zeros (leaves, and rows 32.. of columns ..31, never written) except in the
    // intermediates' places, rows 64.. of columns ..63 and rows 96.. of columns 64..95;
    // those are skipped (U keeps its zeros there), everything else is stored as it is.
    {
        const int i = tid >> 1, c0 = 64 * (tid & 1);
        float* dst = U + (k0 + i) * n + k0 + c0;
        if (bs == CHOL_NB && (n % 4) == 0) {
            const int q0 = c0 == 0 ? (i >= 64 ? 16 : 0) : (i >= 96 ? 8 : 0);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (q >= q0) {
                    const int j = c0 + 4 * q;
                    *(float4*)(dst + 4 * q) = make_float4(A[i][j], A[i][j + 1], A[i][j + 2], A[i][j + 3]);
                }
            }
        } else if (i < bs) {
            for (int q = 0; q < 64; ++q) {
                const int j = c0 + q;
                if (j < bs) dst[q] = j >= i ? A[i][j] : 0.f;
            }
        }
    }
}

__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ U, int64_t n, int64_t k0, int bs,
                                                        int32_t* __restrict__ info) {
    if (*info) return;
    __shared__ __attribute__((aligned(16))) float smem[DIAG_FLOATS];
    diag_block(U, n, k0, bs, info, smem);
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
    static constexpr bool kRmw = true, kFast = true;
    float* U;
    int64_t ld, N;
    __device__ __forceinline__ bool whole(const Tile& t, int bm, int bn) const {
        return t.m0 + bm - 1 <= t.n0 && t.n0 + bn <= N;
    }
    __device__ __forceinline__ float* at(int64_t row, int64_t col) const { return U + row * ld + col; }
    __device__ __forceinline__ float combine(float o, float v) const { return o - v; }
    __device__ __forceinline__ float old(const Tile&, int64_t row, int64_t col) const {
        return (row <= col && col < N) ? U[row * ld + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile&, int64_t row, int64_t col, float v, float o) {
        if (row <= col && col < N) U[row * ld + col] = o - v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

struct EpiSyrkRect {              // A[row][col0 + col] -= acc on the upper triangle (row <= col0 + col)
    static constexpr bool kRmw = true, kFast = true;
    float* U;                     // = A + col0
    int64_t ld, col0, N;
    __device__ __forceinline__ bool whole(const Tile& t, int bm, int bn) const {
        return t.m0 + bm - 1 <= col0 + t.n0 && t.n0 + bn <= N;
    }
    __device__ __forceinline__ float* at(int64_t row, int64_t col) const { return U + row * ld + col; }
    __device__ __forceinline__ float combine(float o, float v) const { return o - v; }
    __device__ __forceinline__ float old(const Tile&, int64_t row, int64_t col) const {
        return (row <= col0 + col && col < N) ? U[row * ld + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile&, int64_t row, int64_t col, float v, float o) {
        if (row <= col0 + col && col < N) U[row * ld + col] = o - v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

struct EpiPush {                  // R[row][col] (+)= acc; the first `fresh` columns are overwritten
    static constexpr bool kRmw = true, kFast = true;
    float* out;
    int64_t ld, M, N, fresh;
    __device__ __forceinline__ bool whole(const Tile& t, int bm, int bn) const {
        return t.m0 + bm <= M && t.n0 + bn <= N && t.n0 >= fresh;
    }
    __device__ __forceinline__ float* at(int64_t row, int64_t col) const { return out + row * ld + col; }
    __device__ __forceinline__ float combine(float o, float v) const { return o + v; }
    __device__ __forceinline__ float old(const Tile&, int64_t row, int64_t col) const {
        return (row < M && col < N && col >= fresh) ? out[row * ld + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile&, int64_t row, int64_t col, float v, float o) {
        if (row < M && col < N) out[row * ld + col] = col < fresh ? v : o + v;
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
typedef GemmTask<64, 64, OpMMajor<0>, OpKMajor<0>, RectMap, EpiStore> FinalizeTask;   // short k: all loads up front
template <int T>
using SyrkTask = GemmTask<T, T, OpMMajor<0>, OpMMajor<0>, UpperMap, EpiSyrk>;
template <int T>
using PushTask = GemmTask<T, T, OpMMajor<0>, OpKMajor<0>, RectMap, EpiPush>;
template <int T>
using SyrkRectTask = GemmTask<T, T, OpMMajor<0>, OpMMajor<0>, RectMap, EpiSyrkRect>;

// A rectangular grid without the tiles at or past (m_from, n_from) in both directions (the
// next diagonal block, updated ahead by the trsm launch); their workgroups do nothing
struct SkipRectMap {
    RectMap r;
    int64_t m_from, n_from;
    __device__ __forceinline__ bool get(int bid, int BM, int BN, Tile& t) const {
        if (!r.get(bid, BM, BN, t)) return false;
        if (t.m0 >= m_from && t.n0 >= n_from) {
            t.kend = t.kbeg;
            return false;
        }
        return true;
    }
};
template <int T>
using SyrkRectSkipTask = GemmTask<T, T, OpMMajor<0>, OpMMajor<0>, SkipRectMap, EpiSyrkRect>;

int ntiles(const RectMap& m) { return m.tiles_m * m.tiles_n; }
int ntiles(const SkipRectMap& m) { return ntiles(m.r); }
int ntiles(const UpperMap& m) { return m.tiles * (m.tiles + 1) / 2; }

// Panels of a super-block: P holds the V columns of its chol_sb(n) blocks side by side (row
// stride pld = chol_sb(n) * CHOL_NB, the workspace's width); block slot t at column t * CHOL_NB.
constexpr int CHOL_SB = 8;
// 256-tile rows x columns of the whole trailing matrix from which the direct-load engine takes
// a far update (its tiles are four times as large, so fewer of them must still fill the chip)
constexpr int64_t FAR_DL_MIN_TILES = 1024;
constexpr int64_t CHOL_LAZY_N = 4096;            // batch the updates from this size on
inline int chol_sb(int64_t n) { return n >= CHOL_LAZY_N ? CHOL_SB : 1; }

// After the last block of a super-block [s0, s1) (depth kf = s1 - s0 of panels in P):
//   A[0:s0, 0:s0] -= P P^T           (upper triangle; P = V[0:s0, s0:s1])
//   R[0:s0, s0:n] (+)= P U[s0:s1, s0:n]   (columns s0..s1 overwritten: they held A)
template <int T>
hipError_t launch_far(float* U, const float* P, int pld, int64_t n, int64_t s0, int kf, int32_t* info, int vu,
                      hipStream_t s) {
    SyrkTask<T> sy{};
    sy.la = OpMMajor<0>{P, pld, s0, kf, 1};
    sy.lb = sy.la;
    sy.map = UpperMap{s0, kf, (int)cdiv(s0, T), 1, cdiv(kf, GEMM_BK) * GEMM_BK, nullptr};
    sy.epi = EpiSyrk{U, n, s0};
    PushTask<T> pu{};
    pu.la = OpMMajor<0>{P, pld, s0, kf, 1};
    pu.lb = OpKMajor<0>{U + s0 * n + s0, n, n - s0, kf, vu && (s0 % 4 == 0)};
    pu.map = rect(T, T, s0, n - s0, kf);
    pu.epi = EpiPush{U + s0, n, s0, n - s0, kf};
    const int n1 = ntiles(sy.map), n2 = ntiles(pu.map);
    hipLaunchKernelGGL((gemm_f32_dual_kernel<SyrkTask<T>, PushTask<T>>), dim3(n1 + n2), dim3(GEMM_THREADS), 0, s, sy, pu, n1,
                       info);
    return hipGetLastError();
}

// launch_far on the direct-load engine (T x T tiles): the same two products, for super-blocks
// a whole number of its stages deep, every row 16-byte aligned
template <int T>
using SyrkDlTask = FdlTask<FdlRows<T>, FdlRows<T>, UpperMap, EpiSyrk>;
template <int T>
using PushDlTask = FdlTask<FdlRows<T>, FdlCols<T>, RectMap, EpiPush>;

// rows of the panels and of U 16-byte aligned, depth whole stages: the direct-load engines apply
inline bool dl_ok(int64_t n, int depth, int pld, int vu) {
    return vu && n % 4 == 0 && pld % 4 == 0 && depth % FDL_BK == 0;
}

template <int T>
hipError_t launch_far_dl(float* U, const float* P, int pld, int64_t n, int64_t s0, int kf, int32_t* info, hipStream_t s) {
    SyrkDlTask<T> sy{};
    sy.la = FdlRows<T>{P, pld, s0};
    sy.lb = sy.la;
    sy.map = UpperMap{s0, kf, (int)cdiv(s0, T), 1, kf, nullptr};
    sy.epi = EpiSyrk{U, n, s0};
    PushDlTask<T> pu{};
    pu.la = FdlRows<T>{P, pld, s0};
    pu.lb = FdlCols<T>{U + s0 * n + s0, n, n - s0};
    pu.map = rect(T, T, s0, n - s0, kf);
    pu.epi = EpiPush{U + s0, n, s0, n - s0, kf};
    const int n1 = ntiles(sy.map), n2 = ntiles(pu.map);
    hipLaunchKernelGGL((gemm_fdl_dual_kernel<SyrkDlTask<T>, PushDlTask<T>>), dim3(n1 + n2), dim3(GEMM_THREADS), 0, s, sy,
                       pu, n1, info);
    return hipGetLastError();
}

// launch_far with its products on bfloat16 MFMA (the 256-tile register-staged engine): P and
// the rows U[s0:s0+kf, s0:n] are cut into their three-piece splits (split3_tiled_block), and
// each float32 product is the sum of the six larger piece products.  The dropped three are
// below 2^-23 of |a| |b| each, so every product term is as accurate as a float32 product,
// and the sums run on the bfloat16 pipe (eight times the float32 rate, six products per term).
// pcs: 3 (panel-padded s0 + panel-padded (n - s0)) kseg bfloat16 values, kseg = kf rounded up
// to 64.
template <bool KMAJ>
__global__ __launch_bounds__(256) void chol_split3_kernel(const float* __restrict__ src, int64_t ld, int64_t M, int64_t K,
                                                          uint16_t* __restrict__ out, int64_t kseg, int64_t pstride) {
    split3_tiled_block<KMAJ>(src, ld, M, K, out, kseg, pstride);
}

using SyrkSplitTask = RsTask<2, DlTiled6, DlTiled6, UpperMap, EpiSyrk>;
using PushSplitTask = RsTask<2, DlTiled6, DlTiled6, XcdRectMap, EpiPush>;

hipError_t launch_far_split(float* U, const float* P, int pld, int64_t n, int64_t s0, int kf, int32_t* info,
                            uint16_t* pcs, hipStream_t s) {
    const int64_t kseg = cdiv(kf, 64) * 64;
    const int64_t ma = dl_panel_pad(s0), mb = dl_panel_pad(n - s0);
    uint16_t* A = pcs;                                   // pieces of P[0:s0, 0:kf]
    uint16_t* B = pcs + 3 * ma * kseg;                   // pieces of U[s0:s0+kf, s0:n]^T
    hipLaunchKernelGGL(chol_split3_kernel<false>, dim3((unsigned)(ma / 64), (unsigned)(kseg / 64)), dim3(256), 0, s, P,
                       (int64_t)pld, s0, (int64_t)kf, A, kseg, ma * kseg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chol_split3_kernel<true>, dim3((unsigned)(mb / 64), (unsigned)(kseg / 64)), dim3(256), 0, s,
                       (const float*)(U + s0 * n + s0), n, n - s0, (int64_t)kf, B, kseg, mb * kseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const uint16_t* A1 = A;
    const uint16_t* A2 = A + ma * kseg;
    const uint16_t* A3 = A + 2 * ma * kseg;
    const uint16_t* B1 = B;
    const uint16_t* B2 = B + mb * kseg;
    const uint16_t* B3 = B + 2 * mb * kseg;
    // (i, j) of the segments: (3,1), (1,3), (2,2), (2,1), (1,2), (1,1)
    const DlTiled6 pa{{A3, A1, A2, A2, A1, A1}, kseg};
    SyrkSplitTask sy{};
    sy.la = pa;
    sy.lb = DlTiled6{{A1, A3, A2, A1, A2, A1}, kseg};
    // both tile sets in the per-XCD band order (each XCD's workgroups share operand panels)
    sy.map = UpperMap{s0, 6 * kseg, (int)cdiv(s0, DL_TILE), 1, 6 * kseg, nullptr, 0, 1};
    sy.epi = EpiSyrk{U, n, s0};
    PushSplitTask pu{};
    pu.la = pa;
    pu.lb = DlTiled6{{B1, B3, B2, B1, B2, B1}, kseg};
    pu.map = XcdRectMap{s0, n - s0, 6 * kseg, (int)cdiv(s0, DL_TILE), (int)cdiv(n - s0, DL_TILE), nullptr};
    pu.epi = EpiPush{U + s0, n, s0, n - s0, kf};
    // n1 a multiple of 8, so the push's workgroups keep their XCD numbering
    const int n1 = xcd_grid(ntiles(sy.map)), n2 = xcd_grid(pu.map.tiles_m * pu.map.tiles_n);
    hipLaunchKernelGGL((gemm_rs_dual_kernel<SyrkSplitTask, PushSplitTask>), dim3(n1 + n2), dim3(GEMM_THREADS), 0, s, sy, pu,
                       n1, (const int32_t*)info);
    return hipGetLastError();
}

// One launch for the update of block k (syrk + push tiles, workgroups 1 ..) and the
// factor of the next diagonal block [kd0, kd0 + NB) (workgroup 0): block k's update of that
// block was applied by block k's trsm launch (pre_update_tile), and the syrk tiles covering
// it are left out of this grid, so the serial diagonal factor overlaps the rest of the update.
template <class TA, class TB>
__global__ __launch_bounds__(GEMM_THREADS, 2) void chol_update_diag_kernel(TA a, TB b, int n1, int32_t* __restrict__ info,
                                                                        float* __restrict__ U, int64_t n, int64_t kd0) {
    if (*info) return;
    constexpr int L0 = TA::LDS > TB::LDS ? TA::LDS : TB::LDS;
    constexpr int L = L0 > DIAG_FLOATS ? L0 : DIAG_FLOATS;
    __shared__ __attribute__((aligned(16))) float lds[L];
    const int bid = (int)blockIdx.x;
    if (bid == 0) diag_block(U, n, kd0, CHOL_NB, info, lds);
    else if (bid - 1 < n1) a.run(bid - 1, lds);
    else b.run(bid - 1 - n1, lds);
}

// After block [k0, k0 + bs) of a super-block starting at s0 < k0, for the blocks of the
// super-block still to come (its panel Pk = V[0:k0, block] in P):
//   A[0:k0, s0:k0] -= Pk Pk[s0:k0]^T       (their columns, every row above)
//   R[s0:k0, k0:n] (+)= Pk[s0:k0] U[block, k0:n]   (their rows; columns k0..k0+bs overwritten)
// together with the factor of the next diagonal block [k0 - NB, k0): block k's trsm launch
// has already applied block k's update to that block, so its syrk tiles are left out and
// workgroup 0 factors it while the other tiles run
template <int T>
hipError_t launch_near_diag(float* U, const float* Pk, int pld, int64_t n, int64_t s0, int64_t k0, int bs,
                            int32_t* info, int vu, hipStream_t s) {
    const int64_t k1 = k0 - CHOL_NB;
    SyrkRectSkipTask<T> sy{};
    sy.la = OpMMajor<0>{Pk, pld, k0, bs, 1};
    sy.lb = OpMMajor<0>{Pk + s0 * pld, pld, k0 - s0, bs, 1};
    sy.map = SkipRectMap{rect(T, T, k0, k0 - s0, bs), k1, k1 - s0};
    sy.epi = EpiSyrkRect{U + s0, n, s0, k0 - s0};
    PushTask<T> pu{};
    pu.la = OpMMajor<0>{Pk + s0 * pld, pld, k0 - s0, bs, 1};
    pu.lb = OpKMajor<0>{U + k0 * n + k0, n, n - k0, bs, vu && (k0 % 4 == 0)};
    pu.map = rect(T, T, k0 - s0, n - k0, bs);
    pu.epi = EpiPush{U + s0 * n + k0, n, k0 - s0, n - k0, bs};
    const int n1 = ntiles(sy.map), n2 = ntiles(pu.map);
    hipLaunchKernelGGL((chol_update_diag_kernel<SyrkRectSkipTask<T>, PushTask<T>>), dim3(1 + n1 + n2),
                       dim3(GEMM_THREADS), 0, s, sy, pu, n1, info, U, n, k1);
    return hipGetLastError();
}

// launch_near_diag on the direct-load engine (T x T tiles, two workgroups per CU at T = 128)
template <int T>
using SyrkRectSkipDlTask = FdlTask<FdlRows<T>, FdlRows<T>, SkipRectMap, EpiSyrkRect>;

template <int T>
hipError_t launch_near_diag_dl(float* U, const float* Pk, int pld, int64_t n, int64_t s0, int64_t k0, int bs,
                               int32_t* info, hipStream_t s) {
    const int64_t k1 = k0 - CHOL_NB;
    SyrkRectSkipDlTask<T> sy{};
    sy.la = FdlRows<T>{Pk, pld, k0};
    sy.lb = FdlRows<T>{Pk + s0 * pld, pld, k0 - s0};
    sy.map = SkipRectMap{rect(T, T, k0, k0 - s0, bs), k1, k1 - s0};
    sy.epi = EpiSyrkRect{U + s0, n, s0, k0 - s0};
    PushDlTask<T> pu{};
    pu.la = FdlRows<T>{Pk + s0 * pld, pld, k0 - s0};
    pu.lb = FdlCols<T>{U + k0 * n + k0, n, n - k0};
    pu.map = rect(T, T, k0 - s0, n - k0, bs);
    pu.epi = EpiPush{U + s0 * n + k0, n, k0 - s0, n - k0, bs};
    const int n1 = ntiles(sy.map), n2 = ntiles(pu.map);
    hipLaunchKernelGGL((chol_update_diag_kernel<SyrkRectSkipDlTask<T>, PushDlTask<T>>), dim3(1 + n1 + n2),
                       dim3(GEMM_THREADS), 0, s, sy, pu, n1, info, U, n, k1);
    return hipGetLastError();
}

// Block k's update of the next diagonal block D = A[k1:k0, k1:k0] (k1 = k0 - NB), done in
// block k's trsm launch: D -= P_D P_D^T with P_D = A[k1:k0, k0:k0+bs] Z_kk^T, the rows of
// block k's panel P that fall in D.  Workgroup t takes the upper 32 x 32 tile (ti, tj) of D
// and forms the two 32-row slices of P_D it needs itself (one on the diagonal), from A and
// Z_kk (upper triangular: column block cb of P takes k from 32 cb on).  Nothing else in
// the launch reads or writes D.
constexpr int PRE_TILES = 10;
constexpr int PP = CHOL_NB + 4;                        // LDS pitch: rows 16-byte aligned
constexpr int PRE_FLOATS = CHOL_NB * PP + 64 * PP;     // Z_kk, two 32-row slices

// 32 x 32 tile of A B^T: A rows [ra, ra+32) of MA, B rows [rb, rb+32) of MB, k over
// [k0, k0 + KN).  Both operands take the k values in the same order: in step s, lane half
// h supplies k0 + 8 s + 4 h + i to MFMA i, so each lane reads its four with one 16-byte load.
template <int KN>
__device__ __forceinline__ f32x16 mfma_abT_x4(const float (*MA)[PP], int ra, const float (*MB)[PP], int rb, int k0,
                                              int lane) {
    static_assert(KN % 8 == 0, "k in steps of 8");
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;
    const int r = lane & 31, kh = k0 + 4 * (lane >> 5);
#pragma unroll
    for (int st = 0; st < KN / 8; ++st) {
        const float4 a = *(const float4*)&MA[ra + r][kh + 8 * st];
        const float4 b = *(const float4*)&MB[rb + r][kh + 8 * st];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
    }
    return acc;
}

// column block cb of a P slice: k over [32 cb, NB)
__device__ __forceinline__ f32x16 p_block(const float (*As)[PP], int ra, const float (*Zs)[PP], int cb, int lane) {
    switch (cb) {
        case 0: return mfma_abT_x4<CHOL_NB>(As, ra, Zs, 0, 0, lane);
        case 1: return mfma_abT_x4<CHOL_NB - 32>(As, ra, Zs, 32, 32, lane);
        case 2: return mfma_abT_x4<CHOL_NB - 64>(As, ra, Zs, 64, 64, lane);
        default: return mfma_abT_x4<CHOL_NB - 96>(As, ra, Zs, 96, 96, lane);
    }
}

__device__ __forceinline__ void pre_update_tile(float* __restrict__ U, int64_t n, int64_t k0, int bs, int t,
                                                float* smem) {
    float (*Zs)[PP] = (float (*)[PP])smem;
    float (*As)[PP] = (float (*)[PP])(smem + CHOL_NB * PP);   // slice of tile row ti, then of tj
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int ti = 0, r = t;
    while (r >= 4 - ti) { r -= 4 - ti; ++ti; }
    const int tj = ti + r;
    const bool diag = ti == tj;
    const int64_t k1 = k0 - CHOL_NB;
    const bool vec = bs == CHOL_NB && (n % 4) == 0 && ((uintptr_t)U & 15) == 0;
    // this thread's four elements of D's tile, read now (nothing in the launch writes them)
    const int dr = tid >> 3, dc = 4 * (tid & 7);
    float* dst = U + (k1 + 32 * ti + dr) * n + k1 + 32 * tj + dc;
    float dold[4];

    // ---------------- load: Z_kk (upper, zero past bs), the slices' columns [k0, k0 + bs), D's tile
    {
        const int i = tid >> 1, c0 = 64 * (tid & 1);
        const float* src = U + (k0 + i) * n + k0 + c0;
        float4 v[16];
        const int ns = diag ? 1 : 2;
        const int rr = tid >> 3, a0 = 16 * (tid & 7);
        float4 w[2][4];
        if (vec) {
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = *(const float4*)(src + 4 * q);
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                if (sl < ns) {
                    const float* a = U + (k1 + 32 * (sl ? tj : ti) + rr) * n + k0 + a0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[sl][q] = *(const float4*)(a + 4 * q);
                }
            }
            const float4 d = *(const float4*)dst;
            dold[0] = d.x; dold[1] = d.y; dold[2] = d.z; dold[3] = d.w;
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                float e[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) e[c] = (i < bs && c0 + 4 * q + c < bs) ? src[4 * q + c] : 0.f;
                v[q] = make_float4(e[0], e[1], e[2], e[3]);
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                if (sl < ns) {
                    const float* a = U + (k1 + 32 * (sl ? tj : ti) + rr) * n + k0 + a0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float e[4];
#pragma unroll
                        for (int c = 0; c < 4; ++c) e[c] = a0 + 4 * q + c < bs ? a[4 * q + c] : 0.f;
                        w[sl][q] = make_float4(e[0], e[1], e[2], e[3]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) dold[q] = dst[q];
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int j = c0 + 4 * q;
            float4 x = v[q];
            if (j < i) x.x = 0.f;
            if (j + 1 < i) x.y = 0.f;
            if (j + 2 < i) x.z = 0.f;
            if (j + 3 < i) x.w = 0.f;
            *(float4*)&Zs[i][j] = x;
        }
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            if (sl < ns) {
#pragma unroll
                for (int q = 0; q < 4; ++q) *(float4*)&As[32 * sl + rr][a0 + 4 * q] = w[sl][q];
            }
        }
    }
    __syncthreads();

    // ---------------- P slices on MFMA: job (slice, column block), balanced over the waves
    // (80 MFMAs each off the diagonal: column blocks 0 + 3 and 1 + 2 of a slice)
    int js0, jc0, js1, jc1;
    if (diag) { js0 = 0; jc0 = wave; js1 = -1; jc1 = 0; }
    else { js0 = js1 = wave & 1; jc0 = wave < 2 ? 0 : 1; jc1 = wave < 2 ? 3 : 2; }
    const f32x16 p0 = p_block(As, 32 * js0, Zs, jc0, lane);
    f32x16 p1;
    if (js1 >= 0) p1 = p_block(As, 32 * js1, Zs, jc1, lane);
    __syncthreads();                                   // every read of As and Zs done
#pragma unroll
    for (int v = 0; v < 16; ++v) As[32 * js0 + acc_row(v, lane)][32 * jc0 + (lane & 31)] = p0[v];
    if (js1 >= 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) As[32 * js1 + acc_row(v, lane)][32 * jc1 + (lane & 31)] = p1[v];
    }
    __syncthreads();

    // ---------------- C = P_ti P_tj^T, k split over the waves (32 each); the four partial
    // tiles (in Z's place) are summed in a fixed order, and D's tile takes -C (upper part
    // on the diagonal)
    const f32x16 c = mfma_abT_x4<32>(As, 0, As, diag ? 0 : 32, 32 * wave, lane);
    float (*Cp)[33] = (float (*)[33])smem;
#pragma unroll
    for (int v = 0; v < 16; ++v) Cp[32 * wave + acc_row(v, lane)][lane & 31] = c[v];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int cc = dc + q;
        const float sum = ((Cp[dr][cc] + Cp[32 + dr][cc]) + Cp[64 + dr][cc]) + Cp[96 + dr][cc];
        if (!diag || cc >= dr) dst[q] = dold[q] - sum;
    }
}

// Block k's trsm + finalize launch: workgroups [0, n0) update the next diagonal block
// (pre_update_tile; n0 = 0 for the last block), then n1 trsm tiles, then finalize tiles.
template <class TA, class TB>
__global__ __launch_bounds__(GEMM_THREADS) void chol_panel_kernel(TA a, TB b, int n0, int n1,
                                                                  const int32_t* __restrict__ info,
                                                                  float* __restrict__ U, int64_t n, int64_t k0, int bs) {
    if (*info) return;
    constexpr int L0 = TA::LDS > TB::LDS ? TA::LDS : TB::LDS;
    constexpr int L = L0 > PRE_FLOATS ? L0 : PRE_FLOATS;
    __shared__ __attribute__((aligned(16))) float lds[L];
    const int bid = (int)blockIdx.x;
    if (bid < n0) pre_update_tile(U, n, k0, bs, bid, lds);
    else if (bid - n0 < n1) a.run(bid - n0, lds);
    else b.run(bid - n0 - n1, lds);
}

// syrk + push of block [k0, k0 + bs) (no super-blocks: depth bs, panel P = V[0:k0, block])
// together with the factor of the diagonal block [k0 - NB, k0)
template <int T>
hipError_t launch_update_diag(float* U, const float* P, int pld, int64_t n, int64_t k0, int bs, int32_t* info, int vu,
                              hipStream_t s) {
    SyrkTask<T> sy{};
    sy.la = OpMMajor<0>{P, pld, k0, bs, 1};
    sy.lb = sy.la;
    sy.map = UpperMap{k0, bs, (int)cdiv(k0, T), 1, cdiv(bs, GEMM_BK) * GEMM_BK, nullptr};
    sy.epi = EpiSyrk{U, n, k0};
    PushTask<T> pu{};
    pu.la = OpMMajor<0>{P, pld, k0, bs, 1};
    pu.lb = OpKMajor<0>{U + k0 * n + k0, n, n - k0, bs, vu && (k0 % 4 == 0)};
    pu.map = rect(T, T, k0, n - k0, bs);
    pu.epi = EpiPush{U + k0, n, k0, n - k0, bs};
    // the last upper tiles in map order are the ones inside [k0 - NB, k0)^2: one of 128, three of 64
    const int n1 = ntiles(sy.map) - (T == 128 ? 1 : 3);
    const int n2 = ntiles(pu.map);
    hipLaunchKernelGGL((chol_update_diag_kernel<SyrkTask<T>, PushTask<T>>), dim3(1 + n1 + n2), dim3(GEMM_THREADS), 0, s,
                       sy, pu, n1, info, U, n, k0 - CHOL_NB);
    return hipGetLastError();
}

// 64 x 64 tiles of a block's trsm and finalize above which they take 128 x 128 tiles
constexpr int64_t PANEL64_MAX_TILES = 256;

// block k's trsm (rows above, into its panel slot Pk) + finalize (block row k right of the
// diagonal), with block k's update of the next diagonal block in workgroups [0, PRE_TILES)
// when `fuse`, on T x T tiles
template <int T>
hipError_t launch_panel(float* U, float* Pk, int pld, int64_t n, int64_t k0, int bs, int64_t r, bool fuse, int vu,
                        int32_t* info, hipStream_t s) {
    GemmTask<T, T, OpMMajor<0>, OpMMajor<0>, RectMap, EpiStore> tt{};
    tt.la = OpMMajor<0>{U + k0, n, k0, bs, vu && (k0 % 4 == 0)};
    tt.lb = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
    tt.map = rect(T, T, k0, bs, bs);
    tt.epi = EpiStore{Pk, pld, k0, bs, 1.f};
    GemmTask<T, T, OpMMajor<0>, OpKMajor<0>, RectMap, EpiStore> ft{};
    ft.la = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
    ft.lb = OpKMajor<0>{U + k0 * n + k0 + bs, n, r, bs, vu && ((k0 + bs) % 4 == 0)};
    ft.map = rect(T, T, bs, r, bs);
    ft.epi = EpiStore{U + k0 * n + k0 + bs, n, bs, r, -1.f};
    const int n0 = fuse ? PRE_TILES : 0;
    const int n1 = k0 > 0 ? ntiles(tt.map) : 0;
    const int n2 = r > 0 ? ntiles(ft.map) : 0;
    if (n0 + n1 + n2 == 0) return hipSuccess;
    hipLaunchKernelGGL((chol_panel_kernel<decltype(tt), decltype(ft)>), dim3(n0 + n1 + n2), dim3(GEMM_THREADS), 0, s, tt,
                       ft, n0, n1, info, U, n, k0, bs);
    return hipGetLastError();
}

}  // namespace

// far products of 256-tile size take the split route (launch_far_split) once the trailing
// matrix holds FAR_DL_MIN_TILES of those tiles
inline bool far_split(int64_t n, int64_t s0) { return cdiv(s0, DL_TILE) * cdiv(n, DL_TILE) >= FAR_DL_MIN_TILES; }
// (the largest far product is the one after the last super-block, which starts at the last
// multiple of CHOL_SB * CHOL_NB below n)
inline bool far_split_possible(int64_t n) {
    constexpr int64_t w = CHOL_SB * CHOL_NB;
    return chol_sb(n) > 1 && far_split(n, (n - 1) / w * w);
}

// the super-block panels P, then (when the split route can run) its pieces
size_t chol_ws_bytes(int64_t n) {
    const size_t panels = (size_t)n * (chol_sb(n) * CHOL_NB) * sizeof(float);
    if (!far_split_possible(n)) return panels;
    return panels + (size_t)3 * (size_t)(dl_panel_pad(n) + DL_TILE) * (size_t)(CHOL_SB * CHOL_NB) * sizeof(uint16_t);
}

hipError_t chol_launch(const float* H, int64_t n, const int32_t* perm, float* U, int32_t* info, void* ws, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipError_t e;
    // a fill kernel, not a memset node, so the sequence can be captured in a graph
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, s, info, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (perm) hipLaunchKernelGGL(copy_perm_kernel, dim3((unsigned)n), dim3(1024), 0, s, H, perm, U, n);
    else hipLaunchKernelGGL(copy_upper_kernel, dim3((unsigned)cdiv(n, 1024), (unsigned)n), dim3(256), 0, s, H, U, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // Blocks of CHOL_NB columns from the last to the first, in super-blocks of chol_sb(n)
    // blocks aligned to their size: the updates a block owes to the matrix above and left of
    // its super-block wait until the super-block is done, and then go as one deeper product.
    float* P = (float*)ws;     // n x pld: the super-block's V panels
    uint16_t* pcs = (uint16_t*)(P + n * (int64_t)(chol_sb(n) * CHOL_NB));   // their split pieces (far_split_possible)
    const int nt = (int)cdiv(n, CHOL_NB);
    const int sb = chol_sb(n);
    const int pld = sb * CHOL_NB;
    const int vu = vec_ok(U, n);
    if (sb == 1) {
        // two launches per block: trsm + finalize of block k (with its update of the diagonal
        // block k - 1), then its syrk + push together with the factor of block k - 1
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, U, n, (int64_t)(nt - 1) * CHOL_NB,
                           (int)(n - (int64_t)(nt - 1) * CHOL_NB), info);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        for (int kb = nt - 1; kb >= 0; --kb) {
            const int64_t k0 = (int64_t)kb * CHOL_NB;
            const int bs = (int)((n - k0) < CHOL_NB ? (n - k0) : CHOL_NB);
            const int64_t r = n - k0 - bs;
            TrsmTask tt{};
            tt.la = OpMMajor<0>{U + k0, n, k0, bs, vu && (k0 % 4 == 0)};
            tt.lb = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
            tt.map = rect(64, 64, k0, bs, bs);
            tt.epi = EpiStore{P, pld, k0, bs, 1.f};
            FinalizeTask ft{};
            ft.la = OpMMajor<0>{U + k0 * n + k0, n, bs, bs, vu && (k0 % 4 == 0)};
            ft.lb = OpKMajor<0>{U + k0 * n + k0 + bs, n, r, bs, vu && ((k0 + bs) % 4 == 0)};
            ft.map = rect(64, 64, bs, r, bs);
            ft.epi = EpiStore{U + k0 * n + k0 + bs, n, bs, r, -1.f};
            const int n0 = k0 > 0 ? PRE_TILES : 0;
            const int n1 = k0 > 0 ? ntiles(tt.map) : 0;
            const int n2 = r > 0 ? ntiles(ft.map) : 0;
            if (n0 + n1 + n2 > 0) {
                hipLaunchKernelGGL((chol_panel_kernel<TrsmTask, FinalizeTask>), dim3(n0 + n1 + n2), dim3(GEMM_THREADS), 0, s,
                                   tt, ft, n0, n1, info, U, n, k0, bs);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            if (k0 == 0) break;
            const int64_t big = cdiv(k0, 128) * cdiv(n, 128);
            e = big >= 512 ? launch_update_diag<128>(U, P, pld, n, k0, bs, info, vu, s)
                           : launch_update_diag<64>(U, P, pld, n, k0, bs, info, vu, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    bool diag_done = false;                              // this block's diagonal factor already launched
    for (int kb = nt - 1; kb >= 0; --kb) {
        const int64_t k0 = (int64_t)kb * CHOL_NB;
        const int bs = (int)((n - k0) < CHOL_NB ? (n - k0) : CHOL_NB);
        const int64_t r = n - k0 - bs;
        const int kb_lo = kb / sb * sb;                  // first block of this super-block
        const int64_t s0 = (int64_t)kb_lo * CHOL_NB;
        float* Pk = P + (kb - kb_lo) * CHOL_NB;          // this block's panel slot
        if (!diag_done) {
            hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, s, U, n, k0, bs, info);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // block kb - 1 in this super-block: this block's update of its diagonal block goes in
        // the trsm launch, and its factor in the near launch
        const bool fuse = kb > kb_lo && k0 > 0;

        // trsm (rows above) + finalize (block row k of U, right of the diagonal): 64 x 64 tiles
        // while they fit one round on the chip (the launch's LDS allows one workgroup per CU),
        // 128 x 128 tiles past that
        const int64_t tiles64 = cdiv(k0, 64) * cdiv(bs, 64) + cdiv(bs, 64) * cdiv(r, 64);
        e = tiles64 > PANEL64_MAX_TILES ? launch_panel<128>(U, Pk, pld, n, k0, bs, r, fuse, vu, info, s)
                                        : launch_panel<64>(U, Pk, pld, n, k0, bs, r, fuse, vu, info, s);
        if (e != hipSuccess) return e;
        diag_done = false;
        if (k0 == 0) break;
        if (fuse) {
            // more blocks of this super-block follow: only what they need now, and the next
            // block's diagonal factor
            const int64_t big = cdiv(k0, 128) * cdiv(k0 - s0, 128) + cdiv(k0 - s0, 128) * cdiv(n - k0, 128);
            e = dl_ok(n, bs, pld, vu) && big >= 256 ? launch_near_diag_dl<128>(U, Pk, pld, n, s0, k0, bs, info, s)
                : big >= 512                          ? launch_near_diag<128>(U, Pk, pld, n, s0, k0, bs, info, vu, s)
                                                      : launch_near_diag<64>(U, Pk, pld, n, s0, k0, bs, info, vu, s);
            diag_done = true;
        } else {
            // super-block done: everything above and right of it, depth = its width
            const int kf = (int)((kb_lo + sb) * (int64_t)CHOL_NB < n ? sb * CHOL_NB : n - s0);
            const int64_t big = cdiv(s0, 128) * cdiv(n, 128);
            // 256-tiles on the split route from 1024 of them (their four-times-larger tiles
            // must still fill the chip), float32 128-tiles (two workgroups per CU) from 256
            const bool dl = dl_ok(n, kf, pld, vu);
            e = far_split(n, s0)     ? launch_far_split(U, P, pld, n, s0, kf, info, pcs, s)
                : dl && big >= 256   ? launch_far_dl<128>(U, P, pld, n, s0, kf, info, s)
                : big >= 512         ? launch_far<128>(U, P, pld, n, s0, kf, info, vu, s)
                                     : launch_far<64>(U, P, pld, n, s0, kf, info, vu, s);
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pwq
