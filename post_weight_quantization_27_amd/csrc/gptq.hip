// GPTQ column loop ("GPTQ: Post-Training INT4", section "The GPTQ Algorithm"): columns in
// processing order, blocks of B, per column quantize / scaled error / in-block rank-1
// update, then one trailing product per block.  Scales follow "Group Quantization" of the
// same page (one float16 scale per row and group) and the per-row quantizer of
// "GPT-2 Quantization Reconstruction Error".  The zero-point form ("Model Quantization
// Mechanics", "Affine Quantization") takes each group's scale and zero from the range
// [min(w, 0), max(w, 0)] of the same current values; its codes are the clamped quotient
// round(w / S) in [-Z, 2^b - 1 - Z] plus Z, so the per-column step is the symmetric one with
// other clamp bounds (symmetric: +-qmax, Z = 0) and one add for the stored code.
//
// Kernels per layer:
//   prologue : float32 working copy Wf of W (columns permuted for act-order), per-row
//              scales from the original row, copy of caller-fixed scales
//   block    : four lanes per row (a quad), sixteen rows per wave64: lane p of a quad holds
//              the panel columns 4 i + p (i < B/4) in registers, and the B x B diagonal block
//              of U sits in LDS split by p, so every lane reads its U entries of row j with
//              16-byte broadcast loads.  For column j the owner value is broadcast inside the
//              quad with one DPP move; all four lanes quantize it (exact-quotient rounding)
//              and form e = (w - s q) / U_jj redundantly, and each lane applies
//              w -= e U[j][col] to its columns at or right of j (U is upper triangular, so
//              finished columns see zeros; the owner's own column is no longer read).  The
//              loop over j is fully unrolled so the register of column j is static.  Group
//              scales are a max over the group's registers plus two DPP steps.  Writes the
//              error panel Err (m x B), codes or INT4 nibbles (staged per wave in LDS) and
//              scales.
//   trailing : Wf[:, end:super] -= Err U[block, end:super] after each block, and
//              Wf[:, super:] -= Err_S U[super block, super:] after each super-block of
//              LAZY_COLS columns (float32 MFMA engine)
//   finish   : act-order only: codes back to the original column order, nibble packing and
//              g_idx.
#include "gemm_f32_dl.h"
#include "../../include/pwq.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int GB = 128;   // widest panel (block size)
// Error panels are kept for a super-block of columns: a block updates only the columns left
// in its super-block, and the columns past it get one product as deep as the super-block when
// it is done (the lazy batching of the column loop, one level up).  1024 columns for more than
// 4096 rows (the read-modify-write of the columns past a super-block then costs half as much
// per flop), else 512 (the row kernels apply the pending part of the super-block to their
// block themselves); except that a group wider than a block must start a super-block (its
// scale reads the columns past the panel, which are current only at a super-block's start):
// then the super-block is the group (up to 2048 columns; wider groups update every column
// after each block).
inline int lazy_cols(int group_size, int block_size, int64_t m) {
    if (group_size == 0 || group_size <= block_size) return m > 4096 ? 1024 : 512;
    return group_size <= 2048 ? group_size : block_size;
}

// zero-point form (zeros_out given): top = 2^bits - 1; fixed zeros are copied clamped to top
// Permuted rows are staged in LDS (one workgroup per CU), so those workgroups take 16 waves to
// keep enough loads in flight; plain rows take 4 (several workgroups per CU).
template <int DT, bool PERM>
__global__ __launch_bounds__(PERM ? 1024 : 256) void gptq_prologue_kernel(const void* __restrict__ W, int64_t ldw, int64_t m, int64_t n,
                                                            const int32_t* __restrict__ perm, float* __restrict__ Wf,
                                                            int row_scales, int qmax, const uint16_t* __restrict__ scales_in,
                                                            uint16_t* __restrict__ scales_out, int64_t ng,
                                                            const int32_t* __restrict__ info, int top,
                                                            const uint16_t* __restrict__ zeros_in,
                                                            uint16_t* __restrict__ zeros_out) {
    if (*info) return;
    typedef typename Elem<DT>::T T;
    constexpr int NT = PERM ? 1024 : 256, NW = NT / 64;
    __shared__ __attribute__((aligned(16))) float row[PERM ? PERM_MAX_N : 1];
    __shared__ float red[2 * NW];
    const int64_t r = blockIdx.x;
    const T* src = (const T*)W + r * ldw;
    float* dst = Wf + r * n;
    float amax = 0.f, hi = 0.f, nlo = 0.f;    // max |w|; max(w, 0), max(-w, 0)
    // rows of whole 4-element vectors, aligned: four weights per load
    const bool v4 = n % 4 == 0 && ldw % 4 == 0 && ((uintptr_t)W % (4 * sizeof(T))) == 0;
    if (PERM && v4) {
        constexpr int UR = 4;                  // vector loads in batches of four per thread
        const int64_t nv = n / 4;
        for (int64_t j0 = 0; j0 < nv; j0 += NT * UR) {
            float4 v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                v[u] = j < nv ? Elem<DT>::get4(src, 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                if (j < nv) *(float4*)(row + 4 * j) = v[u];
                const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    amax = fmaxf(amax, fabsf(e[k]));
                    hi = fmaxf(hi, e[k]);
                    nlo = fmaxf(nlo, -e[k]);
                }
            }
        }
    } else if (PERM) {
        // loads in batches of eight per thread (one memory latency per batch)
        constexpr int UR = 8;
        for (int64_t j0 = 0; j0 < n; j0 += NT * UR) {
            float v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                v[u] = j < n ? Elem<DT>::get(src, j) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                if (j < n) row[j] = v[u];
                amax = fmaxf(amax, fabsf(v[u]));
                hi = fmaxf(hi, v[u]);
                nlo = fmaxf(nlo, -v[u]);
            }
        }
    }
    if (PERM) {
        constexpr int UR = 8;
        __syncthreads();
        for (int64_t p0 = 0; p0 < n; p0 += NT * UR) {
            int32_t pj[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t p = p0 + u * NT + threadIdx.x;
                pj[u] = p < n ? perm[p] : 0;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t p = p0 + u * NT + threadIdx.x;
                if (p < n) dst[p] = row[pj[u]];
            }
        }
    } else if (v4) {
        constexpr int UR = 4;                  // vector loads in batches of four per thread
        const int64_t nv = n / 4;
        for (int64_t j0 = 0; j0 < nv; j0 += NT * UR) {
            float4 v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                v[u] = j < nv ? Elem<DT>::get4(src, 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * NT + threadIdx.x;
                if (j < nv) *(float4*)(dst + 4 * j) = v[u];
                const float e[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    amax = fmaxf(amax, fabsf(e[k]));
                    hi = fmaxf(hi, e[k]);
                    nlo = fmaxf(nlo, -e[k]);
                }
            }
        }
    } else {
        for (int64_t j = threadIdx.x; j < n; j += NT) {
            const float v = Elem<DT>::get(src, j);
            dst[j] = v;
            amax = fmaxf(amax, fabsf(v));
            hi = fmaxf(hi, v);
            nlo = fmaxf(nlo, -v);
        }
    }
    if (scales_in) {
        for (int64_t g = threadIdx.x; g < ng; g += NT) scales_out[r * ng + g] = scales_in[r * ng + g];
        if (zeros_out)
            for (int64_t g = threadIdx.x; g < ng; g += NT) zeros_out[r * ng + g] = (uint16_t)min((int)zeros_in[r * ng + g], top);
    } else if (row_scales) {
        if (zeros_out) {
            hi = wave_max(hi);
            nlo = wave_max(nlo);
            if ((threadIdx.x & 63) == 0) { red[threadIdx.x >> 6] = hi; red[NW + (threadIdx.x >> 6)] = nlo; }
        } else {
            amax = wave_max(amax);
            if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            float a = red[0], nl = zeros_out ? red[NW] : 0.f;
            for (int w = 1; w < NW; ++w) {
                a = fmaxf(a, red[w]);
                if (zeros_out) nl = fmaxf(nl, red[NW + w]);
            }
            if (zeros_out) {
                const uint16_t sb = zp_scale_bits(nl, a, top);
                scales_out[r] = sb;
                zeros_out[r] = (uint16_t)zp_zero(nl, f16_bits_to_f32(sb), (float)top);
            } else {
                scales_out[r] = scale_bits_from_absmax(a, qmax);
            }
        }
    }
}

// DPP quad permutations: every lane of a quad takes lane P's value / a neighbour's value
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int P>
__device__ __forceinline__ float quad_bcast(float v) { return dpp_f<P * 0x55>(v); }
// the lane index folds to a constant once the column loop is unrolled
__device__ __forceinline__ float quad_bcast_of(float v, int src) {
    switch (src) {
        case 0: return quad_bcast<0>(v);
        case 1: return quad_bcast<1>(v);
        case 2: return quad_bcast<2>(v);
        default: return quad_bcast<3>(v);
    }
}
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));        // quad_perm [1, 0, 3, 2]
    return fmaxf(v, dpp_f<0x4E>(v));     // quad_perm [2, 3, 0, 1]
}

struct BlockArgs {
    float* Wf;
    const float* U;
    const int32_t* info;
    int64_t m, n, b0;
    int bw, group_size, qmax, fixed_scales;
    int gsmall, gstart0;     // g <= B: groups start at panel columns j with j % g == 0; g > B: at j == 0 iff gstart0
    int64_t gbase;           // group index of the panel's first column
    uint16_t* scales;        // d_out x ng (already holds per-row / fixed scales)
    int64_t ng;
    int8_t* codes;           // processing order, ld n (nullable)
    uint8_t* packed;         // ld n/2 (nullable; only without act-order)
    float* err;              // this block's columns of the super-block's Err (m x err_ld)
    int err_ld;
    int pend;                // row kernels: columns of the super-block before this block, whose
    const float* err_sb;     // update the kernel applies itself (errors at err_sb, ld err_ld)
    uint16_t* zeros;         // zero-point form: d_out x ng zeros (like scales); NULL if symmetric
    int top;                 // zero-point form: largest code 2^bits - 1
    int nib_off;             // INT4 nibble = code + nib_off (8 symmetric, 0 zero-point)
};

// Clamp bounds of the rounded quotient and the offset of the stored code for a group with
// scale s and zero z: symmetric [-qmax, qmax] and 0, zero-point [-z, top - z] and z.  A
// zero scale gives [0, 0] and 0, so the rounding itself yields code 0 (with rs = 0 it
// returns a value within one of 0, which the clamp turns into 0): no select, and no branch
// the compiler could make of one, on the column-to-column chain.
struct QBounds {
    float lo, hi, z;
};
__device__ __forceinline__ QBounds qbounds(const BlockArgs& a, float z, float s) {
    if (!(s > 0.f)) return QBounds{0.f, 0.f, 0.f};
    if (a.zeros) return QBounds{-z, (float)a.top - z, z};
    return QBounds{-(float)a.qmax, (float)a.qmax, 0.f};
}
__device__ __forceinline__ float stored_zero(const BlockArgs& a, int64_t idx) {
    return a.zeros ? (float)a.zeros[idx] : 0.f;
}

// The panel's diagonal block of U (zero outside bw x bw), read as float4 rows with every
// load of a thread in flight before any is used: element e4 = tid + q NT of the PW x PW / 4
// float4 grid holds U[b0 + j][b0 + c .. c + 3], j = 4 e4 / PW, c = 4 e4 % PW.
template <int PW, int NT>
struct UBlock {
    static constexpr int N4 = PW * PW / 4;
    static constexpr int Q = (N4 + NT - 1) / NT;
    float4 v[Q];
    __device__ __forceinline__ static bool has(int tid, int q) { return N4 % NT == 0 || tid + q * NT < N4; }
    // rows [r0, r0 + PW) x columns [c0, c0 + PW) of U, zero outside rv rows and cv columns
    __device__ __forceinline__ void load_rect(const float* U, int64_t n, int64_t r0, int64_t c0, int rv, int cv, int tid) {
        const bool vec = (rv == PW) && (cv == PW) && (n % 4 == 0) && (c0 % 4 == 0);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if (!has(tid, q)) break;
            const int e = 4 * (tid + q * NT);
            const int j = e / PW, c = e % PW;
            const float* src = U + (r0 + j) * n + c0 + c;
            if (vec) {
                v[q] = *(const float4*)src;
            } else {
                float t[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) t[k] = (j < rv && c + k < cv) ? src[k] : 0.f;
                v[q] = make_float4(t[0], t[1], t[2], t[3]);
            }
        }
    }
    __device__ __forceinline__ void load(const float* U, int64_t n, int64_t b0, int bw, int tid) {
        load_rect(U, n, b0, b0, bw, bw, tid);
    }
};

// PW: panel width (the block size B); NWV: waves per workgroup (16 rows each).
template <int PW, int NWV>
__global__ __launch_bounds__(NWV * 64) void gptq_block_kernel(BlockArgs a) {
    if (*a.info) return;
    constexpr int NT = NWV * 64;
    constexpr int NC = PW / 4;           // columns per lane
    constexpr int UST = NC + 4;          // LDS stride of one lane slice of a U row (16-byte aligned, bank spread)
    __shared__ __attribute__((aligned(16))) float Ub[PW][4][UST];
    __shared__ float dinv[PW];
    __shared__ __attribute__((aligned(16))) int8_t cst[NWV][16][PW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = lane & 3, rq = lane >> 2;

    // diagonal block of U, zero outside the bw x bw panel (so padded columns never move),
    // split by quad lane: Ub[j][c & 3][c >> 2] = U[b0 + j][b0 + c]
    {
        UBlock<PW, NT> ub;
        ub.load(a.U, a.n, a.b0, a.bw, tid);
        float dv = 0.f;
        if (tid < PW && tid < a.bw) dv = 1.0f / a.U[(a.b0 + tid) * a.n + a.b0 + tid];
#pragma unroll
        for (int q = 0; q < UBlock<PW, NT>::Q; ++q) {
            if (!UBlock<PW, NT>::has(tid, q)) break;
            const int e = 4 * (tid + q * NT);
            const int j = e / PW, c = e % PW;        // c % 4 == 0: the four go to lanes 0..3
            Ub[j][0][c >> 2] = ub.v[q].x;
            Ub[j][1][c >> 2] = ub.v[q].y;
            Ub[j][2][c >> 2] = ub.v[q].z;
            Ub[j][3][c >> 2] = ub.v[q].w;
        }
        if (tid < PW) dinv[tid] = dv;
    }
    __syncthreads();

    const int64_t r = (int64_t)blockIdx.x * (NWV * 16) + wave * 16 + rq;
    const bool live = r < a.m;
    const float* wrow = a.Wf + (live ? r : 0) * a.n;
    float w[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) w[i] = (live && 4 * i + p < a.bw) ? wrow[a.b0 + 4 * i + p] : 0.f;

    const int g = a.group_size;
    float s = 0.f, z = 0.f;
    if (g == 0) {
        s = live ? f16_bits_to_f32(a.scales[r]) : 0.f;
        z = live ? stored_zero(a, r) : 0.f;
    } else if (!a.gsmall && !a.gstart0) {
        // a group wider than the panel that began in an earlier panel: its scale was fixed
        // (and stored) when the loop reached the group's first column
        s = live ? f16_bits_to_f32(a.scales[r * a.ng + a.gbase]) : 0.f;
        z = live ? stored_zero(a, r * a.ng + a.gbase) : 0.f;
    }
    float rs = s > 0.f ? 1.0f / s : 0.f;
    QBounds qb_ = qbounds(a, z, s);
    float eown[NC];
    uint32_t qb[(NC + 3) / 4];
#pragma unroll
    for (int i = 0; i < (NC + 3) / 4; ++i) qb[i] = 0u;

    // All PW columns are processed (a constant trip count keeps the loop unrolled, so every
    // register index is static): columns at or past bw hold 0 with zero rows of U and dinv,
    // so they yield q = e = 0 and are never written.  Steps go in windows of four columns
    // (the four lanes' columns of one register): the window's rows of U are read at its
    // start, and its results are pinned at its end.  Inside a window the scheduler is free
    // to hide the next column's dependency chain behind the current column's off-chain
    // updates; the pins keep the compiler from sinking update chains to their last use
    // (which would keep every step's e and U values live at once).
    const bool own[4] = {p == 0, p == 1, p == 2, p == 3};
    // full unrolling is forced: left to its cost model the compiler keeps this loop rolled
    // for PW = 64 and 128, and the register arrays indexed by jw then live in scratch memory
#pragma clang loop unroll(full)
    for (int jw = 0; jw < PW; jw += 4) {
        // this lane's entries of U rows jw .. jw+3 from register jw/4 on (the aligned group
        // holding column jw: the columns left of a pivot see U = 0, a no-op update)
        const int i0 = (jw >> 2) & ~3;
        float u[4][NC];
        float dj[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int i4 = i0; i4 < NC; i4 += 4) {
                const float4 v = *(const float4*)&Ub[jw + t][p][i4];
                u[t][i4] = v.x; u[t][i4 + 1] = v.y; u[t][i4 + 2] = v.z; u[t][i4 + 3] = v.w;
            }
            dj[t] = dinv[jw + t];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int j = jw + t;
            if ((j & 31) == 0 && j < a.bw && g != 0 && (a.gsmall ? (j % g) == 0 : (j == 0 && a.gstart0))) {
                // a group starts here: its scale comes from the current values of its columns,
                // panel columns [j, j + g) and, for a group wider than the panel, the columns
                // right of the panel (which hold every earlier update)
                const int64_t G = a.gbase + (a.gsmall ? j / g : 0);
                uint16_t sb;
                if (a.fixed_scales) {
                    sb = live ? a.scales[r * a.ng + G] : (uint16_t)0;
                    z = live ? stored_zero(a, r * a.ng + G) : 0.f;
                } else {
                    // symmetric: v = max |w|; zero-point: v = max(w, 0), nl = max(-w, 0)
                    const bool zp = a.zeros != nullptr;
                    const int ilim = a.gsmall ? (j + g) / 4 : NC;
                    float v = 0.f, nl = 0.f;
#pragma unroll
                    for (int i = j / 4; i < NC; ++i)
                        if (i < ilim) {
                            v = fmaxf(v, zp ? w[i] : fabsf(w[i]));
                            nl = fmaxf(nl, -w[i]);
                        }
                    if (!a.gsmall && live) {
                        const int64_t col = a.b0;
                        const int64_t gend = col + g < a.n ? col + g : a.n;
                        for (int64_t c = a.b0 + a.bw + p; c < gend; c += 4) {
                            const float x = wrow[c];
                            v = fmaxf(v, zp ? x : fabsf(x));
                            nl = fmaxf(nl, -x);
                        }
                    }
                    v = quad_max(v);
                    if (zp) {
                        nl = quad_max(nl);
                        sb = zp_scale_bits(nl, v, a.top);
                        z = zp_zero(nl, f16_bits_to_f32(sb), (float)a.top);
                        if (p == 0 && live) a.zeros[r * a.ng + G] = (uint16_t)z;
                    } else {
                        sb = scale_bits_from_absmax(v, a.qmax);
                    }
                    if (p == 0 && live) a.scales[r * a.ng + G] = sb;
                }
                s = f16_bits_to_f32(sb);
                rs = s > 0.f ? 1.0f / s : 0.f;
                qb_ = qbounds(a, z, s);
            }
            // column j: owner lane j & 3 (= t), register j >> 2, broadcast inside the quad
            const float wj = quad_bcast_of(w[j >> 2], t);
            // nearest integer to the exact quotient w / s, ties to even, without branches:
            // k = rint(w * rcp(s)) is within one of it, and the signs of the exact residuals
            // w - (k +- 1/2) s (one rounding each in fma) move it to the right integer.
            // s = 0 (an all-zero or underflowed group) gives code 0.
            // The quotient is clamped to [lo, hi] (symmetric +-qmax; zero-point [-z, top - z])
            // and the stored code is it plus z.
            const float kf = fminf(fmaxf(rintf(wj * rs), qb_.lo - 1.f), qb_.hi + 1.f);
            const float hi = fmaf(-(kf + 0.5f), s, wj);
            const float lo = fmaf(-(kf - 0.5f), s, wj);
            const int ki = (int)kf;
            const int odd = ki & 1;
            const int up = (hi > 0.f) | ((hi == 0.f) & odd);
            const int dn = (lo < 0.f) | ((lo == 0.f) & odd);
            const float qf = __builtin_amdgcn_fmed3f((float)(ki + up - dn), qb_.lo, qb_.hi);
            const float e = (wj - s * qf) * dj[t];
            const int q = (int)(qf + qb_.z);
            // the owner lane of column j keeps its error and code (selects, no branches)
            eown[j >> 2] = own[t] ? e : eown[j >> 2];
            qb[j >> 4] = own[t] ? (qb[j >> 4] | ((uint32_t)(q & 0xff) << (8 * ((j >> 2) & 3)))) : qb[j >> 4];
#pragma unroll
            for (int i = i0; i < NC; ++i) w[i] = fmaf(-e, u[t][i], w[i]);
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(w[i]));
#pragma unroll
        for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(eown[i]));
#pragma unroll
        for (int i = 0; i < (NC + 3) / 4; ++i) asm volatile("" : "+v"(qb[i]));
        __builtin_amdgcn_sched_barrier(0);
    }

    // error panel: Err[r][4 i + p]
    if (live) {
        float* erow = a.err + r * a.err_ld;
#pragma unroll
        for (int i = 0; i < NC; ++i)
            if (4 * i + p < a.bw) erow[4 * i + p] = eown[i];
    }
    if (a.codes || a.packed) {
        // codes through LDS: row rq, column 4 i + p, then 32 consecutive codes per lane
#pragma unroll
        for (int i = 0; i < NC; ++i) cst[wave][rq][4 * i + p] = (int8_t)((qb[i >> 2] >> (8 * (i & 3))) & 0xff);
        __syncthreads();                               // uniform branch: every thread gets here
        constexpr int PER = PW / 4;                    // codes per lane in the write-out
        const int c0 = PER * p;
        if (live) {
            const int8_t* src = &cst[wave][rq][c0];
            if (a.codes) {
                int8_t* crow = a.codes + r * a.n + a.b0;
                for (int c = 0; c < PER; ++c)
                    if (c0 + c < a.bw) crow[c0 + c] = src[c];
            }
            if (a.packed) {
                // byte k of the panel holds columns 2k (low nibble) and 2k+1 (high nibble)
                uint8_t* prow = a.packed + r * (a.n / 2) + a.b0 / 2;
                for (int c = 0; c < PER; c += 2)
                    if (c0 + c < a.bw)
                        prow[(c0 + c) / 2] = (uint8_t)(((src[c] + a.nib_off) & 15) | (((src[c + 1] + a.nib_off) & 15) << 4));
            }
        }
    }
}

// a wave-uniform value, marked as such (SGPR), so branches on it are uniform ones
__device__ __forceinline__ float uniform_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// One wave per row, for layers with few rows (latency matters more than issue slots):
// lane l holds panel columns l and l + 64.  Column j's value comes from its lane with a
// readlane at a static lane index (the loop is unrolled), so the quantization runs on a
// uniform value; every lane then updates its two columns.  The next row of U is read one
// step ahead, 1 / U_jj comes from a register by readlane, and the owner lane keeps e and
// the code with selects: no LDS wait and no branch sits on the column-to-column chain.
template <int PW, int NWV>
__global__ __launch_bounds__(NWV * 64) void gptq_row_kernel(BlockArgs a) {
    if (*a.info) return;
    constexpr int NT = NWV * 64;
    constexpr int NS = PW > 64 ? 2 : 1;              // registers per lane
    __shared__ __attribute__((aligned(16))) float Ub[PW][PW];
    __shared__ float esh[NWV][PW];
    __shared__ int8_t qsh[NWV][PW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = (int64_t)blockIdx.x * NWV + wave;
    const bool live = r < a.m;                       // uniform per wave
    const bool lane_in = lane < PW;                  // PW = 32: lanes 32..63 hold no column
    float w[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k)
        w[k] = (live && lane + 64 * k < a.bw && lane_in) ? a.Wf[r * a.n + a.b0 + 64 * k + lane] : 0.f;

    // the update still owed by this block's columns from the earlier blocks of its
    // super-block: w -= Err[r, s0 .. b0) U[s0 .. b0, block], one block's U rows at a time
    // staged in Ub (each block's sum is formed on its own and taken off once, as a product
    // per block would).  The next slice, and finally the diagonal block, is read into
    // registers while the current one is used; the row's errors are read before that, so
    // waiting for them does not wait for the prefetch.
    UBlock<PW, NT> ub;
    if (a.pend > 0) ub.load_rect(a.U, a.n, a.b0 - a.pend, a.b0, PW, a.bw, tid);
    else ub.load(a.U, a.n, a.b0, a.bw, tid);
    for (int c0 = 0; c0 < a.pend; c0 += PW) {
        __syncthreads();                             // the previous slice is consumed
#pragma unroll
        for (int q = 0; q < UBlock<PW, NT>::Q; ++q) {
            if (!UBlock<PW, NT>::has(tid, q)) break;
            const int e = 4 * (tid + q * NT);
            *(float4*)&Ub[e / PW][e % PW] = ub.v[q];
        }
        __syncthreads();
        float ev[NS], acc[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            ev[k] = (live && lane_in) ? a.err_sb[r * a.err_ld + c0 + 64 * k + lane] : 0.f;
            acc[k] = 0.f;
        }
        if (c0 + PW < a.pend) ub.load_rect(a.U, a.n, a.b0 - a.pend + c0 + PW, a.b0, PW, a.bw, tid);
        else ub.load(a.U, a.n, a.b0, a.bw, tid);
        if (live) {
            // sixteen rows' reads go out together, then their FMAs (same summation order)
#pragma unroll
            for (int j0 = 0; j0 < PW; j0 += 16) {
                float uu[16][NS];
#pragma unroll
                for (int jj = 0; jj < 16; ++jj)
#pragma unroll
                    for (int k = 0; k < NS; ++k) uu[jj][k] = lane_in ? Ub[j0 + jj][64 * k + lane] : 0.f;
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    const int j = j0 + jj;
                    const float ej =
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ev[j >> 6]), j & 63));
#pragma unroll
                    for (int k = 0; k < NS; ++k) acc[k] = fmaf(ej, uu[jj][k], acc[k]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int k = 0; k < NS; ++k) w[k] -= acc[k];
        }
    }
    if (a.pend > 0) __syncthreads();                 // the last slice is consumed before Ub is reused
#pragma unroll
    for (int q = 0; q < UBlock<PW, NT>::Q; ++q) {
        if (!UBlock<PW, NT>::has(tid, q)) break;
        const int e = 4 * (tid + q * NT);
        *(float4*)&Ub[e / PW][e % PW] = ub.v[q];
    }
    float dreg[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int j = lane + 64 * k;
        dreg[k] = (j < a.bw && j < PW) ? 1.0f / a.U[(a.b0 + j) * a.n + a.b0 + j] : 0.f;
    }
    __syncthreads();

    if (live) {
        const float* wrow = a.Wf + r * a.n;
        const int g = a.group_size;
        float s = 0.f, z = 0.f;
        if (g == 0) {
            s = f16_bits_to_f32(a.scales[r]);
            z = stored_zero(a, r);
        } else if (!a.gsmall && !a.gstart0) {
            s = f16_bits_to_f32(a.scales[r * a.ng + a.gbase]);
            z = stored_zero(a, r * a.ng + a.gbase);
        }
        s = uniform_f(s);
        float rs = uniform_f(s > 0.f ? 1.0f / s : 0.f);
        QBounds qb_ = qbounds(a, uniform_f(z), s);

        float u[NS], un[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) u[k] = lane_in ? Ub[0][64 * k + lane] : 0.f;
        // fully unrolled (forced: the compiler's cost model keeps PW = 64 and 128 rolled),
        // so the lane of every readlane and the register of every column are static
#pragma clang loop unroll(full)
        for (int j = 0; j < PW; ++j) {
            if (j + 1 < PW) {
#pragma unroll
                for (int k = 0; k < NS; ++k) un[k] = lane_in ? Ub[j + 1][64 * k + lane] : 0.f;
            }
            if ((j & 31) == 0 && j < a.bw && g != 0 && (a.gsmall ? (j % g) == 0 : (j == 0 && a.gstart0))) {
                // a group starts here: current values of its columns (panel columns [j, j+g)
                // and, for a group wider than the panel, the columns right of it)
                const int64_t G = a.gbase + (a.gsmall ? j / g : 0);
                uint16_t sb;
                float zg = 0.f;
                if (a.fixed_scales) {
                    sb = a.scales[r * a.ng + G];
                    zg = stored_zero(a, r * a.ng + G);
                } else {
                    // symmetric: v = max |w|; zero-point: v = max(w, 0), nl = max(-w, 0)
                    const bool zp = a.zeros != nullptr;
                    const int cend = a.gsmall ? j + g : PW;
                    float v = 0.f, nl = 0.f;
#pragma unroll
                    for (int k = 0; k < NS; ++k) {
                        const int c = lane + 64 * k;
                        if (c >= j && c < cend) {
                            v = fmaxf(v, zp ? w[k] : fabsf(w[k]));
                            nl = fmaxf(nl, -w[k]);
                        }
                    }
                    if (!a.gsmall) {
                        const int64_t gend = a.b0 + g < a.n ? a.b0 + g : a.n;
                        for (int64_t c = a.b0 + a.bw + lane; c < gend; c += 64) {
                            const float x = wrow[c];
                            v = fmaxf(v, zp ? x : fabsf(x));
                            nl = fmaxf(nl, -x);
                        }
                    }
                    v = wave_max(v);
                    if (zp) {
                        nl = wave_max(nl);
                        sb = zp_scale_bits(nl, v, a.top);
                        zg = zp_zero(nl, f16_bits_to_f32(sb), (float)a.top);
                        if (lane == 0) a.zeros[r * a.ng + G] = (uint16_t)zg;
                    } else {
                        sb = scale_bits_from_absmax(v, a.qmax);
                    }
                    if (lane == 0) a.scales[r * a.ng + G] = sb;
                }
                s = uniform_f(f16_bits_to_f32(sb));
                rs = uniform_f(s > 0.f ? 1.0f / s : 0.f);
                qb_ = qbounds(a, uniform_f(zg), s);
            }
            // everything from here to e is the same in every lane (wj, s, rs, dj are
            // wave-uniform), so the rare exact-rounding branch is a uniform one
            const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w[j >> 6]), j & 63));
            const float dj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dreg[j >> 6]), j & 63));
            // branch-free exact rounding: no uniform branch (and no refilled instruction
            // buffer) on the column-to-column chain
            // (the quotient clamped to [lo, hi]; the stored code adds the zero, and s = 0 gives
            // code 0 whatever the zero)
            const float qf = round_quot_clamp(wj, s, rs, qb_.lo, qb_.hi);
            const float e = (wj - s * qf) * dj;
            // e and the code are wave-uniform: every lane stores the same value to the same
            // LDS word (no lane select), and each lane reads its own columns back at the end
            esh[wave][j] = e;
            qsh[wave][j] = (int8_t)(int)(qf + qb_.z);
            // columns left of j (and j itself) are final: only registers holding columns
            // >= j need the update, and U is 0 left of j anyway
#pragma unroll
            for (int k = j >> 6; k < NS; ++k) w[k] = fmaf(-e, u[k], w[k]);
#pragma unroll
            for (int k = 0; k < NS; ++k) u[k] = un[k];
            // materialise the step's state (keeps the compiler from sinking the update and
            // select chains to their last use, which would hold every step's values live)
#pragma unroll
            for (int k = 0; k < NS; ++k) asm volatile("" : "+v"(w[k]));
        }
        float eown[NS];
        int qown[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            eown[k] = lane_in ? esh[wave][64 * k + lane] : 0.f;
            qown[k] = lane_in ? qsh[wave][64 * k + lane] : 0;
        }

        float* erow = a.err + r * a.err_ld;
#pragma unroll
        for (int k = 0; k < NS; ++k)
            if (lane + 64 * k < a.bw && lane + 64 * k < PW) erow[64 * k + lane] = eown[k];
        if (a.codes) {
            int8_t* crow = a.codes + r * a.n + a.b0;
#pragma unroll
            for (int k = 0; k < NS; ++k)
                if (lane + 64 * k < a.bw && lane + 64 * k < PW) crow[64 * k + lane] = (int8_t)qown[k];
        }
        if (a.packed) {
            // byte l of the panel holds columns 2l (low nibble) and 2l+1 (high nibble)
            const int src = (2 * lane) & 63;
            const int lo0 = __shfl(qown[0], src, 64), hi0 = __shfl(qown[0], src + 1, 64);
            int lo = lo0, hi = hi0;
            if (NS == 2) {
                const int lo1 = __shfl(qown[NS - 1], src, 64), hi1 = __shfl(qown[NS - 1], src + 1, 64);
                lo = lane < 32 ? lo0 : lo1;
                hi = lane < 32 ? hi0 : hi1;
            }
            if (2 * lane < a.bw && 2 * lane < PW)
                a.packed[r * (a.n / 2) + a.b0 / 2 + lane] =
                    (uint8_t)(((lo + a.nib_off) & 15) | (((hi + a.nib_off) & 15) << 4));
        }
    }
}

// Wf[r][c0 + col] -= acc
struct EpiSub {
    static constexpr bool kRmw = true, kFast = true;
    float* out;
    int64_t ld, M, N;
    __device__ __forceinline__ bool whole(const Tile& t, int bm, int bn) const {
        return t.m0 + bm <= M && t.n0 + bn <= N;
    }
    __device__ __forceinline__ float* at(int64_t row, int64_t col) const { return out + row * ld + col; }
    __device__ __forceinline__ float combine(float o, float v) const { return o - v; }
    __device__ __forceinline__ float old(const Tile&, int64_t row, int64_t col) const {
        return (row < M && col < N) ? out[row * ld + col] : 0.f;
    }
    __device__ __forceinline__ void put(const Tile&, int64_t row, int64_t col, float v, float o) {
        if (row < M && col < N) out[row * ld + col] = o - v;
    }
    __device__ __forceinline__ void finish(const Tile&, int, bool) {}
};

__global__ __launch_bounds__(256) void inv_perm_kernel(const int32_t* __restrict__ perm, int64_t n, int g,
                                                       int32_t* __restrict__ inv, int32_t* __restrict__ g_idx) {
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= n) return;
    const int32_t c = perm[p];
    inv[c] = (int32_t)p;
    g_idx[c] = g == 0 ? 0 : (int32_t)(p / g);
}

// codes back to original column order (row staged in LDS) + optional nibble packing
__global__ __launch_bounds__(256) void unpermute_codes_kernel(const int8_t* __restrict__ cp, const int32_t* __restrict__ inv,
                                                              int64_t n, int8_t* __restrict__ codes, uint8_t* __restrict__ packed,
                                                              int nib_off, const int32_t* __restrict__ info) {
    if (*info) return;
    __shared__ __attribute__((aligned(16))) int8_t row[PERM_MAX_N];
    constexpr int UR = 8;                  // loads in batches of eight per thread
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    if (n % 4 == 0) {
        // four codes per load (rows of n bytes, n a multiple of 4: every row 4-byte aligned)
        const uint32_t* src = (const uint32_t*)(cp + r * n);
        uint32_t* dst = (uint32_t*)row;
        const int64_t nw = n / 4;
        for (int64_t j0 = 0; j0 < nw; j0 += 256 * UR) {
            uint32_t v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * 256 + tid;
                v[u] = j < nw ? src[j] : 0u;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * 256 + tid;
                if (j < nw) dst[j] = v[u];
            }
        }
    } else {
        for (int64_t j0 = 0; j0 < n; j0 += 256 * UR) {
            int8_t v[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * 256 + tid;
                v[u] = j < n ? cp[r * n + j] : (int8_t)0;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t j = j0 + u * 256 + tid;
                if (j < n) row[j] = v[u];
            }
        }
    }
    __syncthreads();
    if (codes)
        for (int64_t c0 = 0; c0 < n; c0 += 256 * UR) {
            int32_t ic[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t c = c0 + u * 256 + tid;
                ic[u] = c < n ? inv[c] : 0;
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t c = c0 + u * 256 + tid;
                if (c < n) codes[r * n + c] = row[ic[u]];
            }
        }
    if (packed)
        for (int64_t b0 = 0; b0 < n / 2; b0 += 256 * UR) {
            int2 ib[UR];
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t b = b0 + u * 256 + tid;
                ib[u] = b < n / 2 ? make_int2(inv[2 * b], inv[2 * b + 1]) : make_int2(0, 0);
            }
#pragma unroll
            for (int u = 0; u < UR; ++u) {
                const int64_t b = b0 + u * 256 + tid;
                if (b < n / 2) {
                    const int lo = row[ib[u].x], hi = row[ib[u].y];
                    packed[r * (n / 2) + b] = (uint8_t)(((lo + nib_off) & 15) | (((hi + nib_off) & 15) << 4));
                }
            }
        }
}

// Wf[:, c0:c1] -= Err[:, 0:kw] U[kb0:kb0+kw, c0:c1]  (Err with row stride ld)
template <int BM, int BN>
hipError_t trailing(float* Wf, const float* err, int ld, const float* U, const int32_t* info, int64_t m, int64_t n,
                    int64_t kb0, int kw, int64_t c0, int64_t c1, hipStream_t s) {
    const int64_t N = c1 - c0;
    OpMMajor<0> a{err, ld, m, kw, (int)(aligned(err, 16) && ld % 4 == 0)};
    OpKMajor<0> b{U + kb0 * n + c0, n, N, kw, (int)((n % 4 == 0) && aligned(U, 16) && (c0 % 4 == 0))};
    RectMap mp{};
    mp.M = m; mp.N = N; mp.K = kw;
    mp.tiles_m = (int)cdiv(m, BM);
    mp.tiles_n = (int)cdiv(N, BN);
    mp.splits = 1;
    mp.kchunk = cdiv(kw, GEMM_BK) * GEMM_BK;
    mp.tri_k = 0;
    mp.guard = info;
    EpiSub ep{Wf + c0, n, m, N};
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, OpMMajor<0>, OpKMajor<0>, RectMap, EpiSub>),
                       dim3(mp.tiles_m * mp.tiles_n), dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

// The same product on the direct-load engine (T x T tiles; kw a whole number of its stages,
// 16-byte aligned rows)
template <int T>
hipError_t trailing_dl(float* Wf, const float* err, int ld, const float* U, const int32_t* info, int64_t m, int64_t n,
                       int64_t kb0, int kw, int64_t c0, int64_t c1, hipStream_t s) {
    const int64_t N = c1 - c0;
    FdlRows<T> a{err, ld, m};
    FdlCols<T> b{U + kb0 * n + c0, n, N};
    RectMap mp{};
    mp.M = m; mp.N = N; mp.K = kw;
    mp.tiles_m = (int)cdiv(m, T);
    mp.tiles_n = (int)cdiv(N, T);
    mp.splits = 1;
    mp.kchunk = kw;
    mp.tri_k = 0;
    mp.guard = info;
    EpiSub ep{Wf + c0, n, m, N};
    hipLaunchKernelGGL((gemm_fdl_kernel<FdlRows<T>, FdlCols<T>, RectMap, EpiSub>), dim3(mp.tiles_m * mp.tiles_n),
                       dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

// The same product on bfloat16 MFMA (the 256-tile register-staged engine): Err[:, 0:kw] and
// the rows U[kb0:kb0+kw, c0:c1] are cut into their three-piece splits (split3_tiled_block)
// and each float32 product is the sum of the six larger piece products, as in the factor's
// far products; the dropped three are below 2^-23 of |a| |b| each.  pcs: 3 (panel-padded m +
// panel-padded (c1 - c0)) kseg values, kseg = kw rounded up to 64.
template <bool KMAJ>
__global__ __launch_bounds__(256) void gptq_split3_kernel(const float* __restrict__ src, int64_t ld, int64_t M, int64_t K,
                                                          uint16_t* __restrict__ out, int64_t kseg, int64_t pstride) {
    split3_tiled_block<KMAJ>(src, ld, M, K, out, kseg, pstride);
}

hipError_t trailing_split(float* Wf, const float* err, int ld, const float* U, const int32_t* info, int64_t m, int64_t n,
                          int64_t kb0, int kw, int64_t c0, int64_t c1, uint16_t* pcs, hipStream_t s) {
    const int64_t N = c1 - c0;
    const int64_t kseg = cdiv(kw, 64) * 64;
    const int64_t ma = dl_panel_pad(m), mb = dl_panel_pad(N);
    uint16_t* A = pcs;                                   // pieces of Err[:, 0:kw]
    uint16_t* B = pcs + 3 * ma * kseg;                   // pieces of U[kb0:kb0+kw, c0:c1]^T
    hipLaunchKernelGGL(gptq_split3_kernel<false>, dim3((unsigned)(ma / 64), (unsigned)(kseg / 64)), dim3(256), 0, s, err,
                       (int64_t)ld, m, (int64_t)kw, A, kseg, ma * kseg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gptq_split3_kernel<true>, dim3((unsigned)(mb / 64), (unsigned)(kseg / 64)), dim3(256), 0, s,
                       U + kb0 * n + c0, n, N, (int64_t)kw, B, kseg, mb * kseg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // (i, j) of the segments: (3,1), (1,3), (2,2), (2,1), (1,2), (1,1)
    const DlTiled6 a{{A + 2 * ma * kseg, A, A + ma * kseg, A + ma * kseg, A, A}, kseg};
    const DlTiled6 b{{B, B + 2 * mb * kseg, B + mb * kseg, B, B + mb * kseg, B}, kseg};
    // tiles in the per-XCD band order: each XCD's workgroups share operand panels
    const XcdRectMap mp{m, N, 6 * kseg, (int)cdiv(m, DL_TILE), (int)cdiv(N, DL_TILE), info};
    EpiSub ep{Wf + c0, n, m, N};
    hipLaunchKernelGGL((gemm_rs_kernel<2, DlTiled6, DlTiled6, XcdRectMap, EpiSub>),
                       dim3((unsigned)xcd_grid(mp.tiles_m * mp.tiles_n)), dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

// 256-tiles from which the direct-load engine takes a trailing product on 256 x 256 tiles;
// below that, 128-tiles from which it takes one on 128 x 128 tiles (two workgroups per CU).
// Products at least TRAIL_SPLIT_MIN_K deep with that many 256-tiles take the split route.
constexpr int64_t TRAIL_DL_MIN_TILES = 512;
constexpr int64_t TRAIL_DL128_MIN_TILES = 256;
constexpr int TRAIL_SPLIT_MIN_K = 512;

inline bool trail_split(int64_t m, int64_t N, int kw) {
    return kw >= TRAIL_SPLIT_MIN_K && cdiv(m, DL_TILE) * cdiv(N, DL_TILE) >= TRAIL_DL_MIN_TILES;
}

// pcs: the split route's pieces, or null where the workspace holds none (the route is off)
hipError_t update(float* Wf, const float* err, int ld, const float* U, const int32_t* info, int64_t m, int64_t n,
                  int64_t kb0, int kw, int64_t c0, int64_t c1, uint16_t* pcs, hipStream_t s) {
    const int64_t big_tiles = cdiv(m, 128) * cdiv(c1 - c0, 128);
    const bool dl = kw % FDL_BK == 0 && ld % 4 == 0 && n % 4 == 0 && c0 % 4 == 0 && aligned(err, 16) && aligned(U, 16);
    if (pcs && trail_split(m, c1 - c0, kw)) {
        // timed as its six bfloat16 products of kseg (the split kernels included)
        prof_begin(PWQ_PROF_UPDATE_SPLIT, s);
        const hipError_t e = trailing_split(Wf, err, ld, U, info, m, n, kb0, kw, c0, c1, pcs, s);
        prof_end(PWQ_PROF_UPDATE_SPLIT, s, 12.0 * m * (cdiv(kw, 64) * 64) * (c1 - c0));
        return e;
    }
    prof_begin(PWQ_PROF_UPDATE, s);
    const hipError_t e =
        dl && cdiv(m, 256) * cdiv(c1 - c0, 256) >= TRAIL_DL_MIN_TILES ? trailing_dl<256>(Wf, err, ld, U, info, m, n, kb0, kw, c0, c1, s)
        : dl && big_tiles >= TRAIL_DL128_MIN_TILES                  ? trailing_dl<128>(Wf, err, ld, U, info, m, n, kb0, kw, c0, c1, s)
        : big_tiles >= 512                                          ? trailing<128, 128>(Wf, err, ld, U, info, m, n, kb0, kw, c0, c1, s)
                                                                    : trailing<64, 64>(Wf, err, ld, U, info, m, n, kb0, kw, c0, c1, s);
    prof_end(PWQ_PROF_UPDATE, s, 2.0 * m * kw * (c1 - c0));
    return e;
}

}  // namespace

GptqWs gptq_ws_layout(int64_t d_out, int64_t d_in, int block_size, int group_size, int act_order) {
    GptqWs w{};
    size_t off = 0;
    w.wf = off;    off = align_up(off + (size_t)d_out * d_in * sizeof(float), 256);
    w.err = off;   off = align_up(off + (size_t)d_out * lazy_cols(group_size, block_size, d_out) * sizeof(float), 256);
    w.codes = off; if (act_order) off = align_up(off + (size_t)d_out * d_in, 256);
    w.inv = off;   if (act_order) off = align_up(off + (size_t)d_in * sizeof(int32_t), 256);
    // the split route's pieces (trailing_split), for the products past each super-block
    const int lz = lazy_cols(group_size, block_size, d_out);
    w.pcs = off;
    if (d_in > lz && trail_split(d_out, d_in - lz, lz))
        off = align_up(off + (size_t)3 * (size_t)(dl_panel_pad(d_out) + dl_panel_pad(d_in)) * (size_t)(cdiv(lz, 64) * 64) *
                                 sizeof(uint16_t), 256);
    w.has_pcs = off > w.pcs;
    w.total = off;
    return w;
}

hipError_t gptq_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, const float* U, const int32_t* info,
                       int bits, int group_size, int block_size, int act_order, const int32_t* perm,
                       const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out, int32_t* g_idx,
                       void* ws, hipStream_t s, const uint16_t* zeros_in, uint16_t* zeros_out) {
    if (m == 0 || n == 0) return hipSuccess;
    hipError_t e;
    const GptqWs L = gptq_ws_layout(m, n, block_size, group_size, act_order);
    const int lz = lazy_cols(group_size, block_size, m);
    char* base = (char*)ws;
    float* Wf = (float*)(base + L.wf);
    float* err = (float*)(base + L.err);
    int8_t* cproc = act_order ? (int8_t*)(base + L.codes) : codes;
    int32_t* inv = act_order ? (int32_t*)(base + L.inv) : nullptr;
    uint16_t* pcs = L.has_pcs ? (uint16_t*)(base + L.pcs) : nullptr;
    const int qmax = (1 << (bits - 1)) - 1;
    const int64_t ng = group_size == 0 ? 1 : cdiv(n, group_size);

    {
        auto k = w_dtype == 0 ? (act_order ? gptq_prologue_kernel<0, true> : gptq_prologue_kernel<0, false>)
                              : (act_order ? gptq_prologue_kernel<1, true> : gptq_prologue_kernel<1, false>);
        hipLaunchKernelGGL(k, dim3((unsigned)m), dim3(act_order ? 1024 : 256), 0, s, W, ldw, m, n, act_order ? perm : nullptr, Wf,
                           (int)(group_size == 0), qmax, scales_in, scales_out, ng, info, (1 << bits) - 1, zeros_in,
                           zeros_out);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    BlockArgs a{};
    a.Wf = Wf; a.U = U; a.info = info; a.m = m; a.n = n;
    a.group_size = group_size; a.qmax = qmax; a.fixed_scales = scales_in != nullptr;
    a.scales = scales_out; a.ng = ng; a.codes = cproc; a.packed = act_order ? nullptr : packed; a.err = err;
    a.zeros = zeros_out; a.top = (1 << bits) - 1; a.nib_off = zeros_out ? 0 : 8;
    // Few rows: one wave per row (the column chain's latency decides the time), workgroups
    // sized so the rows spread over the chip.  Many rows: four lanes per row, sixteen rows
    // per wave (issue slots decide), eight-wave workgroups.
    const bool quad = m > 4096;
    const int rwv = m <= 1024 ? 4 : 16;
    // quad kernel: up to 16384 rows, workgroups of 2 waves (16 rows each; two fit a CU's LDS)
    // spread the rows over every CU in one round, with at most one wave per SIMD (the column
    // chain of a wave issues faster alone); more rows take 8-wave workgroups, one per CU
    const int qwv = m <= 16384 ? 2 : 8;
    const unsigned nblk = quad ? (unsigned)cdiv(m, 16 * qwv) : (unsigned)cdiv(m, rwv);

    for (int64_t b0 = 0; b0 < n; b0 += block_size) {
        const int bw = (int)((n - b0) < block_size ? (n - b0) : block_size);
        const int64_t s0 = b0 / lz * lz;                               // super-block of this block
        const int64_t s1 = s0 + lz < n ? s0 + lz : n;
        a.b0 = b0;
        a.bw = bw;
        a.err = err + (b0 - s0);
        a.err_ld = lz;
        if (group_size != 0) {
            a.gsmall = group_size <= block_size;
            a.gstart0 = (b0 % group_size) == 0;
            a.gbase = b0 / group_size;
        }
        // row kernels take the update owed from the earlier blocks of the super-block
        // themselves; the quad kernel's block receives it from a product after each block
        a.pend = quad ? 0 : (int)(b0 - s0);
        a.err_sb = err;
        prof_begin(PWQ_PROF_COLUMNS, s);
        if (quad) {
#define PWQ_QUAD(PW)                                                                                              \
    do {                                                                                                          \
        if (qwv == 8) hipLaunchKernelGGL((gptq_block_kernel<PW, 8>), dim3(nblk), dim3(512), 0, s, a);            \
        else if (qwv == 4) hipLaunchKernelGGL((gptq_block_kernel<PW, 4>), dim3(nblk), dim3(256), 0, s, a);       \
        else hipLaunchKernelGGL((gptq_block_kernel<PW, 2>), dim3(nblk), dim3(128), 0, s, a);                     \
    } while (0)
            if (block_size == 128) PWQ_QUAD(128);
            else if (block_size == 64) PWQ_QUAD(64);
            else PWQ_QUAD(32);
#undef PWQ_QUAD
        } else if (rwv == 4) {
            if (block_size == 128) hipLaunchKernelGGL((gptq_row_kernel<128, 4>), dim3(nblk), dim3(256), 0, s, a);
            else if (block_size == 64) hipLaunchKernelGGL((gptq_row_kernel<64, 4>), dim3(nblk), dim3(256), 0, s, a);
            else hipLaunchKernelGGL((gptq_row_kernel<32, 4>), dim3(nblk), dim3(256), 0, s, a);
        } else {
            if (block_size == 128) hipLaunchKernelGGL((gptq_row_kernel<128, 16>), dim3(nblk), dim3(1024), 0, s, a);
            else if (block_size == 64) hipLaunchKernelGGL((gptq_row_kernel<64, 16>), dim3(nblk), dim3(1024), 0, s, a);
            else hipLaunchKernelGGL((gptq_row_kernel<32, 16>), dim3(nblk), dim3(1024), 0, s, a);
        }
        prof_end(PWQ_PROF_COLUMNS, s, (double)m * bw * (bw - 1));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int64_t b1 = b0 + bw;
        if (b1 < s1) {                     // the rest of the super-block, from this block's errors
            if (quad && (e = update(Wf, err + (b0 - s0), lz, U, info, m, n, b0, bw, b1, s1, pcs, s)) != hipSuccess) return e;
        } else if (s1 < n) {               // super-block done: every column past it, depth s1 - s0
            if ((e = update(Wf, err, lz, U, info, m, n, s0, (int)(s1 - s0), s1, n, pcs, s)) != hipSuccess) return e;
        }
    }
    if (act_order) {
        hipLaunchKernelGGL(inv_perm_kernel, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, perm, n, group_size, inv, g_idx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(unpermute_codes_kernel, dim3((unsigned)m), dim3(256), 0, s, cproc, inv, n, codes, packed,
                           zeros_out ? 0 : 8, info);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pwq
