// Round-to-nearest quantization and dequantization.
//
// RTN: per output row ("GPT-2 Quantization Reconstruction Error", "What this project
// does": one scale per output channel, 15 levels) or per group of g consecutive weights
// ("Model Quantization Mechanics", "Group-wise Quantization"), symmetric (Z = 0 in
// "Affine Quantization"): s = fp16(fp32(absmax / qmax)), code = round(w / s); or with a
// zero-point per row and group (the same section's Z): the range [min(w, 0), max(w, 0)]
// onto codes 0 .. 2^b - 1, code = round(w / S) + Z.  Each kernel takes the choice as a
// template argument, so the symmetric code is unchanged by the zero-point one.
// Dequant: What = s * (code - z), formed exactly in float32, rounded once to the output type.
//
// Both passes are HBM-bound, so what matters is bytes in flight per CU.
// RTN, groups that tile their rows (n % g == 0, 16-byte aligned rows, g * element size a
// power-of-two multiple of 16 bytes up to 1 KiB): a lane holds one 16-byte vector of its
// group (8 float16 or 4 float32 weights), LG = g * size / 16 lanes make a group, and each
// lane issues eight independent loads (eight sets of 64 / LG groups; nontemporal when rows
// are contiguous) before reducing.  The
// group max is a DPP reduction within rows of 16 lanes, the code a branch-free exact
// rounding; codes go out as 8 or 4 bytes per lane, INT4 nibbles as 4 or 2.
// RTN, other shapes (one scale per row, ragged or unaligned groups): a segment (row,
// group) is handled by L lanes (L = g/4 rounded up to a power of two, at most 64), each
// holding 4 consecutive weights per step.
// Dequant (n and g multiples of 8, no g_idx): 8-column chunks, a lane's four chunks 64
// apart so that loads and stores are contiguous across the wave, all four loads in flight.
// Grid-stride kernels are launched with as many workgroups as fit on the device at once.
#include "gemm_f32.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int RTN_CACHE = 8;   // quads per lane kept in registers between the two passes

template <int DT>
__device__ __forceinline__ float4 load_quad(const typename Elem<DT>::T* row, int64_t c, int64_t c1, bool vec) {
    if (vec && c + 3 < c1) return Elem<DT>::get4(row, c);
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = c + k < c1 ? Elem<DT>::get(row, c + k) : 0.f;
    return make_float4(t[0], t[1], t[2], t[3]);
}

struct RtnArgs {
    const void* W;
    int64_t ldw, m, n, ng, nseg;
    int gl;            // group length in columns (n for one scale per row)
    int L;             // lanes per segment (power of two, <= 64)
    int qmax, vec;
    uint64_t dmul;     // segment -> row: row = (seg * dmul) >> dsh (exact for seg < 2^31)
    int dsh;
    const uint16_t* scales_in;
    int8_t* codes;
    uint8_t* packed;
    uint16_t* scales_out;
    const uint16_t* zeros_in;   // zero-point form: fixed zeros (with scales_in) or NULL
    uint16_t* zeros_out;        // zero-point form: the zero of every (row, group)
    int top;                    // zero-point form: largest code, 2^bits - 1
    float near;                 // 2^(bits - 20): the rounding's margin from half-integers
};

// Zero of a group in the zero-point form: fixed (clamped to [0, top]) or from the range.
__device__ __forceinline__ float rtn_zero(const RtnArgs& a, bool live, int64_t idx, float nlo, float s) {
    if (a.zeros_in) return live ? (float)min((int)a.zeros_in[idx], a.top) : 0.f;
    return zp_zero(nlo, s, (float)a.top);
}

template <int DT, bool ZP>
__global__ __launch_bounds__(256) void rtn_kernel(RtnArgs a) {
    typedef typename Elem<DT>::T T;
    const int lane = threadIdx.x & 63;
    const int L = a.L, spw = 64 / L;
    const int sub = lane / L, li = lane % L;
    const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int64_t iters = cdiv(a.nseg, spw);
    for (int64_t it = wave_id; it < iters; it += nwaves) {
        const int64_t seg = it * spw + sub;
        const bool live = seg < a.nseg;
        const int64_t r = live ? seg / a.ng : 0, G = live ? seg % a.ng : 0;
        const int64_t c0 = G * a.gl;
        const int64_t c1 = live ? (c0 + a.gl < a.n ? c0 + a.gl : a.n) : c0;
        const T* row = (const T*)a.W + r * a.ldw;

        float4 cache[RTN_CACHE];
        float amax = 0.f, nlo = 0.f;     // symmetric: max |w|; zero-point: max(w, 0), max(-w, 0)
        int qi = 0;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L, ++qi) {
            const float4 v = load_quad<DT>(row, c, c1, a.vec);
            if (qi < RTN_CACHE) cache[qi] = v;
            if (ZP) {
                amax = fmaxf(amax, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
                nlo = fmaxf(nlo, fmaxf(fmaxf(-v.x, -v.y), fmaxf(-v.z, -v.w)));
            } else {
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
        }
        amax = group_max(amax, L);
        if (ZP) nlo = group_max(nlo, L);
        uint16_t sb;
        if (a.scales_in) sb = live ? a.scales_in[r * a.ng + G] : 0;
        else sb = ZP ? zp_scale_bits(nlo, amax, a.top) : scale_bits_from_absmax(amax, a.qmax);
        if (live && li == 0) a.scales_out[r * a.ng + G] = sb;
        const float s = f16_bits_to_f32(sb);
        const float rs = s > 0.f ? 1.0f / s : 0.f;
        const float z = ZP ? rtn_zero(a, live, r * a.ng + G, nlo, s) : 0.f;
        if (ZP && live && li == 0) a.zeros_out[r * a.ng + G] = (uint16_t)z;
        const float qlo = ZP ? -z : -(float)a.qmax, qhi = ZP ? (float)a.top - z : (float)a.qmax;

        qi = 0;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L, ++qi) {
            const float4 v = qi < RTN_CACHE ? cache[qi] : load_quad<DT>(row, c, c1, a.vec);
            int q[4];
            if (ZP) {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) q[k] = s > 0.f ? (int)(round_quot_clamp(vv[k], s, rs, qlo, qhi) + z) : 0;
            } else {
                q[0] = s > 0.f ? quant_code(v.x, s, rs, a.qmax) : 0;
                q[1] = s > 0.f ? quant_code(v.y, s, rs, a.qmax) : 0;
                q[2] = s > 0.f ? quant_code(v.z, s, rs, a.qmax) : 0;
                q[3] = s > 0.f ? quant_code(v.w, s, rs, a.qmax) : 0;
            }
            const bool full = c + 3 < c1;
            if (a.codes) {
                int8_t* dst = a.codes + r * a.n + c;
                if (full && a.vec && (a.n % 4 == 0)) {
                    *(uint32_t*)dst = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                      ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
                } else {
                    for (int k = 0; k < 4; ++k)
                        if (c + k < c1) dst[k] = (int8_t)q[k];
                }
            }
            if (a.packed) {
                uint8_t* dst = a.packed + r * (a.n / 2) + c / 2;
                constexpr int OFF = ZP ? 0 : 8;           // nibble = code (+ 8 for signed codes)
                const uint8_t b0 = (uint8_t)((q[0] + OFF) | ((q[1] + OFF) << 4));
                const uint8_t b1 = (uint8_t)((q[2] + OFF) | ((q[3] + OFF) << 4));
                if (full && a.vec && (a.n % 4 == 0)) {
                    *(uint16_t*)dst = (uint16_t)(b0 | (b1 << 8));
                } else {
                    if (c + 1 < c1) dst[0] = b0;
                    if (c + 3 < c1) dst[1] = b1;
                }
            }
        }
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// max over aligned groups of LG lanes: swaps within quads, then the mirror of each 8-lane
// half-row and of each 16-lane row (DPP, no LDS), then lane shuffles across rows.  The
// values are maxima of |w| (or of w, -w and 0): at least 0 or -0, whose bit patterns as
// signed integers order as the floats do (-0 below +0), so an integer max serves.
template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int LG>
__device__ __forceinline__ float lanes_max(float f) {
    int v = __builtin_bit_cast(int, f);
    if (LG >= 2) v = max(v, dpp_mov_i<0xB1>(v));       // quad_perm [1, 0, 3, 2]
    if (LG >= 4) v = max(v, dpp_mov_i<0x4E>(v));       // quad_perm [2, 3, 0, 1]
    if (LG >= 8) v = max(v, dpp_mov_i<0x141>(v));      // row_half_mirror
    if (LG >= 16) v = max(v, dpp_mov_i<0x140>(v));     // row_mirror
    if (LG >= 32) v = max(v, __shfl_xor(v, 16, 64));
    if (LG >= 64) v = max(v, __shfl_xor(v, 32, 64));
    return __builtin_bit_cast(float, v);
}

// Groups that tile their rows, LG lanes per group (LG = g * sizeof(T) / 16).  The host
// guarantees that W, the codes and the nibbles each span less than 4 GiB, so addresses are
// 32-bit offsets from the (uniform) base pointers, and that there are fewer than 2^31
// groups; the scale index of a group is its segment number.
// FAST: rows contiguous (ldw = n) and scales (and zeros) computed here, the common case:
// a group's offsets are multiples of its segment number, and a zero scale needs no branch
// (reciprocal 0 and clamp bounds [0, 0] give the code 0, or Z = 0).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT, int LG, bool ZP, bool FAST>
__global__ __launch_bounds__(256) void rtn_group_kernel(RtnArgs a) {
    typedef typename Elem<DT>::T T;
    constexpr int ES = (int)sizeof(T);
    constexpr int EPV = 16 / ES;                           // weights per 16-byte vector
    constexpr int SPW = 64 / LG;                           // groups per wave load
    constexpr int U = 8;                                   // loads in flight per lane
    const int lane = threadIdx.x & 63;
    const int sub = lane / LG, li = lane % LG;
    const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const char* Wb = (const char*)a.W;
    const uint32_t ng = (uint32_t)a.ng, nseg = (uint32_t)a.nseg;
    const uint32_t ldb = (uint32_t)(a.ldw * ES), glb = (uint32_t)(a.gl * ES), n = (uint32_t)a.n;
    const int64_t iters = cdiv(a.nseg, (int64_t)SPW * U);
    for (int64_t it = wave_id; it < iters; it += nwaves) {
        uint4 raw[U];
        uint32_t rr[U], seg[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t sg0 = (uint32_t)((it * U + u) * SPW) + (uint32_t)sub;
            live[u] = sg0 < nseg;
            seg[u] = live[u] ? sg0 : 0u;                   // a dead slot reads group 0
            if (FAST) {
                rr[u] = 0;
                // W is read once: nontemporal, so it does not displace what is cached
                const u32x4 t4 = __builtin_nontemporal_load((const u32x4*)(Wb + (seg[u] * glb + (uint32_t)li * 16u)));
                raw[u] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
            } else {
                rr[u] = (uint32_t)(((uint64_t)seg[u] * a.dmul) >> a.dsh);
                const uint32_t G = seg[u] - rr[u] * ng;
                raw[u] = *(const uint4*)(Wb + (rr[u] * ldb + G * glb + (uint32_t)li * 16u));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[EPV];
            const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
            if (DT == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = __builtin_bit_cast(float, w4[k]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    v[2 * k] = f16_bits_to_f32((uint16_t)(w4[k] & 0xffff));
                    v[2 * k + 1] = f16_bits_to_f32((uint16_t)(w4[k] >> 16));
                }
            }
            float amax = 0.f, nlo = 0.f;
            if (ZP) {
#pragma unroll
                for (int k = 0; k < EPV; ++k) { amax = fmaxf(amax, v[k]); nlo = fmaxf(nlo, -v[k]); }
                amax = lanes_max<LG>(amax);
                nlo = lanes_max<LG>(nlo);
            } else {
#pragma unroll
                for (int k = 0; k < EPV; ++k) amax = fmaxf(amax, fabsf(v[k]));
                amax = lanes_max<LG>(amax);
            }
            uint16_t sb;
            if (!FAST && a.scales_in) sb = live[u] ? a.scales_in[seg[u]] : 0;
            else sb = ZP ? zp_scale_bits(nlo, amax, a.top) : scale_bits_from_absmax(amax, a.qmax);
            if (live[u] && li == 0) a.scales_out[seg[u]] = sb;
            const float sc = f16_bits_to_f32(sb);
            int q[EPV];
            if (FAST) {
                // stored code = clamp(rne(w / s) + off, lo, hi): off = Z (zero-point form) or
                // qmax + 1 (the nibble's offset; the signed code is 8 less)
                const bool pos = sc > 0.f;
                const float rs = pos ? __builtin_amdgcn_rcpf(sc) : 0.f;
                float off, lo, hi;
                if (ZP) {
                    const float topf = (float)a.top;
                    off = pos ? round_quot_clamp(nlo, sc, rs, 0.f, topf) : 0.f;
                    if (live[u] && li == 0) a.zeros_out[seg[u]] = (uint16_t)off;
                    lo = 0.f;
                    hi = pos ? topf : 0.f;
                } else {
                    off = (float)(a.qmax + 1);
                    lo = pos ? off - (float)a.qmax : off;
                    hi = pos ? off + (float)a.qmax : off;
                }
                // t = fma(w, 1/s, off) is within 2^(bits - 21) of w / s + off wherever the
                // clamp leaves it unchanged (|t| < 2^(bits + 1), the reciprocal within one
                // ulp), so rint(t) is exact unless t lies within near = 2^(bits - 20) of a
                // half-integer; then (rarely, one branch per wave) the vector takes the
                // exact rounding
                float kf[EPV];
                float dev = 0.f;                         // largest |t - rint(t)| of the vector
#pragma unroll
                for (int k = 0; k < EPV; ++k) {
                    const float t = fmaf(v[k], rs, off);
                    kf[k] = rintf(t);
                    dev = fmaxf(dev, fabsf(t - kf[k]));
                }
                if (__builtin_amdgcn_ballot_w64(dev > 0.5f - a.near) != 0) {
#pragma unroll
                    for (int k = 0; k < EPV; ++k) kf[k] = round_quot_clamp(v[k], sc, rs, lo - off, hi - off) + off;
                }
#pragma unroll
                for (int k = 0; k < EPV; ++k) q[k] = (int)__builtin_amdgcn_fmed3f(kf[k], lo, hi);
            } else {
                const float rs = __builtin_amdgcn_rcpf(sc);   // only a first guess: the fma check is exact
                if (ZP) {
                    const float z = rtn_zero(a, live[u], seg[u], nlo, sc);
                    if (live[u] && li == 0) a.zeros_out[seg[u]] = (uint16_t)z;
                    const float qlo = -z, qhi = (float)a.top - z;
#pragma unroll
                    for (int k = 0; k < EPV; ++k)
                        q[k] = sc > 0.f ? (int)(round_quot_clamp(v[k], sc, rs, qlo, qhi) + z) : 0;
                } else {
#pragma unroll
                    for (int k = 0; k < EPV; ++k) q[k] = sc > 0.f ? quant_code_sel(v[k], sc, rs, a.qmax) : 0;
                }
            }
            if (!live[u]) continue;
            // FAST: row rr * n + column c of the group = seg * gl + li * EPV (rows contiguous)
            const uint32_t c = FAST ? seg[u] * (uint32_t)a.gl + (uint32_t)(li * EPV)
                                    : (seg[u] - rr[u] * ng) * (uint32_t)a.gl + (uint32_t)(li * EPV);
            // FAST leaves the stored code (the nibble) in q; the signed code is 8 less
            const int qo = FAST && !ZP ? a.qmax + 1 : 0;
            if (a.codes) {
                int8_t* dst = a.codes + (rr[u] * n + c);
                uint32_t b[EPV / 4];
#pragma unroll
                for (int k = 0; k < EPV / 4; ++k)
                    b[k] = (uint32_t)((q[4 * k] - qo) & 0xff) | ((uint32_t)((q[4 * k + 1] - qo) & 0xff) << 8) |
                           ((uint32_t)((q[4 * k + 2] - qo) & 0xff) << 16) |
                           ((uint32_t)((q[4 * k + 3] - qo) & 0xff) << 24);
                if (EPV == 8) *(uint2*)dst = make_uint2(b[0], b[EPV / 4 - 1]);
                else *(uint32_t*)dst = b[0];
            }
            if (a.packed) {
                uint8_t* dst = a.packed + (rr[u] * (n / 2) + c / 2);
                uint32_t nib = 0;
#pragma unroll
                for (int k = 0; k < EPV; ++k) nib |= (uint32_t)(q[k] + (ZP || FAST ? 0 : 8)) << (4 * k);
                if (EPV == 8) *(uint32_t*)dst = nib;
                else *(uint16_t*)dst = (uint16_t)nib;
            }
        }
    }
}

struct DqArgs {
    const uint8_t* packed;
    const int8_t* codes;        // zero-point form: the bytes are unsigned codes
    const uint16_t* scales;
    const uint16_t* zeros;      // zero-point form: d_out x ng zeros; NULL for symmetric codes
    const int32_t* g_idx;
    int64_t m, n, ng, chunks;   // chunks of 8 columns per row
    int g;                      // 0 = one scale per row
    int vec;                    // n % 8 == 0, aligned buffers, uniform group per chunk
    void* out;
};

// code relative to the group's zero: q - z (zero-point form) or q (symmetric, nibble - 8)
template <bool ZP>
__device__ __forceinline__ int dq_code(const DqArgs& a, int64_t r, int64_t c, int64_t G) {
    if (ZP) {
        const int z = a.zeros[r * a.ng + G];
        if (a.packed) {
            const uint8_t b = a.packed[r * (a.n / 2) + c / 2];
            return (int)((c & 1) ? (b >> 4) : (b & 15)) - z;
        }
        return (int)(uint8_t)a.codes[r * a.n + c] - z;
    }
    if (a.packed) {
        const uint8_t b = a.packed[r * (a.n / 2) + c / 2];
        return (int)((c & 1) ? (b >> 4) : (b & 15)) - 8;
    }
    return a.codes[r * a.n + c];
}

// eight codes of one chunk, relative to the zero z (symmetric: z = 0, nibbles offset by 8)
template <bool ZP>
__device__ __forceinline__ void dq_unpack8(const DqArgs& a, uint2 w, int z, int q[8]) {
    if (a.packed) {
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = (int)((w.x >> (4 * k)) & 15) - (ZP ? z : 8);
    } else if (ZP) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[k] = (int)((w.x >> (8 * k)) & 0xff) - z;
            q[4 + k] = (int)((w.y >> (8 * k)) & 0xff) - z;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            q[k] = (int8_t)((w.x >> (8 * k)) & 0xff);
            q[4 + k] = (int8_t)((w.y >> (8 * k)) & 0xff);
        }
    }
}

__device__ __forceinline__ int64_t dq_group(const DqArgs& a, int64_t c) {
    return a.g == 0 ? 0 : (a.g_idx ? (int64_t)a.g_idx[c] : c / a.g);
}

template <int OT>
__device__ __forceinline__ void dq_store(void* out, int64_t i, float v) {
    if (OT == 0) ((float*)out)[i] = v;
    else if (OT == 1) ((uint16_t*)out)[i] = f32_to_f16_bits(v);
    else ((uint16_t*)out)[i] = f32_to_bf16_bits(v);
}

// n % 8 == 0, one group per 8-column chunk (g == 0 or g % 8 == 0, no g_idx), aligned
// buffers.  Chunks of 8 columns are numbered row-major; a wave takes 256 consecutive chunks
// per pass, lane l the chunks 64 j + l (j < 4): each load instruction reads 4 (nibbles) or 8
// (codes) contiguous bytes per lane, each store writes 16 or 32 contiguous bytes per lane,
// and the four loads of a lane are in flight together.
// GI: columns carry their own group (g_idx, act-order): each of a chunk's 8 columns takes the
// scale (and zero) of its group, read through one 32-byte load of g_idx.
template <int OT, bool ZP, bool GI = false>
__global__ __launch_bounds__(256) void dequant_vec_kernel(DqArgs a) {
    constexpr int U = 4;
    const int lane = threadIdx.x & 63;
    const int64_t cpr = a.n / 8;
    const int64_t total = a.m * cpr;
    const int64_t wave_id = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t base = wave_id * 64 * U; base < total; base += nwaves * 64 * U) {
        uint2 w[U];
        float sc[U];
        int zz[U];
        int64_t r[U], c0[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t t = base + 64 * u + lane;
            live[u] = t < total;
            const int64_t tt = live[u] ? t : 0;
            r[u] = tt / cpr;
            c0[u] = (tt - r[u] * cpr) * 8;
            if (a.packed) w[u] = make_uint2(*(const uint32_t*)(a.packed + r[u] * (a.n / 2) + c0[u] / 2), 0u);
            else w[u] = *(const uint2*)(a.codes + r[u] * a.n + c0[u]);
            if (!GI) {
                const int64_t gi = r[u] * a.ng + (a.g == 0 ? 0 : c0[u] / a.g);
                sc[u] = f16_bits_to_f32(a.scales[gi]);
                zz[u] = ZP ? (int)a.zeros[gi] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!live[u]) continue;
            int q[8];
            float v[8];
            if (GI) {
                const int4 g0 = *(const int4*)(a.g_idx + c0[u]), g1 = *(const int4*)(a.g_idx + c0[u] + 4);
                const int gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                dq_unpack8<ZP>(a, w[u], 0, q);             // zero-point form: the stored codes
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int64_t gi = r[u] * a.ng + gk[k];
                    const int z = ZP ? (int)a.zeros[gi] : 0;
                    v[k] = f16_bits_to_f32(a.scales[gi]) * (float)(q[k] - z);
                }
            } else {
                dq_unpack8<ZP>(a, w[u], zz[u], q);
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = sc[u] * (float)q[k];     // exact: 11 x at most 8 significant bits (zeros within the code range)
            }
            if (OT == 0) {
                float4* o = (float4*)((float*)a.out + r[u] * a.n + c0[u]);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
                uint32_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint16_t lo = OT == 1 ? f32_to_f16_bits(v[2 * k]) : f32_to_bf16_bits(v[2 * k]);
                    const uint16_t hi = OT == 1 ? f32_to_f16_bits(v[2 * k + 1]) : f32_to_bf16_bits(v[2 * k + 1]);
                    h[k] = (uint32_t)lo | ((uint32_t)hi << 16);
                }
                *(uint4*)((uint16_t*)a.out + r[u] * a.n + c0[u]) = make_uint4(h[0], h[1], h[2], h[3]);
            }
        }
    }
}

// Float16 output from nibbles whose groups tile the rows (g = 8 * 2^gsh, no g_idx), rows
// contiguous: chunk t of 8 columns is nibble word t, output vector t, group t >> gsh.  The
// arithmetic is packed float16: 1024 + n is exact (the bits 0x6400 | n), so is
// (1024 + n) - (1024 + z) = n - z, and the product with the scale is rounded once, like the
// float32 product (exact) rounded to float16.  Fewer than 2^31 chunks (host check).
typedef _Float16 dq_h2 __attribute__((ext_vector_type(2)));
typedef unsigned int dq_u4 __attribute__((ext_vector_type(4)));
template <bool ZP>
__global__ __launch_bounds__(256) void dequant_f16_kernel(DqArgs a, int gsh) {
    constexpr int U = 4;
    const uint32_t total = (uint32_t)(a.m * a.chunks);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave_id = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const uint32_t nwaves = (gridDim.x * blockDim.x) >> 6;
    const uint32_t* P = (const uint32_t*)a.packed;
    dq_u4* O = (dq_u4*)a.out;
    for (uint32_t base = wave_id * 64 * U; base < total; base += nwaves * 64 * U) {
        uint32_t w[U], s2[U], o2[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = base + 64 * u + lane;
            const uint32_t tt = t < total ? t : 0u;
            w[u] = P[tt];
            const uint32_t gi = tt >> gsh;
            const uint32_t sb = a.scales[gi];
            s2[u] = sb | (sb << 16);
            const uint32_t ob = 0x6400u | (ZP ? (uint32_t)a.zeros[gi] : 8u);
            o2[u] = ob | (ob << 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t t = base + 64 * u + lane;
            if (t >= total) continue;
            const uint32_t lo = w[u] & 0x0F0F0F0Fu, hi = (w[u] >> 4) & 0x0F0F0F0Fu;
            dq_u4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // low half: byte j of lo (nibble 2j), high half: byte j of hi (nibble 2j + 1)
                const uint32_t sel = (uint32_t)j | 0x0C00u | ((uint32_t)(4 + j) << 16) | 0x0C000000u;
                const uint32_t h = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
                const dq_h2 x = __builtin_bit_cast(dq_h2, h) - __builtin_bit_cast(dq_h2, o2[u]);
                r[j] = __builtin_bit_cast(uint32_t, x * __builtin_bit_cast(dq_h2, s2[u]));
            }
            __builtin_nontemporal_store(r, O + t);
        }
    }
}

template <int OT, bool ZP>
__global__ __launch_bounds__(256) void dequant_kernel(DqArgs a) {
    const int64_t total = a.m * a.chunks;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t r = t / a.chunks, c0 = (t % a.chunks) * 8;
        if (a.vec) {
            float v[8];
            int q[8];
            const uint2 w = a.packed ? make_uint2(*(const uint32_t*)(a.packed + r * (a.n / 2) + c0 / 2), 0u)
                                     : *(const uint2*)(a.codes + r * a.n + c0);
            const int64_t gi = r * a.ng + dq_group(a, c0);
            dq_unpack8<ZP>(a, w, ZP ? (int)a.zeros[gi] : 0, q);
            const float s = f16_bits_to_f32(a.scales[gi]);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = s * (float)q[k];      // exact: 11 x at most 8 significant bits (zeros within the code range)
            if (OT == 0) {
                float4* o = (float4*)((float*)a.out + r * a.n + c0);
                o[0] = make_float4(v[0], v[1], v[2], v[3]);
                o[1] = make_float4(v[4], v[5], v[6], v[7]);
            } else {
                uint32_t h[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint16_t lo = OT == 1 ? f32_to_f16_bits(v[2 * k]) : f32_to_bf16_bits(v[2 * k]);
                    const uint16_t hi = OT == 1 ? f32_to_f16_bits(v[2 * k + 1]) : f32_to_bf16_bits(v[2 * k + 1]);
                    h[k] = (uint32_t)lo | ((uint32_t)hi << 16);
                }
                *(uint4*)((uint16_t*)a.out + r * a.n + c0) = make_uint4(h[0], h[1], h[2], h[3]);
            }
        } else {
            for (int k = 0; k < 8; ++k) {
                const int64_t c = c0 + k;
                if (c >= a.n) break;
                const int64_t G = dq_group(a, c);
                const float s = f16_bits_to_f32(a.scales[r * a.ng + G]);
                dq_store<OT>(a.out, r * a.n + c, s * (float)dq_code<ZP>(a, r, c, G));
            }
        }
    }
}

// Workgroups of 256 that fit on the device at once for kernel K (all CUs at K's occupancy),
// at most `want`: grid-stride kernels launched with this many take one round.  Both
// figures are taken once per kernel.
template <auto K>
int64_t resident_blocks(int64_t want) {
    static const int64_t cap = [] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, (const void*)K, 256, 0) != hipSuccess || per <= 0) per = 1;
        return (int64_t)cus * per;
    }();
    return want < cap ? (want > 0 ? want : 1) : cap;
}

// Per-tensor quantizer, first pass: the maxima of |w| (symmetric) or of w and -w (zero-point,
// each at least 0) over rows blockIdx.x, blockIdx.x + gridDim.x, ...; one pair per workgroup.
template <int DT>
__global__ __launch_bounds__(256) void tensor_max_kernel(const void* __restrict__ Wv, int64_t ldw, int64_t m, int64_t n,
                                                         int vec, float2* __restrict__ part) {
    typedef typename Elem<DT>::T T;
    __shared__ float2 red[4];
    float hi = 0.f, nlo = 0.f;
    for (int64_t r = blockIdx.x; r < m; r += gridDim.x) {
        const T* row = (const T*)Wv + r * ldw;
        if (vec) {
            for (int64_t c = 4 * (int64_t)threadIdx.x; c < n; c += 4 * 256) {
                const float4 v = Elem<DT>::get4(row, c);
                hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
                nlo = fmaxf(nlo, fmaxf(fmaxf(-v.x, -v.y), fmaxf(-v.z, -v.w)));
            }
        } else {
            for (int64_t c = threadIdx.x; c < n; c += 256) {
                const float v = Elem<DT>::get(row, c);
                hi = fmaxf(hi, v);
                nlo = fmaxf(nlo, -v);
            }
        }
    }
    hi = wave_max(hi);
    nlo = wave_max(nlo);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(hi, nlo);
    __syncthreads();
    if (threadIdx.x == 0) {
        float2 t = red[0];
        for (int w = 1; w < 4; ++w) t = make_float2(fmaxf(t.x, red[w].x), fmaxf(t.y, red[w].y));
        part[blockIdx.x] = t;
    }
}

// Second pass (one workgroup): the tensor's quantizer from the partial maxima, written to
// every row (the per-row format with one shared value).  Maxima are order-independent, so
// the result does not depend on the split into workgroups.
__global__ __launch_bounds__(256) void tensor_scale_kernel(const float2* __restrict__ part, int nparts, int64_t m, int bits,
                                                           uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
    __shared__ float2 red[4];
    __shared__ uint16_t sz[2];
    float hi = 0.f, nlo = 0.f;
    for (int k = threadIdx.x; k < nparts; k += 256) {
        hi = fmaxf(hi, part[k].x);
        nlo = fmaxf(nlo, part[k].y);
    }
    hi = wave_max(hi);
    nlo = wave_max(nlo);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(hi, nlo);
    __syncthreads();
    if (threadIdx.x == 0) {
        float2 t = red[0];
        for (int w = 1; w < 4; ++w) t = make_float2(fmaxf(t.x, red[w].x), fmaxf(t.y, red[w].y));
        if (zeros) {
            const int top = (1 << bits) - 1;
            const uint16_t sb = zp_scale_bits(t.y, t.x, top);
            sz[0] = sb;
            sz[1] = (uint16_t)zp_zero(t.y, f16_bits_to_f32(sb), (float)top);
        } else {
            sz[0] = scale_bits_from_absmax(fmaxf(t.x, t.y), (1 << (bits - 1)) - 1);
            sz[1] = 0;
        }
    }
    __syncthreads();
    for (int64_t r = threadIdx.x; r < m; r += 256) {
        scales[r] = sz[0];
        if (zeros) zeros[r] = sz[1];
    }
}

}  // namespace

constexpr int TENSOR_PARTS = 1024;

size_t tensor_scales_ws_bytes() { return TENSOR_PARTS * sizeof(float2); }

hipError_t tensor_scales_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, int bits,
                                uint16_t* scales, uint16_t* zeros, void* ws, hipStream_t s) {
    if (m == 0) return hipSuccess;
    const int nb = (int)(m < TENSOR_PARTS ? m : TENSOR_PARTS);
    const size_t es = w_dtype == 0 ? 4 : 2;
    const int vec = (n % 4 == 0) && (ldw % 4 == 0) && aligned(W, 4 * es);
    float2* part = (float2*)ws;
    if (w_dtype == 0) hipLaunchKernelGGL(tensor_max_kernel<0>, dim3(nb), dim3(256), 0, s, W, ldw, m, n, vec, part);
    else hipLaunchKernelGGL(tensor_max_kernel<1>, dim3(nb), dim3(256), 0, s, W, ldw, m, n, vec, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tensor_scale_kernel, dim3(1), dim3(256), 0, s, part, nb, m, bits, scales, zeros);
    return hipGetLastError();
}

hipError_t rtn_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, int bits, int group_size,
                      const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out, hipStream_t s,
                      const uint16_t* zeros_in, uint16_t* zeros_out) {
    if (m == 0 || n == 0) return hipSuccess;
    RtnArgs a{};
    a.W = W; a.ldw = ldw; a.m = m; a.n = n;
    a.gl = group_size == 0 ? (int)n : group_size;
    a.ng = group_size == 0 ? 1 : cdiv(n, group_size);
    a.nseg = m * a.ng;
    int L = 1;
    while (L < 64 && 4 * L < a.gl) L <<= 1;
    a.L = L;
    a.qmax = (1 << (bits - 1)) - 1;
    const size_t es = w_dtype == 0 ? 4 : 2;
    a.vec = (ldw % 4 == 0) && (a.gl % 4 == 0) && aligned(W, 4 * es) && (!codes || aligned(codes, 4)) &&
            (!packed || aligned(packed, 2));
    a.scales_in = scales_in; a.codes = codes; a.packed = packed; a.scales_out = scales_out;
    a.zeros_in = zeros_in; a.zeros_out = zeros_out; a.top = (1 << bits) - 1;
    a.near = ldexpf(1.f, bits - 20);
    const bool zp = zeros_out != nullptr;
    // group path: whole groups per row, 16-byte vectors, LG a power of two <= 64
    const int64_t gbytes = group_size * (int64_t)es;
    int lg = (int)(gbytes / 16);
    const bool pow2 = lg > 0 && (lg & (lg - 1)) == 0;
    const int epv = w_dtype == 0 ? 4 : 8;
    if (group_size > 0 && n % group_size == 0 && gbytes % 16 == 0 && pow2 && lg <= 64 && (ldw % epv) == 0 &&
        aligned(W, 16) && (!codes || (n % epv == 0 && aligned(codes, epv))) && (!packed || aligned(packed, epv / 2)) &&
        a.nseg < ((int64_t)1 << 31) && m * ldw * (int64_t)es < ((int64_t)1 << 32) && m * n < ((int64_t)1 << 32)) {
        // row = floor(seg / ng) as (seg * dmul) >> (31 + l), dmul = ceil(2^(31 + l) / ng),
        // l = ceil(log2 ng): exact for every seg < 2^31 (division by an invariant integer)
        int l = 0;
        while (((int64_t)1 << l) < a.ng) ++l;
        a.dsh = 31 + l;
        a.dmul = (uint64_t)((((unsigned __int128)1 << a.dsh) + (unsigned __int128)a.ng - 1) / (unsigned __int128)a.ng);
        const int64_t waves = cdiv(a.nseg, (int64_t)(64 / lg) * 4);
        const int64_t want = cdiv(waves, 4);
        const bool fast = !scales_in && !zeros_in && ldw == n;
#define PWQ_RTN_K(DT, LGV, ZPV, FV)                                                                            \
        hipLaunchKernelGGL((rtn_group_kernel<DT, LGV, ZPV, FV>),                                               \
                           dim3((unsigned)resident_blocks<rtn_group_kernel<DT, LGV, ZPV, FV>>(want)), dim3(256), 0, s, a)
#define PWQ_RTN_G(DT, LGV)                                                                                  \
        do {                                                                                                    \
            if (zp) { if (fast) PWQ_RTN_K(DT, LGV, true, true); else PWQ_RTN_K(DT, LGV, true, false); }        \
            else { if (fast) PWQ_RTN_K(DT, LGV, false, true); else PWQ_RTN_K(DT, LGV, false, false); }         \
        } while (0)
#define PWQ_RTN_LG(DT)                                      \
        switch (lg) {                                       \
        case 1: PWQ_RTN_G(DT, 1); break;                    \
        case 2: PWQ_RTN_G(DT, 2); break;                    \
        case 4: PWQ_RTN_G(DT, 4); break;                    \
        case 8: PWQ_RTN_G(DT, 8); break;                    \
        case 16: PWQ_RTN_G(DT, 16); break;                  \
        case 32: PWQ_RTN_G(DT, 32); break;                  \
        default: PWQ_RTN_G(DT, 64); break;                  \
        }
        if (w_dtype == 0) { PWQ_RTN_LG(0) }
        else { PWQ_RTN_LG(1) }
#undef PWQ_RTN_LG
#undef PWQ_RTN_G
#undef PWQ_RTN_K
        return hipGetLastError();
    }
    const int64_t waves = cdiv(a.nseg, 64 / L);
    int64_t blocks = cdiv(waves, 4);
    if (blocks > 65536) blocks = 65536;
    if (w_dtype == 0) {
        if (zp) hipLaunchKernelGGL((rtn_kernel<0, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((rtn_kernel<0, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    } else {
        if (zp) hipLaunchKernelGGL((rtn_kernel<1, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((rtn_kernel<1, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t dequant_launch(const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                          int64_t m, int64_t n, int bits, int group_size, void* out, int out_dtype, hipStream_t s,
                          const uint16_t* zeros) {
    (void)bits;
    if (m == 0 || n == 0) return hipSuccess;
    DqArgs a{};
    a.packed = packed; a.codes = codes; a.scales = scales; a.zeros = zeros; a.g_idx = g_idx;
    const bool zp = zeros != nullptr;
    a.m = m; a.n = n; a.g = group_size;
    a.ng = group_size == 0 ? 1 : cdiv(n, group_size);
    a.chunks = cdiv(n, 8);
    a.out = out;
    const size_t os = out_dtype == 0 ? 4 : 2;
    a.vec = (n % 8 == 0) && (group_size == 0 || (group_size % 8 == 0 && !g_idx)) && aligned(out, 8 * os) &&
            (!packed || aligned(packed, 4)) && (!codes || aligned(codes, 8));
    const bool vec_gi = g_idx && group_size > 0 && (n % 8 == 0) && aligned(g_idx, 16) && aligned(out, 8 * os) &&
                        (!packed || aligned(packed, 4)) && (!codes || aligned(codes, 8));
    const int64_t gc = group_size / 8;
    if (packed && out_dtype == 1 && group_size > 0 && group_size % 8 == 0 && (gc & (gc - 1)) == 0 &&
        n % group_size == 0 && !g_idx && aligned(packed, 4) && aligned(out, 16) && m * a.chunks < ((int64_t)1 << 31)) {
        int gsh = 0;
        while (((int64_t)1 << gsh) < gc) ++gsh;
        const int64_t want = cdiv(m * a.chunks, 4 * 256);
        if (zp) hipLaunchKernelGGL((dequant_f16_kernel<true>), dim3((unsigned)resident_blocks<dequant_f16_kernel<true>>(want)),
                                   dim3(256), 0, s, a, gsh);
        else hipLaunchKernelGGL((dequant_f16_kernel<false>), dim3((unsigned)resident_blocks<dequant_f16_kernel<false>>(want)),
                                dim3(256), 0, s, a, gsh);
        return hipGetLastError();
    }
    if (a.vec || vec_gi) {
        const int64_t want = cdiv(m * a.chunks, 4 * 256);
#define PWQ_DQV(OT, ZPV, GIV) \
        hipLaunchKernelGGL((dequant_vec_kernel<OT, ZPV, GIV>), \
                           dim3((unsigned)resident_blocks<dequant_vec_kernel<OT, ZPV, GIV>>(want)), dim3(256), 0, s, a)
#define PWQ_DQV2(OT, GIV) do { if (zp) PWQ_DQV(OT, true, GIV); else PWQ_DQV(OT, false, GIV); } while (0)
        if (vec_gi) {
            if (out_dtype == 0) PWQ_DQV2(0, true);
            else if (out_dtype == 1) PWQ_DQV2(1, true);
            else PWQ_DQV2(2, true);
        } else {
            if (out_dtype == 0) PWQ_DQV2(0, false);
            else if (out_dtype == 1) PWQ_DQV2(1, false);
            else PWQ_DQV2(2, false);
        }
#undef PWQ_DQV2
#undef PWQ_DQV
        return hipGetLastError();
    }
    int64_t blocks = cdiv(m * a.chunks, 256);
    if (blocks > 65536) blocks = 65536;
#define PWQ_DQ(OT, ZPV) hipLaunchKernelGGL((dequant_kernel<OT, ZPV>), dim3((unsigned)blocks), dim3(256), 0, s, a)
    if (out_dtype == 0) { if (zp) PWQ_DQ(0, true); else PWQ_DQ(0, false); }
    else if (out_dtype == 1) { if (zp) PWQ_DQ(1, true); else PWQ_DQ(1, false); }
    else { if (zp) PWQ_DQ(2, true); else PWQ_DQ(2, false); }
#undef PWQ_DQ
    return hipGetLastError();
}

}  // namespace pwq
