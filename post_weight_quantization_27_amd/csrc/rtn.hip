// Round-to-nearest quantization and dequantization.
//
// RTN: per output row ("GPT-2 Quantization Reconstruction Error", "What this project
// does": one scale per output channel, 15 levels) or per group of g consecutive weights
// ("Model Quantization Mechanics", "Group-wise Quantization"), symmetric (Z = 0 in
// "Affine Quantization"): s = fp16(fp32(absmax / qmax)), code = round(w / s).
// Dequant: What = s * code, formed exactly in float32, rounded once to the output type.
//
// Both passes are HBM-bound.  RTN: a segment (row, group) is handled by L lanes of a
// wave (L = g/4 rounded up to a power of two, at most 64), each lane holding 4 consecutive
// weights per step in registers (float4 / 4 x half loads), so a wave64 covers 256
// weights per load and several g = 128 groups at once; the group max is an L-lane
// shuffle reduction.  Codes go out as 4 bytes per lane, INT4 nibbles as 2 bytes per lane.
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
    const uint16_t* scales_in;
    int8_t* codes;
    uint8_t* packed;
    uint16_t* scales_out;
};

template <int DT>
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
        float amax = 0.f;
        int qi = 0;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L, ++qi) {
            const float4 v = load_quad<DT>(row, c, c1, a.vec);
            if (qi < RTN_CACHE) cache[qi] = v;
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        amax = group_max(amax, L);
        uint16_t sb;
        if (a.scales_in) sb = live ? a.scales_in[r * a.ng + G] : 0;
        else sb = scale_bits_from_absmax(amax, a.qmax);
        if (live && li == 0) a.scales_out[r * a.ng + G] = sb;
        const float s = f16_bits_to_f32(sb);
        const float rs = s > 0.f ? 1.0f / s : 0.f;

        qi = 0;
        for (int64_t c = c0 + 4 * li; c < c1; c += 4 * L, ++qi) {
            const float4 v = qi < RTN_CACHE ? cache[qi] : load_quad<DT>(row, c, c1, a.vec);
            int q[4];
            q[0] = s > 0.f ? quant_code(v.x, s, rs, a.qmax) : 0;
            q[1] = s > 0.f ? quant_code(v.y, s, rs, a.qmax) : 0;
            q[2] = s > 0.f ? quant_code(v.z, s, rs, a.qmax) : 0;
            q[3] = s > 0.f ? quant_code(v.w, s, rs, a.qmax) : 0;
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
                const uint8_t b0 = (uint8_t)((q[0] + 8) | ((q[1] + 8) << 4));
                const uint8_t b1 = (uint8_t)((q[2] + 8) | ((q[3] + 8) << 4));
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

struct DqArgs {
    const uint8_t* packed;
    const int8_t* codes;
    const uint16_t* scales;
    const int32_t* g_idx;
    int64_t m, n, ng, chunks;   // chunks of 8 columns per row
    int g;                      // 0 = one scale per row
    int vec;                    // n % 8 == 0, aligned buffers, uniform group per chunk
    void* out;
};

__device__ __forceinline__ int dq_code(const DqArgs& a, int64_t r, int64_t c) {
    if (a.packed) {
        const uint8_t b = a.packed[r * (a.n / 2) + c / 2];
        return (int)((c & 1) ? (b >> 4) : (b & 15)) - 8;
    }
    return a.codes[r * a.n + c];
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

template <int OT>
__global__ __launch_bounds__(256) void dequant_kernel(DqArgs a) {
    const int64_t total = a.m * a.chunks;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t r = t / a.chunks, c0 = (t % a.chunks) * 8;
        if (a.vec) {
            float v[8];
            int q[8];
            if (a.packed) {
                const uint32_t w = *(const uint32_t*)(a.packed + r * (a.n / 2) + c0 / 2);
#pragma unroll
                for (int k = 0; k < 8; ++k) q[k] = (int)((w >> (4 * k)) & 15) - 8;
            } else {
                const uint2 w = *(const uint2*)(a.codes + r * a.n + c0);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    q[k] = (int8_t)((w.x >> (8 * k)) & 0xff);
                    q[4 + k] = (int8_t)((w.y >> (8 * k)) & 0xff);
                }
            }
            const float s = f16_bits_to_f32(a.scales[r * a.ng + dq_group(a, c0)]);
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = s * (float)q[k];      // exact: 11 x 4 significant bits
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
                const float s = f16_bits_to_f32(a.scales[r * a.ng + dq_group(a, c)]);
                dq_store<OT>(a.out, r * a.n + c, s * (float)dq_code(a, r, c));
            }
        }
    }
}

}  // namespace

hipError_t rtn_launch(const void* W, int w_dtype, int64_t m, int64_t n, int64_t ldw, int bits, int group_size,
                      const uint16_t* scales_in, int8_t* codes, uint8_t* packed, uint16_t* scales_out, hipStream_t s) {
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
    const int64_t waves = cdiv(a.nseg, 64 / L);
    int64_t blocks = cdiv(waves, 4);
    if (blocks > 65536) blocks = 65536;
    if (w_dtype == 0) hipLaunchKernelGGL(rtn_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(rtn_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t dequant_launch(const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                          int64_t m, int64_t n, int bits, int group_size, void* out, int out_dtype, hipStream_t s) {
    (void)bits;
    if (m == 0 || n == 0) return hipSuccess;
    DqArgs a{};
    a.packed = packed; a.codes = codes; a.scales = scales; a.g_idx = g_idx;
    a.m = m; a.n = n; a.g = group_size;
    a.ng = group_size == 0 ? 1 : cdiv(n, group_size);
    a.chunks = cdiv(n, 8);
    a.out = out;
    const size_t os = out_dtype == 0 ? 4 : 2;
    a.vec = (n % 8 == 0) && (group_size == 0 || (group_size % 8 == 0 && !g_idx)) && aligned(out, 8 * os) &&
            (!packed || aligned(packed, 4)) && (!codes || aligned(codes, 8));
    int64_t blocks = cdiv(m * a.chunks, 256);
    if (blocks > 65536) blocks = 65536;
    if (out_dtype == 0) hipLaunchKernelGGL(dequant_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else if (out_dtype == 1) hipLaunchKernelGGL(dequant_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dequant_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pwq
