// Shared device helpers for the gfx950 kernels of libpwq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pwq {

constexpr int WAVE = 64;

// ------------------------------------------------------------------ 16-bit formats
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {       // one RNE rounding
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {      // one RNE rounding
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ------------------------------------------------------------------ quantizer
// Scale of a symmetric group: absmax / qmax as one IEEE float32 division, then one RNE
// rounding to float16 (the stored 16-bit scale of "GPTQ: Post-Training INT4", section
// "Group Quantization"; symmetric S with Z = 0 of "Model Quantization Mechanics",
// "Affine Quantization").  The division relies on hipcc's default correctly rounded
// float32 divide (no fast-math flags anywhere in this library).
__device__ __forceinline__ uint16_t scale_bits_from_absmax(float absmax, int qmax) {
    float s32 = absmax / (float)qmax;
    return f32_to_f16_bits(s32);
}

// Code of w for scale s (s = a float16 value, > 0): the integer nearest to the EXACT
// quotient w / s, ties to even, clamped to [-qmax, qmax].
// k0 = rint(w * (1/s)) is within one of the answer; the signs of w - (k0 +- 1/2) s decide
// exactly, because (k0 +- 1/2) s has at most 16 significant bits (exact in float32) and a
// fused multiply-add rounds w - (k0 +- 1/2) s once, which preserves its sign and zero.
__device__ __forceinline__ int quant_code(float w, float s, float rs, int qmax) {
    float k = rintf(w * rs);
    float lim = (float)(qmax + 1);
    k = fminf(fmaxf(k, -lim), lim);
    float hi = fmaf(-(k + 0.5f), s, w);
    float lo = fmaf(-(k - 0.5f), s, w);
    int ki = (int)k;
    if (hi > 0.f || (hi == 0.f && (ki & 1))) {
        ki += 1;
    } else if (lo < 0.f || (lo == 0.f && (ki & 1))) {
        ki -= 1;
    }
    ki = ki < -qmax ? -qmax : ki;
    ki = ki > qmax ? qmax : ki;
    return ki;
}

// code for a possibly-zero scale (all-zero group -> code 0)
// The same code as quant_code, without branches and with one residual.  k = rint(w * rs)
// (rs any approximation of 1 / s that leaves w * rs within 1/2 of w / s) is the answer or
// its neighbour on the side where w * rs lies; h = k +- 1/2 is the half-integer between
// them.  The exact residual e = w - h s (h s has at most 20 significant bits for
// qmax <= 127, so the fma's one rounding keeps the sign and the zero of w - h s) says
// whether w / s lies past h, on it, or short of it, and rint(h + sign(e) / 4) is then the
// integer past h, the even neighbour (a tie), or k.  Finite inputs give exactly
// quant_code's result (s > 0; the callers give s = 0 the code 0).  quant_code_self returns
// the code as a float.
// round_quot_clamp is the same rounding clamped to [lo, hi] (integers with |lo|, |hi| <= 256,
// lo <= hi): the quotient only needs to be exact where it is not clamped, and there
// |k| <= 257 keeps h s exact.
__device__ __forceinline__ float round_quot_clamp(float w, float s, float rs, float lo, float hi) {
    const float t = w * rs;
    const float k = rintf(t);
    const float h = k + copysignf(0.5f, t - k);
    const float e = fmaf(-h, s, w);
    const float d = e != 0.f ? copysignf(0.25f, e) : 0.f;
    return __builtin_amdgcn_fmed3f(rintf(h + d), lo, hi);
}
__device__ __forceinline__ float quant_code_self(float w, float s, float rs, float qmaxf) {
    return round_quot_clamp(w, s, rs, -qmaxf, qmaxf);
}

// Zero-point quantizer of a group ("Model Quantization Mechanics", "Affine Quantization":
// code = round(w / S) + Z, value S (code - Z)).  The range [lo, hi] = [min(w, 0), max(w, 0)]
// is mapped onto the codes 0 .. top = 2^b - 1: S = fp16(fp32(hi - lo) / top) (one float32
// subtraction, one float32 division, one rounding to float16), Z = the integer nearest to
// -lo / S (exact quotient, ties to even) clamped to [0, top], and Z = 0 when S = 0.  The
// callers pass nlo = -lo >= 0 (a maximum of -w, like hi a maximum of w).
__device__ __forceinline__ uint16_t zp_scale_bits(float nlo, float hi, int top) {
    return f32_to_f16_bits((hi + nlo) / (float)top);
}
__device__ __forceinline__ float zp_zero(float nlo, float s, float topf) {
    return s > 0.f ? round_quot_clamp(nlo, s, __builtin_amdgcn_rcpf(s), 0.f, topf) : 0.f;
}
__device__ __forceinline__ int quant_code_sel(float w, float s, float rs, int qmax) {
    return (int)quant_code_self(w, s, rs, (float)qmax);
}

__device__ __forceinline__ int quant_code_s(float w, float s, int qmax) {
    return s > 0.f ? quant_code(w, s, 1.0f / s, qmax) : 0;
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
// max over aligned groups of `width` lanes (width a power of two <= 64)
__device__ __forceinline__ float group_max(float v, int width) {
    for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float load_as_f32(const void* p, int dtype, int64_t i) {
    // dtype: 0 f32, 1 f16, 2 bf16
    if (dtype == 0) return ((const float*)p)[i];
    if (dtype == 1) return f16_bits_to_f32(((const uint16_t*)p)[i]);
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

}  // namespace pwq
