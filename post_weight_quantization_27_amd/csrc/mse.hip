// Per-layer reconstruction error ("GPT-2 Quantization Reconstruction Error", "What this
// project does", step 5; the layer objective ||WX - What X||^2 of "GPTQ: Post-Training
// INT4", "OBQ Foundation"), with the same calibration X for W and its quantized copy:
//
//   mse = sum_{t, o} (X (W - What)^T)[t, o]^2 / (n_tok * d_out)
//
// One fused pass on the float32 MFMA engine: the B operand loader decodes What from the
// INT4 nibbles (or int8 codes) and scales and forms dW = W - What while staging the tile,
// the epilogue squares and sums the output tile in registers; the product is never
// written.  Per-workgroup partial sums (float64) are added in a fixed order.
#include "gemm_bf16.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// Element (o, c) = W[o][c] - s[o][group(c)] * code[o][c], rows of o with c contiguous.
template <int DTW>
struct OpDeltaW {
    static constexpr int PAD = 1;
    typedef typename Elem<DTW>::T T;
    const T* W;
    int64_t ldw, M, K;          // M = d_out, K = d_in
    const uint8_t* packed;
    const int8_t* codes;
    const uint16_t* scales;
    const int32_t* g_idx;
    int64_t ng;
    int g, vec;                 // vec: aligned W rows, d_in % 4 == 0, one group per quad

    template <int BM>
    struct Regs { float4 v[BM * GEMM_BK / (4 * GEMM_THREADS)]; };

    __device__ __forceinline__ int code(int64_t o, int64_t c) const {
        if (packed) {
            const uint8_t b = packed[o * (K / 2) + c / 2];
            return (int)((c & 1) ? (b >> 4) : (b & 15)) - 8;
        }
        return codes[o * K + c];
    }
    __device__ __forceinline__ float scale(int64_t o, int64_t c) const {
        const int64_t G = g == 0 ? 0 : (g_idx ? (int64_t)g_idx[c] : c / g);
        return f16_bits_to_f32(scales[o * ng + G]);
    }

    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = GEMM_BK / 4;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int mr = idx / PER_ROW, kc = (idx % PER_ROW) * 4;
            const int64_t o = m0 + mr, c = k0 + kc;
            float d[4] = {0.f, 0.f, 0.f, 0.f};
            if (o < M) {
                if (vec && c + 3 < K) {
                    const float4 w = Elem<DTW>::get4(W, o * ldw + c);
                    int q[4];
                    if (packed) {
                        const uint16_t b = *(const uint16_t*)(packed + o * (K / 2) + c / 2);
                        q[0] = (int)(b & 15) - 8; q[1] = (int)((b >> 4) & 15) - 8;
                        q[2] = (int)((b >> 8) & 15) - 8; q[3] = (int)((b >> 12) & 15) - 8;
                    } else {
                        const uint32_t b = *(const uint32_t*)(codes + o * K + c);
                        q[0] = (int8_t)(b & 0xff); q[1] = (int8_t)((b >> 8) & 0xff);
                        q[2] = (int8_t)((b >> 16) & 0xff); q[3] = (int8_t)(b >> 24);
                    }
                    const float s = scale(o, c);
                    d[0] = w.x - s * (float)q[0];
                    d[1] = w.y - s * (float)q[1];
                    d[2] = w.z - s * (float)q[2];
                    d[3] = w.w - s * (float)q[3];
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (c + k < K) d[k] = Elem<DTW>::get(W, o * ldw + c + k) - scale(o, c + k) * (float)code(o, c + k);
                }
            }
            r.v[i] = make_float4(d[0], d[1], d[2], d[3]);
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(float* S, const Regs<BM>& r, int tid) const {
        constexpr int NV = BM * GEMM_BK / (4 * GEMM_THREADS);
        constexpr int PER_ROW = GEMM_BK / 4;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int mr = idx / PER_ROW, kc = (idx % PER_ROW) * 4;
            S[(kc + 0) * (BM + PAD) + mr] = r.v[i].x;
            S[(kc + 1) * (BM + PAD) + mr] = r.v[i].y;
            S[(kc + 2) * (BM + PAD) + mr] = r.v[i].z;
            S[(kc + 3) * (BM + PAD) + mr] = r.v[i].w;
        }
    }
};

// Same dW as OpDeltaW, for the bfloat16 engine: 8 consecutive columns per chunk, each value
// split as hi = bf16(d), lo = bf16(d - hi); both tiles go to LDS (NSPLIT = 2).
template <int DTW>
struct Bf16DeltaWSplit {
    typedef typename Elem<DTW>::T T;
    const T* W;
    int64_t ldw, M, K;
    const uint8_t* packed;
    const int8_t* codes;
    const uint16_t* scales;
    const int32_t* g_idx;
    int64_t ng;
    int g, vec;                      // vec: aligned rows, d_in % 8 == 0, one group per 8 columns

    template <int BM>
    struct Regs { uint4 hi[BM * BK16 / 8 / GEMM_THREADS], lo[BM * BK16 / 8 / GEMM_THREADS]; };

    __device__ __forceinline__ float delta(int64_t o, int64_t c) const {
        int q;
        if (packed) {
            const uint8_t b = packed[o * (K / 2) + c / 2];
            q = (int)((c & 1) ? (b >> 4) : (b & 15)) - 8;
        } else {
            q = codes[o * K + c];
        }
        const int64_t G = g == 0 ? 0 : (g_idx ? (int64_t)g_idx[c] : c / g);
        return Elem<DTW>::get(W, o * ldw + c) - f16_bits_to_f32(scales[o * ng + G]) * (float)q;
    }

    template <int BM>
    __device__ __forceinline__ void load(Regs<BM>& r, int64_t m0, int64_t k0, int tid) const {
        constexpr int NV = BM * BK16 / 8 / GEMM_THREADS;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int row = idx >> 3, kc = (idx & 7) * 8;
            const int64_t o = m0 + row, c = k0 + kc;
            float d[8];
            if (o < M && vec && c + 7 < K) {
                const float4 w0 = Elem<DTW>::get4(W, o * ldw + c), w1 = Elem<DTW>::get4(W, o * ldw + c + 4);
                int q[8];
                if (packed) {
                    const uint32_t b = *(const uint32_t*)(packed + o * (K / 2) + c / 2);
#pragma unroll
                    for (int k = 0; k < 8; ++k) q[k] = (int)((b >> (4 * k)) & 15) - 8;
                } else {
                    const uint2 b = *(const uint2*)(codes + o * K + c);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        q[k] = (int8_t)((b.x >> (8 * k)) & 0xff);
                        q[4 + k] = (int8_t)((b.y >> (8 * k)) & 0xff);
                    }
                }
                const float s = f16_bits_to_f32(scales[o * ng + (g == 0 ? 0 : c / g)]);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) d[k] = wv[k] - s * (float)q[k];
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) d[k] = (o < M && c + k < K) ? delta(o, c + k) : 0.f;
            }
            uint32_t h[4], l[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint16_t h0 = f32_to_bf16_bits(d[2 * k]), h1 = f32_to_bf16_bits(d[2 * k + 1]);
                h[k] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                l[k] = pack_bf16x2(d[2 * k] - bf16_bits_to_f32(h0), d[2 * k + 1] - bf16_bits_to_f32(h1));
            }
            r.hi[i] = make_uint4(h[0], h[1], h[2], h[3]);
            r.lo[i] = make_uint4(l[0], l[1], l[2], l[3]);
        }
    }
    template <int BM>
    __device__ __forceinline__ void store(uint16_t* S, const Regs<BM>& r, int tid) const {
        constexpr int NV = BM * BK16 / 8 / GEMM_THREADS;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = tid + i * GEMM_THREADS;
            const int row = idx >> 3, kc = (idx & 7) * 8;
            *(uint4*)(S + row * LROW + kc) = r.hi[i];
            *(uint4*)(S + BM * LROW + row * LROW + kc) = r.lo[i];
        }
    }
};

// squares of the tile, summed per workgroup into part[blockIdx.x] (float64)
struct EpiSq {
    double* part;
    int64_t M, N;
    float acc;
    __device__ __forceinline__ void element(const Tile&, int64_t row, int64_t col, float v) {
        if (row < M && col < N) acc = fmaf(v, v, acc);
    }
    __device__ __forceinline__ void finish(const Tile&, int tid, bool) {
        __shared__ double red[GEMM_THREADS / 64];
        double d = wave_sum_d((double)acc);
        if ((tid & 63) == 0) red[tid >> 6] = d;
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < GEMM_THREADS / 64; ++w) s += red[w];
            part[blockIdx.x] = s;
        }
    }
};

__global__ __launch_bounds__(256) void mse_final_kernel(const double* __restrict__ part, int64_t nparts, double denom,
                                                        double* __restrict__ mse) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < nparts; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) *mse = red[0] / denom;
}

__global__ void set_double_kernel(double* p, double v) { *p = v; }

inline int mse_bm(int64_t n_tok, int64_t d_out) { return cdiv(n_tok, 128) * cdiv(d_out, 128) >= 512 ? 128 : 64; }

template <int BM, int DTX, int DTW>
hipError_t mse_gemm(const void* X, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W, int64_t ldw,
                    const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx, int64_t d_out,
                    int group_size, double* part, hipStream_t s, int64_t* nblocks) {
    typedef typename Elem<DTX>::T TX;
    typedef typename Elem<DTW>::T TW;
    OpMMajor<DTX> a{(const TX*)X, ldx, n_tok, d_in, (int)((ldx % 4 == 0) && aligned(X, 4 * sizeof(TX)))};
    OpDeltaW<DTW> b{};
    b.W = (const TW*)W; b.ldw = ldw; b.M = d_out; b.K = d_in;
    b.packed = packed; b.codes = codes; b.scales = scales; b.g_idx = g_idx;
    b.ng = group_size == 0 ? 1 : cdiv(d_in, group_size);
    b.g = group_size;
    b.vec = (ldw % 4 == 0) && (d_in % 4 == 0) && aligned(W, 4 * sizeof(TW)) && !g_idx &&
            (group_size == 0 || group_size % 4 == 0) && (!packed || aligned(packed, 2)) && (!codes || aligned(codes, 4));
    RectMap mp{};
    mp.M = n_tok; mp.N = d_out; mp.K = d_in;
    mp.tiles_m = (int)cdiv(n_tok, BM);
    mp.tiles_n = (int)cdiv(d_out, BM);
    mp.splits = 1;
    mp.kchunk = cdiv(d_in, GEMM_BK) * GEMM_BK;
    mp.tri_k = 0;
    mp.guard = nullptr;
    EpiSq ep{part, n_tok, d_out, 0.f};
    *nblocks = (int64_t)mp.tiles_m * mp.tiles_n;
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BM, OpMMajor<DTX>, OpDeltaW<DTW>, RectMap, EpiSq>), dim3((unsigned)*nblocks),
                       dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

// bfloat16 X: X is exact in bf16, dW rides as a bf16 hi + lo pair (two MFMAs per step)
template <int DTW>
hipError_t mse_gemm_bf16(const void* X, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W, int64_t ldw,
                         const uint8_t* packed, const int8_t* codes, const uint16_t* scales, const int32_t* g_idx,
                         int64_t d_out, int group_size, double* part, hipStream_t s, int64_t* nblocks) {
    typedef typename Elem<DTW>::T TW;
    Bf16MMajor a{(const uint16_t*)X, ldx, n_tok, d_in, (int)((ldx % 8 == 0) && aligned(X, 16))};
    Bf16DeltaWSplit<DTW> b{};
    b.W = (const TW*)W; b.ldw = ldw; b.M = d_out; b.K = d_in;
    b.packed = packed; b.codes = codes; b.scales = scales; b.g_idx = g_idx;
    b.ng = group_size == 0 ? 1 : cdiv(d_in, group_size);
    b.g = group_size;
    b.vec = (ldw % 8 == 0) && (d_in % 8 == 0) && aligned(W, 8 * sizeof(TW)) && !g_idx &&
            (group_size == 0 || group_size % 8 == 0) && (!packed || aligned(packed, 4)) && (!codes || aligned(codes, 8));
    RectMap mp{};
    mp.M = n_tok; mp.N = d_out; mp.K = d_in;
    mp.tiles_m = (int)cdiv(n_tok, 128);
    mp.tiles_n = (int)cdiv(d_out, 128);
    mp.splits = 1;
    mp.kchunk = cdiv(d_in, BK16) * BK16;
    mp.tri_k = 0;
    mp.guard = nullptr;
    EpiSq ep{part, n_tok, d_out, 0.f};
    *nblocks = (int64_t)mp.tiles_m * mp.tiles_n;
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, Bf16MMajor, Bf16DeltaWSplit<DTW>, RectMap, EpiSq>),
                       dim3((unsigned)*nblocks), dim3(GEMM_THREADS), 0, s, a, b, mp, ep);
    return hipGetLastError();
}

template <int BM>
hipError_t mse_dispatch(int x_dtype, int w_dtype, const void* X, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W,
                        int64_t ldw, const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                        const int32_t* g_idx, int64_t d_out, int group_size, double* part, hipStream_t s, int64_t* nb) {
    if (x_dtype == 0 && w_dtype == 0)
        return mse_gemm<BM, 0, 0>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, nb);
    if (x_dtype == 0)
        return mse_gemm<BM, 0, 1>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, nb);
    if (w_dtype == 0)
        return mse_gemm<BM, 2, 0>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, nb);
    return mse_gemm<BM, 2, 1>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, nb);
}

}  // namespace

size_t mse_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out) {
    (void)d_in;
    const int bm = mse_bm(n_tok, d_out);
    const int64_t nf = cdiv(n_tok, bm) * cdiv(d_out, bm), nb = cdiv(n_tok, 128) * cdiv(d_out, 128);
    return (size_t)(nf > nb ? nf : nb) * sizeof(double);
}

hipError_t mse_launch(const void* X, int x_dtype, int64_t n_tok, int64_t d_in, int64_t ldx, const void* W, int w_dtype,
                      int64_t ldw, const uint8_t* packed, const int8_t* codes, const uint16_t* scales,
                      const int32_t* g_idx, int64_t d_out, int bits, int group_size, double* mse, void* ws, hipStream_t s) {
    (void)bits;
    hipError_t e;
    if (n_tok == 0 || d_out == 0) {
        hipLaunchKernelGGL(set_double_kernel, dim3(1), dim3(1), 0, s, mse, 0.0);
        return hipGetLastError();
    }
    double* part = (double*)ws;
    int64_t nb = 0;
    if (x_dtype == 2)
        e = w_dtype == 0 ? mse_gemm_bf16<0>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, &nb)
                         : mse_gemm_bf16<1>(X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, &nb);
    else if (mse_bm(n_tok, d_out) == 128)
        e = mse_dispatch<128>(x_dtype, w_dtype, X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, &nb);
    else
        e = mse_dispatch<64>(x_dtype, w_dtype, X, n_tok, d_in, ldx, W, ldw, packed, codes, scales, g_idx, d_out, group_size, part, s, &nb);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(256), 0, s, part, nb, (double)n_tok * (double)d_out, mse);
    return hipGetLastError();
}

}  // namespace pwq
