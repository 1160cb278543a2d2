// QK RMS-norm + rotary prologue for gfx950: from one packed QK projection
// [tokens, 2 * heads, D] (query heads first) to the separate Q and K tensors attention reads.
//
// Method (prior art, other hardware): modded-nanogpt "qkv_rope.py", the module docstring and
// qk_norm_rope_forward with its forward kernel: each (token, input head) row is normalised
// in fp32 by rsqrt(mean(x^2) + 2^-23) with no weight, mixed with its pair-swapped copy
// through per-token factor tables (y = factor1 * x + factor2 * swap(x)), optionally remapped
// to paired heads (token 2t + h / (heads/2), head h % (heads/2), second table half for odd
// h) or given the previous token's normalised stationary elements (key offset, keys only).
//
// gfx950 design: pure streaming (a few FLOPs per byte), so the kernel is shaped for HBM and
// L2, not for MFMA.  Each lane moves one 16-byte chunk of a row (8 bf16 / fp16 or 4 fp32
// elements); the D / 8 (D / 4) lanes of a row are consecutive, so a wave's loads and stores
// cover whole rows and consecutive rows are consecutive heads of one token (contiguous in
// the usual packed projection).  The sum of squares is reduced across the row's lanes with
// xor shuffles; the pair swap never leaves the lane (chunks start on even elements).  The
// factor tables are per token and shared by all 2 * heads rows of it, so they are read
// through L2 about once per token.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

constexpr int kRopeThreads = 256;
constexpr float kRmsEps = 1.1920928955078125e-7f;   // 2^-23

// Element access for one 16-byte chunk: EPL elements, to and from float.
template <class E>
struct Chunk16 {
    static constexpr int EPL = 8;
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const typename E::v8 v = *reinterpret_cast<const typename E::v8*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const typename E::s xe = v[e];
            x[e] = (float)xe;
        }
    }
    static __device__ __forceinline__ void store(void* p, const float* y) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack2<E>(y[2 * i], y[2 * i + 1]);
        *reinterpret_cast<u32x4*>(p) = w;
    }
};

template <>
struct Chunk16<float> {
    static constexpr int EPL = 4;
    static __device__ __forceinline__ void load(const void* p, float* x) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
    static __device__ __forceinline__ void store(void* p, const float* y) {
        *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
    }
};

template <class E> constexpr int kElemSize = 2;
template <> constexpr int kElemSize<float> = 4;

// sum over the LPR consecutive lanes of a row (LPR a power of two)
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <class E, int D>
__global__ __launch_bounds__(kRopeThreads) void qk_norm_rope_kernel(
    const char* __restrict__ qk, int64_t st, int64_t sh, const float* __restrict__ f1,
    const float* __restrict__ f2, int64_t fst, char* __restrict__ out_q,
    char* __restrict__ out_k, int tokens, int heads, int rotary_dim, int paired,
    int key_offset) {
    using CK = Chunk16<E>;
    constexpr int EPL = CK::EPL, LPR = D / EPL, ES = kElemSize<E>;
    const int heads2 = 2 * heads;
    const int64_t rows = (int64_t)tokens * heads2;
    const int64_t row = ((int64_t)blockIdx.x * kRopeThreads + threadIdx.x) / LPR;
    const int c = threadIdx.x % LPR;   // chunk of the row this lane moves
    const bool live = row < rows;
    const int t = live ? (int)(row / heads2) : 0;
    const int ih = live ? (int)(row % heads2) : 0;
    const int d0 = c * EPL;

    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = 0.f;
    if (live) CK::load(qk + ((int64_t)t * st + (int64_t)ih * sh + d0) * ES, x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
    const float rstd = rsqrtf(row_sum<LPR>(ss) * (1.f / D) + kRmsEps);

    const int lh = ih % heads;
    int ot = t, oh = lh, off = 0;
    if (paired) {
        ot = 2 * t + lh / (heads / 2);
        oh = lh % (heads / 2);
        off = (lh % 2) * D;
    }
    float y[EPL];
    if (live) {
        const f32x4* p1 = reinterpret_cast<const f32x4*>(f1 + (int64_t)t * fst + off + d0);
        const f32x4* p2 = reinterpret_cast<const f32x4*>(f2 + (int64_t)t * fst + off + d0);
#pragma unroll
        for (int q4 = 0; q4 < EPL / 4; ++q4) {
            const f32x4 a = p1[q4], b = p2[q4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * q4 + e;
                // pair partner of element i: i ^ 1 (pairs start on even elements)
                y[i] = a[e] * (x[i] * rstd) + b[e] * (x[i ^ 1] * rstd);
            }
        }
    }
    if (key_offset) {
        // keys of tokens after the first: the stationary elements (index >= rotary_dim) are
        // the previous token's normalised row
        const bool shift = live && ih >= heads && t > 0;
        float xp[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) xp[e] = 0.f;
        if (shift) CK::load(qk + ((int64_t)(t - 1) * st + (int64_t)ih * sh + d0) * ES, xp);
        float sp = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sp = fmaf(xp[e], xp[e], sp);
        const float rp = rsqrtf(row_sum<LPR>(sp) * (1.f / D) + kRmsEps);
        if (shift) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                if (d0 + e >= rotary_dim) y[e] = xp[e] * rp;
        }
    }
    if (!live) return;
    const int oheads = paired ? heads / 2 : heads;
    char* out = ih < heads ? out_q : out_k;
    CK::store(out + (((int64_t)ot * oheads + oh) * D + d0) * ES, y);
}

template <class E, int D>
hipError_t launch_rope_t(const RopeArgs& a) {
    constexpr int LPR = D / Chunk16<E>::EPL;
    static_assert(LPR >= 1 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row must fit a wave");
    const int64_t rows = (int64_t)a.tokens * 2 * a.heads;
    const int64_t threads = rows * LPR;
    const unsigned grid = (unsigned)((threads + kRopeThreads - 1) / kRopeThreads);
    log_launch("qk_norm_rope_kernel", a.dtype == 0 ? "f32" : a.dtype == 1 ? "bf16" : "f16", D,
               grid, kRopeThreads, 0, 1, a.tokens, a.tokens, a.heads, a.heads, 0, 0);
    hipLaunchKernelGGL((qk_norm_rope_kernel<E, D>), dim3(grid), dim3(kRopeThreads), 0, a.stream,
                       (const char*)a.qk, a.st, a.sh, a.f1, a.f2, a.fst, (char*)a.out_q,
                       (char*)a.out_k, a.tokens, a.heads, a.rotary_dim, a.paired, a.key_offset);
    return hipGetLastError();
}

template <class E>
hipError_t launch_rope_e(const RopeArgs& a) {
    switch (a.D) {
        case 16: return launch_rope_t<E, 16>(a);
        case 32: return launch_rope_t<E, 32>(a);
        case 64: return launch_rope_t<E, 64>(a);
        case 128: return launch_rope_t<E, 128>(a);
        case 256: return launch_rope_t<E, 256>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qk_norm_rope(const RopeArgs& a) {
    if (a.dtype == 0) return launch_rope_e<float>(a);
    if (a.dtype == 1) return launch_rope_e<Bf16>(a);
    return launch_rope_e<F16>(a);
}

}  // namespace fa
