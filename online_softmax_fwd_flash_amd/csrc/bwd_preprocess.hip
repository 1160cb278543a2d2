// Backward stage 1: Dvec[b,h,i] = sum_d dO[b,i,h,d] * O[b,i,h,d] in fp32 — the row dot the
// Graphcore page (flashAttentionQKVPackedGrad) computes as rowsum(O * grad) and the forge page
// ("flash_attention.metal", backward section) passes to its dQ / dK kernels; it equals
// rowsum(dP * P).  Memory-bound: each (b, i, h) row of O and dO is read once with 16-byte
// loads by a team of 8 lanes, reduced across the team with lane exchanges.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

constexpr int kTeam = 8, kThreads = 256;

// fp32 dot of the elements in two 16-byte words: 4 floats, or 8 bf16 / fp16 (dot8)
template <typename E>
__device__ __forceinline__ float dot16B(const u32x4& a, const u32x4& b) {
    return dot8<E>(a, b, 0.f);
}

template <>
__device__ __forceinline__ float dot16B<float>(const u32x4& a, const u32x4& b) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // bit-cast a copied element: casting the vector-element lvalue itself reads element 0
        const uint32_t x = a[i], y = b[i];
        s = fmaf(__builtin_bit_cast(float, x), __builtin_bit_cast(float, y), s);
    }
    return s;
}

// element size in bytes of the I/O type
template <typename E> constexpr int kElemBytes = 2;
template <> constexpr int kElemBytes<float> = 4;

template <typename Elem>
__global__ __launch_bounds__(kThreads) void bwd_preprocess_kernel(
    const void* __restrict__ Ov, const void* __restrict__ dOv, float* __restrict__ Dv, int B,
    int T, int H, int D, Layout lq) {
    constexpr int ES = kElemBytes<Elem>;
    const char* O = static_cast<const char*>(Ov);
    const char* dO = static_cast<const char*>(dOv);
    // row = (b*T + i)*H + h; O and dO of that row start at b*lq.b + i*lq.t + h*lq.h
    const int64_t rows = (int64_t)B * T * H;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / kTeam) + threadIdx.x / kTeam;
    const int sub = threadIdx.x % kTeam;
    const int nch = D * ES / 16;   // 16-byte chunks per row
    const int h = (int)(row % H);
    const int64_t bi = row / H;
    const int i = (int)(bi % T);
    const int64_t b = bi / T;
    float s = 0.f;
    if (row < rows) {
        const int64_t off = (b * lq.b + (int64_t)i * lq.t + (int64_t)h * lq.h) * ES;
        const char* o = O + off;
        const char* go = dO + off;
        for (int ch = sub; ch < nch; ch += kTeam) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(o + ch * 16);
            const u32x4 c = *reinterpret_cast<const u32x4*>(go + ch * 16);
            s += dot16B<Elem>(a, c);
        }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    if (row < rows && sub == 0) Dv[(b * H + h) * T + i] = s;
}

}  // namespace

hipError_t launch_bwd_preprocess(const void* O, const void* dO, float* Dvec, int B, int T, int H,
                                 int D, int dtype, hipStream_t stream, Layout lq) {
    const int64_t rows = (int64_t)B * T * H;
    const int64_t per = kThreads / kTeam;
    const unsigned grid = (unsigned)((rows + per - 1) / per);
    log_launch("bwd_preprocess_kernel", dtype == 0 ? "f32" : dtype == 1 ? "bf16" : "f16", D, grid,
               kThreads, 0, B, T, T, H, H, 0, 0);
    if (dtype == 0)
        hipLaunchKernelGGL(bwd_preprocess_kernel<float>, dim3(grid), dim3(kThreads), 0, stream,
                           O, dO, Dvec, B, T, H, D, lq);
    else if (dtype == 1)
        hipLaunchKernelGGL(bwd_preprocess_kernel<Bf16>, dim3(grid), dim3(kThreads), 0, stream,
                           O, dO, Dvec, B, T, H, D, lq);
    else
        hipLaunchKernelGGL(bwd_preprocess_kernel<F16>, dim3(grid), dim3(kThreads), 0, stream,
                           O, dO, Dvec, B, T, H, D, lq);
    return hipGetLastError();
}

}  // namespace fa
