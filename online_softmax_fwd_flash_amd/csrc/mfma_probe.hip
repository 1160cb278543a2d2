// MFMA throughput probe: a loop of independent bf16 16x16x32 MFMAs (the shape every 16-bit
// attention kernel here uses) on operands the caller supplies, to measure the matrix rate the
// chip sustains on a given operand distribution (the rate depends on the data: the chip runs
// under a power limit, and operand bits that toggle cost power).  Only the MFMAs run inside
// the loop; the operands are loaded once.
//
// Each wave keeps NACC independent accumulators (so the MFMA pipe always has independent work)
// and cycles through NOP operand pairs, so consecutive MFMAs see different values.
#include "common.h"
#include "kernels.h"

namespace fa {

namespace {

constexpr int kProbeThreads = 256;   // 4 waves, one per SIMD of a CU
constexpr int kProbeWgs = 2;         // workgroups per CU: 2 waves per SIMD
constexpr int kNacc = 8;             // independent accumulators per wave
constexpr int kNop = 4;              // operand pairs per lane

}  // namespace

__global__ __launch_bounds__(kProbeThreads, kProbeWgs) void mfma_probe_kernel(
    const uint16_t* __restrict__ ops, float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    // lane l's fragments: A_i = ops[(i * 64 + l) * 8 .. +7], B_i = ops[((kNop + i) * 64 + l) * 8 ..]
    bf16x8 a[kNop], b[kNop];
#pragma unroll
    for (int i = 0; i < kNop; ++i) {
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ops + (i * 64 + lane) * 8));
        b[i] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const u32x4*>(ops + ((kNop + i) * 64 + lane) * 8));
    }
    f32x4 acc[kNacc];
#pragma unroll
    for (int c = 0; c < kNacc; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[c][r] = 0.f;
    // kNop * kNacc = 32 MFMAs per iteration, each operand pair used by several accumulators
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kNop; ++i)
#pragma unroll
            for (int c = 0; c < kNacc; ++c)
                acc[c] = mfma16x16x32(a[(i + c) % kNop], b[(i + 2 * c + c / kNop) % kNop], acc[c]);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kNacc; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += acc[c][r];
    out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(const void* ops, float* out, int grid, int iters,
                             hipStream_t stream) {
    log_launch("mfma_probe_kernel", "bf16", 0, (unsigned)grid, kProbeThreads, 0, 0, 0, 0, 0, 0,
               0, 0);
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                       (const uint16_t*)ops, out, iters);
    return hipGetLastError();
}

}  // namespace fa
