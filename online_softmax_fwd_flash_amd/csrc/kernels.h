// Host-side launch interface between the C-ABI layer (api.hip) and the kernel translation
// units.  Arguments have been validated before any of these is called.
#pragma once

#include <atomic>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

namespace fa {

constexpr int kMaxDeviceSlots = 64;

// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once per device.  The
// per-device flags are atomics, so host threads making their first calls at the same time do
// not race (the attribute call itself is idempotent; the flag only saves repeating it).
inline hipError_t allow_dynamic_lds(const void* kernel, size_t bytes,
                                    std::atomic<bool>* flags) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDeviceSlots) return hipErrorInvalidDevice;
    if (!flags[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        flags[dev].store(true, std::memory_order_release);
    }
    return hipSuccess;
}

// With the environment variable FA_LOG set to a non-empty value other than "0" (read once per
// process), every launch prints the kernel instantiation it chose and its launch shape to
// stderr.
inline bool log_enabled() {
    static const bool on = [] {
        const char* v = getenv("FA_LOG");
        return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
    }();
    return on;
}

inline void log_launch(const char* kernel, const char* elem, int D, unsigned grid,
                       unsigned block, size_t lds, int B, int T, int Tk, int H, int HKV,
                       int causal, int window) {
    if (!log_enabled()) return;
    fprintf(stderr,
            "flash_attn: %s elem=%s D=%d grid=%u block=%u lds=%zu B=%d T=%d Tk=%d H=%d "
            "HKV=%d causal=%d window=%d\n",
            kernel, elem, D, grid, block, lds, B, T, Tk, H, HKV, causal, window);
}

// Element strides of a [B, T, heads, D] view (batch, row, head); the D axis is contiguous.
// Q, O, dO and dQ share one layout, K, V, dK and dV another.
struct Layout {
    int64_t b, t, h;
};

struct AttnArgs {
    const void* Q;
    const void* K;
    const void* V;
    const void* O;     // forward output / backward input
    void* Oout;        // forward output pointer (same buffer as O in the forward)
    float* L;          // forward output
    const float* Lin;  // backward input
    const void* dO;
    float* Dvec;
    float* dQ;
    float* dK;
    float* dV;
    int B, T, H, HKV, D;   // T: query rows
    int Tk;                 // keys (T unless the two lengths differ)
    float scale;
    int causal, window;
    hipStream_t stream;
    Layout lq, lk;   // query-side and key-side layouts
    int f16;         // 16-bit kernels: 1 = IEEE half elements, 0 = bfloat16
    int g16;         // 16-bit kernels: 1 = dQ, dK, dV stored in the element type, 0 = float32
};

// Tilings of the 16-bit kernels: query rows x keys handled per workgroup block.  Each kernel
// translation unit static_asserts its own constants against these.
constexpr int kB16FwdBq = 128, kB16FwdBk = 32;    // forward: q-tile x staged key block
constexpr int kB16DkdvBq = 32, kB16DkdvBk = 128;  // dK/dV: staged query block x key tile
constexpr int kB16DqBq = 128, kB16DqBk = 64;      // dQ: q-tile x staged key block

bool f32_tiles_supported(int bq, int bk);
hipError_t launch_fwd_f32(const AttnArgs& a, int bq, int bk);
hipError_t launch_dkdv_f32(const AttnArgs& a, int bq, int bk);
hipError_t launch_dq_f32(const AttnArgs& a, int bq, int bk);

// 16-bit (bf16 / fp16 by a.f16) kernels
hipError_t launch_fwd_b16(const AttnArgs& a);
hipError_t launch_dkdv_b16(const AttnArgs& a);
hipError_t launch_dq_b16(const AttnArgs& a);
// dQ that also computes Dvec[b,h,i] = rowsum(dO * O) for its own rows from a.O and writes it
// to a.Dvec (the dK/dV pass launched after it reads those values)
hipError_t launch_dq_b16_fused_d(const AttnArgs& a);

// QK RMS-norm + rotary prologue: qk [tokens, 2*heads, D] with element strides st (token),
// sh (head); float32 factor tables [tokens, D * (paired ? 2 : 1)] with row stride fst;
// out_q / out_k contiguous [tokens, heads, D] ([2*tokens, heads/2, D] when paired).
struct RopeArgs {
    const void* qk;
    int64_t st, sh;
    const float* f1;
    const float* f2;
    int64_t fst;
    void* out_q;
    void* out_k;
    int tokens, heads, D, rotary_dim, paired, key_offset;
    int dtype;   // 0 = f32, 1 = bf16, 2 = fp16
    hipStream_t stream;
};
hipError_t launch_qk_norm_rope(const RopeArgs& a);

// Capacity of the fixed device scratch that flash_attn_bwd_noalloc uses for Dvec, in floats
// (16 MiB per device): B * H * T may not exceed it.
constexpr int64_t kNoAllocDvecFloats = int64_t(1) << 22;

// Device address of the current device's fixed Dvec scratch (at least `floats` floats); looked
// up on the first call per device.  No allocation.  hipErrorInvalidValue if `floats` exceeds
// kNoAllocDvecFloats.
hipError_t noalloc_dvec(size_t floats, float** out);

// MFMA throughput probe: grid workgroups of 256 threads, each wave running iters x 32
// bf16 16x16x32 MFMAs on the 4096 bf16 operand values at ops; out gets grid * 256 floats.
hipError_t launch_mfma_probe(const void* ops, float* out, int grid, int iters,
                             hipStream_t stream);

// dtype: 0 = f32, 1 = bf16, 2 = fp16
hipError_t launch_bwd_preprocess(const void* O, const void* dO, float* Dvec, int B, int T,
                                 int H, int D, int dtype, hipStream_t stream, Layout lq);

}  // namespace fa
