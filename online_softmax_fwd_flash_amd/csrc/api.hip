// C-ABI layer: argument validation, tiling choice and dispatch to the kernel launchers.
// Nothing is enqueued unless every argument is valid.  See include/flash_attn.h.
#include <math.h>
#include <stdint.h>

#include "flash_attn.h"
#include "block_class.h"
#include "kernels.h"

namespace {

constexpr int kF32DefaultBq = 64, kF32DefaultBk = 64;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fa_status_t check_dims(int B, int T, int H, int HKV, int D, float scale, int causal, int window,
                       fa_dtype_t dtype) {
    if (B < 1 || T < 1 || H < 1 || HKV < 1 || D < 1) return FA_ERR_INVALID_ARG;
    if (H % HKV != 0) return FA_ERR_INVALID_ARG;
    if (window < 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    // every element offset and every grid stays far inside its integer type
    const double elems = (double)B * T * H * D;
    if (elems > (double)(1ll << 40)) return FA_ERR_INVALID_ARG;
    if ((double)B * H * ((T + 15) / 16) > 2147483647.0) return FA_ERR_INVALID_ARG;
    if (dtype == FA_DTYPE_F32) {
        if (D % 8 != 0 || D > 128) return FA_ERR_UNSUPPORTED;
    } else {
        if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
        // the bf16 kernels address one batch slice of a tensor with 32-bit buffer offsets
        if ((double)T * (H > HKV ? H : HKV) * D * 2.0 >= 2147483648.0) return FA_ERR_INVALID_ARG;
    }
    return FA_OK;
}

fa_status_t check_ptrs(std::initializer_list<const void*> ps) {
    for (const void* p : ps) {
        if (p == nullptr) return FA_ERR_INVALID_ARG;
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    }
    return FA_OK;
}

fa_status_t resolve_f32_tiles(int& bq, int& bk) {
    if (bq == 0 && bk == 0) {
        bq = kF32DefaultBq;
        bk = kF32DefaultBk;
    }
    return fa::f32_tiles_supported(bq, bk) ? FA_OK : FA_ERR_INVALID_ARG;
}

fa_status_t hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

fa::AttnArgs make_args(int B, int T, int H, int HKV, int D, float scale, int causal, int window,
                       hipStream_t stream) {
    fa::AttnArgs a{};
    a.B = B; a.T = T; a.H = H; a.HKV = HKV; a.D = D;
    a.scale = scale; a.causal = causal; a.window = window; a.stream = stream;
    return a;
}

}  // namespace

extern "C" {

const char* flash_attn_status_string(fa_status_t s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_UNKNOWN_STATUS";
}

int flash_attn_version(void) { return 100; }

int flash_attn_block_class(int T, int bq, int bk, int causal, int window, int i, int j, int* off) {
    if (T < 1 || bq < 1 || bk < 1 || window < 0 || i < 0 || j < 0) return -1;
    if ((long long)(i + 1) * bq > (1ll << 30) || (long long)(j + 1) * bk > (1ll << 30)) return -1;
    if (off) *off = i * bq - j * bk;
    return fa::block_class(T, i * bq, i * bq + bq, j * bk, j * bk + bk, causal != 0, window);
}

fa_status_t flash_attn_kv_block_range(int T, int bq, int bk, int causal, int window, int i,
                                      int* j_lo, int* j_hi) {
    if (T < 1 || bq < 1 || bk < 1 || window < 0 || i < 0 || !j_lo || !j_hi)
        return FA_ERR_INVALID_ARG;
    if ((long long)(i + 1) * bq > (1ll << 30)) return FA_ERR_INVALID_ARG;
    fa::kv_block_range(T, i * bq, i * bq + bq, bk, causal != 0, window, *j_lo, *j_hi);
    return FA_OK;
}

fa_status_t flash_attn_default_tiles(fa_dtype_t dtype, int D, int pass, int* bq, int* bk) {
    if (!bq || !bk || pass < 0 || pass > 2) return FA_ERR_INVALID_ARG;
    if (dtype == FA_DTYPE_F32) {
        if (D < 8 || D > 128 || D % 8) return FA_ERR_UNSUPPORTED;
        *bq = kF32DefaultBq;
        *bk = kF32DefaultBk;
        return FA_OK;
    }
    if (dtype != FA_DTYPE_BF16) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    const int tq[3] = {fa::kBf16FwdBq, fa::kBf16DkdvBq, fa::kBf16DqBq};
    const int tk[3] = {fa::kBf16FwdBk, fa::kBf16DkdvBk, fa::kBf16DqBk};
    *bq = tq[pass];
    *bk = tk[pass];
    return FA_OK;
}

fa_status_t flash_attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* L,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    fa_status_t s = check_ptrs({Q, K, V, O, L});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype)) != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, H, HKV, D, scale, causal, window, stream);
    a.Q = Q; a.K = K; a.V = V; a.Oout = O; a.O = O; a.L = L;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_fwd_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kBf16FwdBq && bk == fa::kBf16FwdBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_fwd_bf16(a));
}

fa_status_t flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B,
                           int T, int H, int HKV, int D, float scale, int causal, int window,
                           fa_dtype_t dtype, hipStream_t stream) {
    return flash_attn_fwd_ex(Q, K, V, O, L, B, T, H, HKV, D, scale, causal, window, dtype, stream,
                             0, 0);
}

fa_status_t flash_attn_bwd_preprocess(const void* O, const void* dO, float* Dvec, int B, int T,
                                      int H, int D, fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t s = check_ptrs({O, dO, Dvec});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, H, D, 1.0f, 0, 0, dtype)) != FA_OK) return s;
    return hip_status(fa::launch_bwd_preprocess(O, dO, Dvec, B, T, H, D,
                                                dtype == FA_DTYPE_F32 ? 0 : 1, stream));
}

fa_status_t flash_attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dvec, float* dK, float* dV, int B,
                                int T, int H, int HKV, int D, float scale, int causal, int window,
                                fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    fa_status_t s = check_ptrs({Q, K, V, dO, L, Dvec, dK, dV});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype)) != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, H, HKV, D, scale, causal, window, stream);
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.Lin = L; a.Dvec = const_cast<float*>(Dvec);
    a.dK = dK; a.dV = dV;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_dkdv_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kBf16DkdvBq && bk == fa::kBf16DkdvBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_dkdv_bf16(a));
}

fa_status_t flash_attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                              const float* L, const float* Dvec, float* dQ, int B, int T, int H,
                              int HKV, int D, float scale, int causal, int window,
                              fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    fa_status_t s = check_ptrs({Q, K, V, dO, L, Dvec, dQ});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype)) != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, H, HKV, D, scale, causal, window, stream);
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.Lin = L; a.Dvec = const_cast<float*>(Dvec);
    a.dQ = dQ;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_dq_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kBf16DqBq && bk == fa::kBf16DqBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_dq_bf16(a));
}

fa_status_t flash_attn_bwd_dq_dvec(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* L, float* Dvec, float* dQ, int B,
                                   int T, int H, int HKV, int D, float scale, int causal,
                                   int window, fa_dtype_t dtype, hipStream_t stream, int bq,
                                   int bk) {
    fa_status_t s = check_ptrs({Q, K, V, O, dO, L, Dvec, dQ});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype)) != FA_OK) return s;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        s = flash_attn_bwd_preprocess(O, dO, Dvec, B, T, H, D, dtype, stream);
        if (s != FA_OK) return s;
        return flash_attn_bwd_dq(Q, K, V, dO, L, Dvec, dQ, B, T, H, HKV, D, scale, causal,
                                 window, dtype, stream, bq, bk);
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kBf16DqBq && bk == fa::kBf16DqBk)))
        return FA_ERR_INVALID_ARG;
    fa::AttnArgs a = make_args(B, T, H, HKV, D, scale, causal, window, stream);
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.Lin = L; a.Dvec = Dvec; a.dQ = dQ;
    return hip_status(fa::launch_dq_bf16_fused_d(a));
}

fa_status_t flash_attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O,
                              const float* L, const void* dO, float* dQ, float* dK, float* dV,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    fa_status_t s = check_ptrs({Q, K, V, O, L, dO, dQ, dK, dV});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype)) != FA_OK) return s;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
    } else if (!(bq == 0 && bk == 0)) {
        return FA_ERR_INVALID_ARG;
    }
    float* Dvec = nullptr;
    const size_t bytes = (size_t)B * H * T * sizeof(float);
    if (hipMallocAsync((void**)&Dvec, bytes, stream) != hipSuccess) return FA_ERR_HIP;
    s = flash_attn_bwd_dq_dvec(Q, K, V, O, dO, L, Dvec, dQ, B, T, H, HKV, D, scale, causal,
                               window, dtype, stream, bq, bk);
    if (s == FA_OK)
        s = flash_attn_bwd_dkdv(Q, K, V, dO, L, Dvec, dK, dV, B, T, H, HKV, D, scale, causal,
                                window, dtype, stream, bq, bk);
    const hipError_t fe = hipFreeAsync(Dvec, stream);
    if (s == FA_OK && fe != hipSuccess) s = FA_ERR_HIP;
    return s;
}

fa_status_t flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                           const float* L, const void* dO, float* dQ, float* dK, float* dV, int B,
                           int T, int H, int HKV, int D, float scale, int causal, int window,
                           fa_dtype_t dtype, hipStream_t stream) {
    return flash_attn_bwd_ex(Q, K, V, O, L, dO, dQ, dK, dV, B, T, H, HKV, D, scale, causal,
                             window, dtype, stream, 0, 0);
}

}  // extern "C"
