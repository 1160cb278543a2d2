// C-ABI layer: argument validation, tiling choice and dispatch to the kernel launchers.
// Nothing is enqueued unless every argument is valid.  See include/flash_attn.h.
#include <math.h>
#include <stdint.h>

#include "flash_attn.h"
#include "block_class.h"
#include "kernels.h"
#include "workspace.h"

namespace {

constexpr int kF32DefaultBq = 64, kF32DefaultBk = 64;
// Longest query or key sequence: row and block indices (plus a tile) stay far inside int.
constexpr int kMaxRows = 1 << 30;
static_assert(FA_NOALLOC_MAX_DVEC == fa::kNoAllocDvecFloats, "no-alloc scratch size differs");

// A window of at least Tk keys constrains no row (row positions are below Tk), so it is the
// same as no window; the kernels and helpers take it as 0, which keeps their index arithmetic
// (row + window) inside int.
int effective_window(int window, int Tk) { return window >= Tk ? 0 : window; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

fa_status_t check_dims(int B, int T, int H, int HKV, int D, float scale, int causal, int window,
                       fa_dtype_t dtype, int Tk = -1) {
    if (Tk < 0) Tk = T;
    if (B < 1 || T < 1 || Tk < 1 || H < 1 || HKV < 1 || D < 1) return FA_ERR_INVALID_ARG;
    if (T > kMaxRows || Tk > kMaxRows) return FA_ERR_INVALID_ARG;
    if (H % HKV != 0) return FA_ERR_INVALID_ARG;
    if (window < 0 || (causal != 0 && causal != 1)) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    // every element offset and every grid stays far inside its integer type
    const double elems = (double)B * (T > Tk ? T : Tk) * H * D;
    if (elems > (double)(1ll << 40)) return FA_ERR_INVALID_ARG;
    if ((double)B * H * (((int64_t)(T > Tk ? T : Tk) + 15) / 16) > 2147483647.0)
        return FA_ERR_INVALID_ARG;
    if (dtype == FA_DTYPE_F32) {
        if (D % 8 != 0 || D > 128) return FA_ERR_UNSUPPORTED;
    } else {
        if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    }
    return FA_OK;
}

// A [B, T, heads, D] view with element strides l (D contiguous) that the kernels can use:
// strides non-negative and multiples of 16 bytes (every row starts 16-byte aligned), rows at
// least D apart (so a head's rows end before row T begins: the bf16 kernels read rows past T
// as zeros), distinct (b, t, h) never overlap, and, for bf16, one head's T rows (plus the
// staging tiles' overhang) span less than 2 GiB (32-bit buffer offsets within a head).
fa_status_t check_layout(const fa_layout_t& l, int B, int T, int heads, int D, fa_dtype_t dtype) {
    const int64_t esz = dtype == FA_DTYPE_F32 ? 4 : 2, align = 16 / esz;
    const int64_t st[3] = {l.row, l.head, l.batch};
    const int64_t ext[3] = {T, heads, B};
    for (int i = 0; i < 3; ++i) {
        if (st[i] < 0) return FA_ERR_INVALID_ARG;
        // the row stride is used even when T = 1 (for the rows past T the kernels read as zeros)
        if ((i == 0 || ext[i] > 1) && st[i] % align != 0) return FA_ERR_INVALID_ARG;
    }
    if (l.row < D) return FA_ERR_INVALID_ARG;
    // non-overlap: order the axes of extent > 1 by stride; each must step past the block the
    // smaller ones span (the innermost block is the D contiguous elements)
    int idx[3], n = 0;
    for (int i = 0; i < 3; ++i)
        if (ext[i] > 1) idx[n++] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && st[idx[j]] < st[idx[j - 1]]; --j) {
            const int t = idx[j]; idx[j] = idx[j - 1]; idx[j - 1] = t;
        }
    double span = D;
    for (int i = 0; i < n; ++i) {
        if ((double)st[idx[i]] < span) return FA_ERR_INVALID_ARG;
        span = (double)st[idx[i]] * (double)ext[idx[i]];
    }
    if (span * esz > 9.0e18) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && ((double)(T - 1) * l.row + D + 128.0 * l.row) * esz >= 2147483648.0)
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// a * b, saturated at INT64_MAX (the sizes are not validated yet when the layouts of the
// contiguous entry points are formed; a saturated stride fails the layout check)
int64_t sat_mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

// The layouts of contiguous [B, T, H, D] (queries) and [B, T, HKV, D] (keys) tensors.
fa_layout_t dense_layout(int T, int heads, int D) {
    fa_layout_t l;
    l.batch = sat_mul(sat_mul(T, heads), D);
    l.row = sat_mul(heads, D);
    l.head = D;
    return l;
}

fa::Layout to_layout(const fa_layout_t& l) { return fa::Layout{l.batch, l.row, l.head}; }

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

fa::AttnArgs make_args(int B, int T, int Tk, int H, int HKV, int D, float scale, int causal, int window,
                       hipStream_t stream, const fa_layout_t& lq, const fa_layout_t& lk,
                       fa_dtype_t dtype) {
    fa::AttnArgs a{};
    a.f16 = dtype == FA_DTYPE_F16 ? 1 : 0;
    a.B = B; a.T = T; a.Tk = Tk; a.H = H; a.HKV = HKV; a.D = D;
    a.scale = scale; a.causal = causal; a.window = effective_window(window, Tk);
    a.stream = stream;
    a.lq = to_layout(lq); a.lk = to_layout(lk);
    return a;
}

// Shared validation of the attention entry points: pointers, sizes and both layouts.
fa_status_t check_all(std::initializer_list<const void*> ps, int B, int T, int Tk, int H, int HKV,
                      int D,
                      float scale, int causal, int window, fa_dtype_t dtype,
                      const fa_layout_t& lq, const fa_layout_t& lk) {
    fa_status_t s = check_ptrs(ps);
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, HKV, D, scale, causal, window, dtype, Tk)) != FA_OK) return s;
    if ((s = check_layout(lq, B, T, H, D, dtype)) != FA_OK) return s;
    return check_layout(lk, B, Tk, HKV, D, dtype);
}

fa_status_t fwd_impl(const void* Q, const void* K, const void* V, void* O, float* L, int B, int T, int Tk,
                     int H, int HKV, int D, float scale, int causal, int window,
                     fa_dtype_t dtype, hipStream_t stream, int bq, int bk,
                     const fa_layout_t& lq, const fa_layout_t& lk) {
    fa_status_t s = check_all({Q, K, V, O, L}, B, T, Tk, H, HKV, D, scale, causal, window, dtype, lq, lk);
    if (s != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, Tk, H, HKV, D, scale, causal, window, stream, lq, lk, dtype);
    a.Q = Q; a.K = K; a.V = V; a.Oout = O; a.O = O; a.L = L;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_fwd_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kB16FwdBq && bk == fa::kB16FwdBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_fwd_b16(a));
}

fa_status_t preprocess_impl(const void* O, const void* dO, float* Dvec, int B, int T, int H,
                            int D, fa_dtype_t dtype, hipStream_t stream, const fa_layout_t& lq) {
    fa_status_t s = check_ptrs({O, dO, Dvec});
    if (s != FA_OK) return s;
    if ((s = check_dims(B, T, H, H, D, 1.0f, 0, 0, dtype)) != FA_OK) return s;
    if ((s = check_layout(lq, B, T, H, D, dtype)) != FA_OK) return s;
    return hip_status(fa::launch_bwd_preprocess(O, dO, Dvec, B, T, H, D,
                                                dtype == FA_DTYPE_F32 ? 0 : dtype == FA_DTYPE_BF16 ? 1 : 2, stream,
                                                to_layout(lq)));
}

fa_status_t dkdv_impl(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                      const float* Dvec, float* dK, float* dV, int B, int T, int Tk, int H, int HKV,
                      int D, float scale, int causal, int window, fa_dtype_t dtype,
                      hipStream_t stream, int bq, int bk, const fa_layout_t& lq,
                      const fa_layout_t& lk, int g16 = 0) {
    fa_status_t s = check_all({Q, K, V, dO, L, Dvec, dK, dV}, B, T, Tk, H, HKV, D, scale, causal,
                              window, dtype, lq, lk);
    if (s != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, Tk, H, HKV, D, scale, causal, window, stream, lq, lk, dtype);
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.Lin = L; a.Dvec = const_cast<float*>(Dvec);
    a.dK = dK; a.dV = dV; a.g16 = g16;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_dkdv_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kB16DkdvBq && bk == fa::kB16DkdvBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_dkdv_b16(a));
}

fa_status_t dq_impl(const void* Q, const void* K, const void* V, const void* dO, const float* L,
                    const float* Dvec, float* dQ, int B, int T, int Tk, int H, int HKV, int D,
                    float scale, int causal, int window, fa_dtype_t dtype, hipStream_t stream,
                    int bq, int bk, const fa_layout_t& lq, const fa_layout_t& lk) {
    fa_status_t s = check_all({Q, K, V, dO, L, Dvec, dQ}, B, T, Tk, H, HKV, D, scale, causal, window,
                              dtype, lq, lk);
    if (s != FA_OK) return s;
    fa::AttnArgs a = make_args(B, T, Tk, H, HKV, D, scale, causal, window, stream, lq, lk, dtype);
    a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.Lin = L; a.Dvec = const_cast<float*>(Dvec);
    a.dQ = dQ;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        return hip_status(fa::launch_dq_f32(a, bq, bk));
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kB16DqBq && bk == fa::kB16DqBk)))
        return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_dq_b16(a));
}

fa_status_t dq_dvec_impl(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* L, float* Dvec, float* dQ, int B, int T, int Tk,
                         int H, int HKV, int D, float scale, int causal, int window,
                         fa_dtype_t dtype, hipStream_t stream, int bq, int bk,
                         const fa_layout_t& lq, const fa_layout_t& lk, int g16 = 0) {
    fa_status_t s = check_all({Q, K, V, O, dO, L, Dvec, dQ}, B, T, Tk, H, HKV, D, scale, causal,
                              window, dtype, lq, lk);
    if (s != FA_OK) return s;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
        s = preprocess_impl(O, dO, Dvec, B, T, H, D, dtype, stream, lq);
        if (s != FA_OK) return s;
        return dq_impl(Q, K, V, dO, L, Dvec, dQ, B, T, Tk, H, HKV, D, scale, causal, window, dtype,
                       stream, bq, bk, lq, lk);
    }
    if (!((bq == 0 && bk == 0) || (bq == fa::kB16DqBq && bk == fa::kB16DqBk)))
        return FA_ERR_INVALID_ARG;
    fa::AttnArgs a = make_args(B, T, Tk, H, HKV, D, scale, causal, window, stream, lq, lk, dtype);
    a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.Lin = L; a.Dvec = Dvec; a.dQ = dQ;
    a.g16 = g16;
    return hip_status(fa::launch_dq_b16_fused_d(a));
}

// Where the backward's Dvec workspace comes from: the library's per-device workspace cache
// (allocates on first use and on growth only), or its fixed per-device scratch (never
// allocates).
enum class Workspace { kCached, kFixedScratch };

fa_status_t bwd_impl(const void* Q, const void* K, const void* V, const void* O, const float* L,
                     const void* dO, float* dQ, float* dK, float* dV, int B, int T, int Tk, int H,
                     int HKV, int D, float scale, int causal, int window, fa_dtype_t dtype,
                     hipStream_t stream, int bq, int bk, const fa_layout_t& lq,
                     const fa_layout_t& lk, int g16 = 0,
                     Workspace ws = Workspace::kCached) {
    fa_status_t s = check_all({Q, K, V, O, L, dO, dQ, dK, dV}, B, T, Tk, H, HKV, D, scale, causal,
                              window, dtype, lq, lk);
    if (s != FA_OK) return s;
    if (dtype == FA_DTYPE_F32) {
        if ((s = resolve_f32_tiles(bq, bk)) != FA_OK) return s;
    } else if (!(bq == 0 && bk == 0)) {
        return FA_ERR_INVALID_ARG;
    }
    float* Dvec = nullptr;
    const size_t floats = (size_t)B * H * T;
    fa::WorkspaceLease lease;
    if (ws == Workspace::kFixedScratch) {
        // every Dvec row the dK/dV pass reads (rows < T) is written by the dQ pass first, so
        // the scratch needs no clearing between calls
        if (floats > (size_t)fa::kNoAllocDvecFloats) return FA_ERR_UNSUPPORTED;
        if (fa::noalloc_dvec(floats, &Dvec) != hipSuccess) return FA_ERR_HIP;
    } else {
        if (lease.acquire(floats * sizeof(float), stream) != hipSuccess) return FA_ERR_HIP;
        Dvec = lease.ptr();
    }
    s = dq_dvec_impl(Q, K, V, O, dO, L, Dvec, dQ, B, T, Tk, H, HKV, D, scale, causal, window, dtype,
                     stream, bq, bk, lq, lk, g16);
    if (s == FA_OK)
        s = dkdv_impl(Q, K, V, dO, L, Dvec, dK, dV, B, T, Tk, H, HKV, D, scale, causal, window,
                      dtype, stream, bq, bk, lq, lk, g16);
    if (lease.release() != hipSuccess && s == FA_OK) s = FA_ERR_HIP;
    return s;
}

}  // namespace

extern "C" {

const char* flash_attn_status_string(fa_status_t s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        default: break;
    }
    return "FA_UNKNOWN_STATUS";
}

int flash_attn_version(void) { return 102; }

fa_status_t flash_attn_mfma_rate_probe(const void* operands, float* out, int grid, int iters,
                                       hipStream_t stream) {
    fa_status_t s = check_ptrs({operands, out});
    if (s != FA_OK) return s;
    if (grid < 1 || grid > (1 << 20) || iters < 1 || iters > (1 << 24)) return FA_ERR_INVALID_ARG;
    return hip_status(fa::launch_mfma_probe(operands, out, grid, iters, stream));
}

fa_status_t flash_attn_check_layout(fa_layout_t layout, int B, int T, int heads, int D,
                                    fa_dtype_t dtype) {
    if (B < 1 || T < 1 || heads < 1 || D < 1) return FA_ERR_INVALID_ARG;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    return check_layout(layout, B, T, heads, D, dtype);
}

int flash_attn_block_class(int T, int bq, int bk, int causal, int window, int i, int j, int* off) {
    if (T < 1 || T > kMaxRows || bq < 1 || bk < 1 || window < 0 || i < 0 || j < 0) return -1;
    if (((long long)i + 1) * bq > (1ll << 30) || ((long long)j + 1) * bk > (1ll << 30)) return -1;
    if (off) *off = i * bq - j * bk;
    return fa::block_class(T, T, i * bq, i * bq + bq, j * bk, j * bk + bk, causal != 0,
                           effective_window(window, T));
}

int flash_attn_block_class_qk(int Tq, int Tk, int bq, int bk, int causal, int window, int i,
                              int j) {
    if (Tq < 1 || Tk < 1 || Tq > kMaxRows || Tk > kMaxRows || bq < 1 || bk < 1 || window < 0 ||
        i < 0 || j < 0)
        return -1;
    if (((long long)i + 1) * bq > (1ll << 30) || ((long long)j + 1) * bk > (1ll << 30)) return -1;
    return fa::block_class(Tq, Tk, i * bq, i * bq + bq, j * bk, j * bk + bk, causal != 0,
                           effective_window(window, Tk));
}

fa_status_t flash_attn_kv_block_range_qk(int Tq, int Tk, int bq, int bk, int causal, int window,
                                         int i, int* j_lo, int* j_hi) {
    if (Tq < 1 || Tk < 1 || Tq > kMaxRows || Tk > kMaxRows || bq < 1 || bk < 1 || window < 0 ||
        i < 0 || !j_lo || !j_hi)
        return FA_ERR_INVALID_ARG;
    if (((long long)i + 1) * bq > (1ll << 30)) return FA_ERR_INVALID_ARG;
    fa::kv_block_range(Tq, Tk, i * bq, i * bq + bq, bk, causal != 0, effective_window(window, Tk),
                       *j_lo, *j_hi);
    return FA_OK;
}

fa_status_t flash_attn_kv_block_range(int T, int bq, int bk, int causal, int window, int i,
                                      int* j_lo, int* j_hi) {
    if (T < 1 || T > kMaxRows || bq < 1 || bk < 1 || window < 0 || i < 0 || !j_lo || !j_hi)
        return FA_ERR_INVALID_ARG;
    if (((long long)i + 1) * bq > (1ll << 30)) return FA_ERR_INVALID_ARG;
    fa::kv_block_range(T, T, i * bq, i * bq + bq, bk, causal != 0, effective_window(window, T),
                       *j_lo, *j_hi);
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
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID_ARG;
    if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
    const int tq[3] = {fa::kB16FwdBq, fa::kB16DkdvBq, fa::kB16DqBq};
    const int tk[3] = {fa::kB16FwdBk, fa::kB16DkdvBk, fa::kB16DqBk};
    *bq = tq[pass];
    *bk = tk[pass];
    return FA_OK;
}

fa_status_t flash_attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* L,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    return fwd_impl(Q, K, V, O, L, B, T, T, H, HKV, D, scale, causal, window, dtype, stream, bq, bk,
                    dense_layout(T, H, D), dense_layout(T, HKV, D));
}

fa_status_t flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* L, int B,
                           int T, int H, int HKV, int D, float scale, int causal, int window,
                           fa_dtype_t dtype, hipStream_t stream) {
    return flash_attn_fwd_ex(Q, K, V, O, L, B, T, H, HKV, D, scale, causal, window, dtype, stream,
                             0, 0);
}

fa_status_t flash_attn_fwd_strided(const void* Q, const void* K, const void* V, void* O,
                                   float* L, int B, int T, int Tk, int H, int HKV, int D,
                                   float scale, int causal, int window, fa_dtype_t dtype,
                                   hipStream_t stream, fa_layout_t q_layout,
                                   fa_layout_t kv_layout) {
    return fwd_impl(Q, K, V, O, L, B, T, Tk, H, HKV, D, scale, causal, window, dtype, stream, 0,
                    0, q_layout, kv_layout);
}

fa_status_t flash_attn_bwd_preprocess(const void* O, const void* dO, float* Dvec, int B, int T,
                                      int H, int D, fa_dtype_t dtype, hipStream_t stream) {
    return preprocess_impl(O, dO, Dvec, B, T, H, D, dtype, stream, dense_layout(T, H, D));
}

fa_status_t flash_attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dvec, float* dK, float* dV, int B,
                                int T, int H, int HKV, int D, float scale, int causal, int window,
                                fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    return dkdv_impl(Q, K, V, dO, L, Dvec, dK, dV, B, T, T, H, HKV, D, scale, causal, window, dtype,
                     stream, bq, bk, dense_layout(T, H, D), dense_layout(T, HKV, D));
}

fa_status_t flash_attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                              const float* L, const float* Dvec, float* dQ, int B, int T, int H,
                              int HKV, int D, float scale, int causal, int window,
                              fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    return dq_impl(Q, K, V, dO, L, Dvec, dQ, B, T, T, H, HKV, D, scale, causal, window, dtype,
                   stream, bq, bk, dense_layout(T, H, D), dense_layout(T, HKV, D));
}

fa_status_t flash_attn_bwd_dq_dvec(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* L, float* Dvec, float* dQ, int B,
                                   int T, int H, int HKV, int D, float scale, int causal,
                                   int window, fa_dtype_t dtype, hipStream_t stream, int bq,
                                   int bk) {
    return dq_dvec_impl(Q, K, V, O, dO, L, Dvec, dQ, B, T, T, H, HKV, D, scale, causal, window,
                        dtype, stream, bq, bk, dense_layout(T, H, D), dense_layout(T, HKV, D));
}

fa_status_t flash_attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O,
                              const float* L, const void* dO, float* dQ, float* dK, float* dV,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk) {
    return bwd_impl(Q, K, V, O, L, dO, dQ, dK, dV, B, T, T, H, HKV, D, scale, causal, window, dtype,
                    stream, bq, bk, dense_layout(T, H, D), dense_layout(T, HKV, D));
}

fa_status_t flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                           const float* L, const void* dO, float* dQ, float* dK, float* dV, int B,
                           int T, int H, int HKV, int D, float scale, int causal, int window,
                           fa_dtype_t dtype, hipStream_t stream) {
    return flash_attn_bwd_ex(Q, K, V, O, L, dO, dQ, dK, dV, B, T, H, HKV, D, scale, causal,
                             window, dtype, stream, 0, 0);
}

fa_status_t flash_attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                                   const float* L, const void* dO, float* dQ, float* dK,
                                   float* dV, int B, int T, int H, int HKV, int D, float scale,
                                   int causal, int window, fa_dtype_t dtype, hipStream_t stream) {
    return bwd_impl(Q, K, V, O, L, dO, dQ, dK, dV, B, T, T, H, HKV, D, scale, causal, window, dtype,
                    stream, 0, 0, dense_layout(T, H, D), dense_layout(T, HKV, D), 0,
                    Workspace::kFixedScratch);
}

fa_status_t flash_attn_bwd_strided(const void* Q, const void* K, const void* V, const void* O,
                                   const float* L, const void* dO, float* dQ, float* dK,
                                   float* dV, int B, int T, int Tk, int H, int HKV, int D,
                                   float scale, int causal, int window, fa_dtype_t dtype,
                                   hipStream_t stream, fa_layout_t q_layout,
                                   fa_layout_t kv_layout) {
    return bwd_impl(Q, K, V, O, L, dO, dQ, dK, dV, B, T, Tk, H, HKV, D, scale, causal, window,
                    dtype, stream, 0, 0, q_layout, kv_layout);
}

fa_status_t flash_attn_bwd_grad16(const void* Q, const void* K, const void* V, const void* O,
                                  const float* L, const void* dO, void* dQ, void* dK, void* dV,
                                  int B, int T, int Tk, int H, int HKV, int D, float scale,
                                  int causal, int window, fa_dtype_t dtype, hipStream_t stream,
                                  fa_layout_t q_layout, fa_layout_t kv_layout) {
    if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_INVALID_ARG;
    return bwd_impl(Q, K, V, O, L, dO, static_cast<float*>(dQ), static_cast<float*>(dK),
                    static_cast<float*>(dV), B, T, Tk, H, HKV, D, scale, causal, window, dtype,
                    stream, 0, 0, q_layout, kv_layout, 1);
}

fa_status_t flash_attn_qk_norm_rope(const void* qk, int64_t qk_stride_t, int64_t qk_stride_h,
                                   const float* factor1, const float* factor2,
                                   int64_t factor_stride_t, void* out_q, void* out_k, int tokens,
                                   int heads, int qk_dim, int rotary_dim, int paired,
                                   int key_offset, fa_dtype_t dtype, hipStream_t stream) {
    fa_status_t s = check_ptrs({qk, factor1, factor2, out_q, out_k});
    if (s != FA_OK) return s;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
        return FA_ERR_INVALID_ARG;
    if (tokens < 1 || heads < 1 || (paired != 0 && paired != 1) ||
        (key_offset != 0 && key_offset != 1) || (paired && key_offset) || (paired && heads % 2))
        return FA_ERR_INVALID_ARG;
    if (!(qk_dim == 16 || qk_dim == 32 || qk_dim == 64 || qk_dim == 128 || qk_dim == 256))
        return FA_ERR_UNSUPPORTED;
    if (rotary_dim < 0 || rotary_dim > qk_dim || rotary_dim % 2) return FA_ERR_INVALID_ARG;
    const int64_t esz = dtype == FA_DTYPE_F32 ? 4 : 2, align = 16 / esz;
    // rows of a token stored together, heads at least D apart, 16-byte aligned
    if (qk_stride_h < qk_dim || qk_stride_h % align) return FA_ERR_INVALID_ARG;
    if (qk_stride_t < (int64_t)(2 * heads - 1) * qk_stride_h + qk_dim || qk_stride_t % align)
        return FA_ERR_INVALID_ARG;
    if (factor_stride_t < (int64_t)qk_dim * (paired ? 2 : 1) || factor_stride_t % 4)
        return FA_ERR_INVALID_ARG;
    if ((double)tokens * qk_stride_t * esz > 9.0e18 || (double)tokens * 2 * heads * qk_dim > 4.0e12)
        return FA_ERR_INVALID_ARG;
    fa::RopeArgs a{};
    a.qk = qk; a.st = qk_stride_t; a.sh = qk_stride_h;
    a.f1 = factor1; a.f2 = factor2; a.fst = factor_stride_t;
    a.out_q = out_q; a.out_k = out_k;
    a.tokens = tokens; a.heads = heads; a.D = qk_dim; a.rotary_dim = rotary_dim;
    a.paired = paired; a.key_offset = key_offset;
    a.dtype = dtype == FA_DTYPE_F32 ? 0 : dtype == FA_DTYPE_BF16 ? 1 : 2;
    a.stream = stream;
    return hip_status(fa::launch_qk_norm_rope(a));
}

}  // extern "C"
