// Host-only harness for the C-ABI layer (api.hip) built with AddressSanitizer and
// UndefinedBehaviorSanitizer: the kernel launchers are replaced by stubs that record their
// arguments, so every validation path, every dispatch path and the host-side classifier
// helpers run on the CPU under the sanitizers.  Prints "abi-asan ok" and exits 0 when every
// check passes.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>
#include <vector>

#include "flash_attn.h"
#include "kernels.h"

namespace {
std::vector<std::string> g_calls;
fa::AttnArgs g_last{};
int g_last_bq = 0, g_last_bk = 0;
int g_fail = 0;

void check(bool ok, const char* what, int line) {
    if (!ok) {
        printf("FAIL line %d: %s\n", line, what);
        ++g_fail;
    }
}
#define CHECK(c) check((c), #c, __LINE__)

hipError_t record(const char* name, const fa::AttnArgs& a, int bq = 0, int bk = 0) {
    g_calls.push_back(name);
    g_last = a;
    g_last_bq = bq;
    g_last_bk = bk;
    return hipSuccess;
}
}  // namespace

namespace fa {
// the tilings the f32 kernels are instantiated for, as flash_attn.h documents them
bool f32_tiles_supported(int bq, int bk) {
    return (bq == 32 || bq == 64) && (bk == 16 || bk == 32 || bk == 64);
}
hipError_t launch_fwd_f32(const AttnArgs& a, int bq, int bk) { return record("fwd_f32", a, bq, bk); }
hipError_t launch_dkdv_f32(const AttnArgs& a, int bq, int bk) { return record("dkdv_f32", a, bq, bk); }
hipError_t launch_dq_f32(const AttnArgs& a, int bq, int bk) { return record("dq_f32", a, bq, bk); }
hipError_t launch_fwd_b16(const AttnArgs& a) { return record("fwd_b16", a); }
hipError_t launch_dkdv_b16(const AttnArgs& a) { return record("dkdv_b16", a); }
hipError_t launch_dq_b16(const AttnArgs& a) { return record("dq_b16", a); }
hipError_t launch_dq_b16_fused_d(const AttnArgs& a) { return record("dq_b16_fused_d", a); }
hipError_t launch_qk_norm_rope(const RopeArgs&) {
    g_calls.push_back("rope");
    return hipSuccess;
}
hipError_t launch_bwd_preprocess(const void*, const void*, float*, int, int, int, int, int,
                                 hipStream_t, Layout) {
    g_calls.push_back("preprocess");
    return hipSuccess;
}
hipError_t launch_mfma_probe(const void*, float*, int, int, hipStream_t) {
    g_calls.push_back("mfma_probe");
    return hipSuccess;
}
alignas(256) float g_fake_scratch[64];
size_t g_scratch_request = 0;
hipError_t noalloc_dvec(size_t floats, float** out) {
    g_calls.push_back("scratch");
    g_scratch_request = floats;
    *out = floats <= (size_t)kNoAllocDvecFloats ? g_fake_scratch : nullptr;
    return floats <= (size_t)kNoAllocDvecFloats ? hipSuccess : hipErrorInvalidValue;
}
}  // namespace fa

namespace {

// 16-byte-aligned addresses inside a host buffer: never dereferenced by the stubs, but real
// memory so that any stray host access would be caught by the sanitizer.
alignas(64) char g_buf[4096];
void* P(int i) { return g_buf + 64 * i; }
void* const MIS = g_buf + 4;

struct Dims {
    int B = 2, T = 40, H = 8, HKV = 2, D = 64;
    float scale = 0.125f;
    int causal = 1, window = 0;
    fa_dtype_t dt = FA_DTYPE_BF16;
};

fa_status_t fwd(const Dims& d, void* q = P(0)) {
    return flash_attn_fwd(q, P(1), P(2), P(3), (float*)P(4), d.B, d.T, d.H, d.HKV, d.D, d.scale,
                          d.causal, d.window, d.dt, nullptr);
}
fa_status_t bwd(const Dims& d, float* dq = (float*)P(6)) {
    return flash_attn_bwd(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), dq, (float*)P(7),
                          (float*)P(8), d.B, d.T, d.H, d.HKV, d.D, d.scale, d.causal, d.window,
                          d.dt, nullptr);
}
fa_status_t dkdv(const Dims& d, int bq = 0, int bk = 0) {
    return flash_attn_bwd_dkdv(P(0), P(1), P(2), P(5), (const float*)P(4), (const float*)P(9),
                               (float*)P(7), (float*)P(8), d.B, d.T, d.H, d.HKV, d.D, d.scale,
                               d.causal, d.window, d.dt, nullptr, bq, bk);
}
fa_status_t dq_dvec(const Dims& d, int bq = 0, int bk = 0) {
    return flash_attn_bwd_dq_dvec(P(0), P(1), P(2), P(3), P(5), (const float*)P(4), (float*)P(9),
                                  (float*)P(6), d.B, d.T, d.H, d.HKV, d.D, d.scale, d.causal,
                                  d.window, d.dt, nullptr, bq, bk);
}

void test_validation() {
    struct Bad {
        Dims d;
        fa_status_t want;
    };
    std::vector<Bad> bad;
    auto add = [&](void (*f)(Dims&), fa_status_t w) {
        Dims d;
        f(d);
        bad.push_back({d, w});
    };
    add([](Dims& d) { d.B = 0; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.T = 0; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.H = -3; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.HKV = 3; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.D = 0; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.window = -1; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.causal = 7; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.scale = NAN; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.scale = INFINITY; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.scale = -1.f; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.dt = (fa_dtype_t)9; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.D = 96; }, FA_ERR_UNSUPPORTED);
    add([](Dims& d) { d.dt = FA_DTYPE_F32; d.D = 12; }, FA_ERR_UNSUPPORTED);
    add([](Dims& d) { d.dt = FA_DTYPE_F32; d.D = 136; }, FA_ERR_UNSUPPORTED);
    add([](Dims& d) { d.B = INT_MAX; d.T = INT_MAX; d.H = INT_MAX; d.HKV = 1; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.T = 1 << 24; d.H = 64; d.HKV = 8; d.D = 128; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.T = INT_MAX; d.B = 1; d.H = 1; d.HKV = 1; }, FA_ERR_INVALID_ARG);
    add([](Dims& d) { d.T = (1 << 30) + 1; d.B = 1; d.H = 1; d.HKV = 1; d.dt = FA_DTYPE_F32; d.D = 8; },
        FA_ERR_INVALID_ARG);
    for (const Bad& b : bad) {
        g_calls.clear();
        CHECK(fwd(b.d) == b.want);
        CHECK(bwd(b.d) == b.want);
        CHECK(dkdv(b.d) == b.want);
        CHECK(dq_dvec(b.d) == b.want);
        CHECK(g_calls.empty());
    }
    Dims d;
    g_calls.clear();
    CHECK(fwd(d, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(fwd(d, MIS) == FA_ERR_INVALID_ARG);
    CHECK(bwd(d, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(bwd(d, (float*)MIS) == FA_ERR_INVALID_ARG);
    CHECK(dkdv(d, 64, 64) == FA_ERR_INVALID_ARG);       // 16-bit types take one tiling
    Dims f = d;
    f.dt = FA_DTYPE_F32;
    CHECK(dkdv(f, 48, 16) == FA_ERR_INVALID_ARG);
    CHECK(dq_dvec(f, 64, 8) == FA_ERR_INVALID_ARG);
    CHECK(g_calls.empty());
    // layouts
    fa_layout_t good_q{(int64_t)d.T * d.H * d.D, (int64_t)d.H * d.D, d.D};
    fa_layout_t good_k{(int64_t)d.T * d.HKV * d.D, (int64_t)d.HKV * d.D, d.D};
    const fa_layout_t bad_layouts[] = {
        {-good_q.batch, good_q.row, good_q.head},   // negative
        {good_q.batch, d.D - 8, good_q.head},       // rows overlap
        {good_q.batch, good_q.row, 4},              // heads overlap
        {good_q.batch + 4, good_q.row, good_q.head},   // not 16-byte aligned (bf16)
        {INT64_MAX, INT64_MAX, INT64_MAX},          // overflow
        {0, good_q.row, good_q.head},               // batches overlap
    };
    for (const fa_layout_t& l : bad_layouts) {
        CHECK(flash_attn_check_layout(l, d.B, d.T, d.H, d.D, d.dt) == FA_ERR_INVALID_ARG);
        CHECK(flash_attn_fwd_strided(P(0), P(1), P(2), P(3), (float*)P(4), d.B, d.T, d.T, d.H,
                                     d.HKV, d.D, d.scale, d.causal, d.window, d.dt, nullptr, l,
                                     good_k) == FA_ERR_INVALID_ARG);
    }
    CHECK(g_calls.empty());
    CHECK(flash_attn_check_layout(good_q, d.B, d.T, d.H, d.D, d.dt) == FA_OK);
    // [B, H, T, D] strides are usable
    fa_layout_t bhtd{(int64_t)d.H * d.T * d.D, d.D, (int64_t)d.T * d.D};
    CHECK(flash_attn_check_layout(bhtd, d.B, d.T, d.H, d.D, d.dt) == FA_OK);
    // grad16 refuses f32; rope refuses bad head dims, strides and flags
    CHECK(flash_attn_bwd_grad16(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), P(6), P(7),
                                P(8), d.B, d.T, d.T, d.H, d.HKV, d.D, d.scale, 1, 0, FA_DTYPE_F32,
                                nullptr, good_q, good_k) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_qk_norm_rope(P(0), 8 * 64, 64, (const float*)P(1), (const float*)P(2), 64,
                                  P(3), P(4), 16, 4, 48, 48, 0, 0, FA_DTYPE_BF16, nullptr) ==
          FA_ERR_UNSUPPORTED);
    CHECK(flash_attn_qk_norm_rope(P(0), 8 * 64, 32, (const float*)P(1), (const float*)P(2), 64,
                                  P(3), P(4), 16, 4, 64, 64, 0, 0, FA_DTYPE_BF16, nullptr) ==
          FA_ERR_INVALID_ARG);
    CHECK(flash_attn_qk_norm_rope(P(0), 8 * 64, 64, (const float*)P(1), (const float*)P(2), 64,
                                  P(3), P(4), 16, 3, 64, 64, 1, 0, FA_DTYPE_BF16, nullptr) ==
          FA_ERR_INVALID_ARG);
    CHECK(flash_attn_qk_norm_rope(P(0), 8 * 64, 64, (const float*)P(1), (const float*)P(2), 64,
                                  P(3), P(4), 16, 4, 64, 63, 0, 0, FA_DTYPE_BF16, nullptr) ==
          FA_ERR_INVALID_ARG);
    CHECK(g_calls.empty());
}

void test_dispatch() {
    Dims d;
    g_calls.clear();
    CHECK(fwd(d) == FA_OK);
    CHECK(g_calls.size() == 1 && g_calls[0] == "fwd_b16");
    CHECK(g_last.B == d.B && g_last.T == d.T && g_last.Tk == d.T && g_last.H == d.H &&
          g_last.HKV == d.HKV && g_last.D == d.D && g_last.f16 == 0 && g_last.Q == P(0) &&
          g_last.Oout == P(3) && g_last.lq.t == (int64_t)d.H * d.D && g_last.lk.h == d.D);
    Dims h = d;
    h.dt = FA_DTYPE_F16;
    g_calls.clear();
    CHECK(fwd(h) == FA_OK && g_calls.size() == 1 && g_last.f16 == 1);
    Dims f = d;
    f.dt = FA_DTYPE_F32;
    f.D = 8;
    g_calls.clear();
    CHECK(fwd(f) == FA_OK);
    CHECK(g_calls.size() == 1 && g_calls[0] == "fwd_f32" && g_last_bq == 64 && g_last_bk == 64);
    g_calls.clear();
    CHECK(dq_dvec(f, 32, 16) == FA_OK);
    CHECK(g_calls.size() == 2 && g_calls[0] == "preprocess" && g_calls[1] == "dq_f32" &&
          g_last_bq == 32 && g_last_bk == 16);
    g_calls.clear();
    CHECK(dq_dvec(d) == FA_OK && g_calls.size() == 1 && g_calls[0] == "dq_b16_fused_d");
    // a window of T keys or more reaches the kernels as no window; shorter ones unchanged
    Dims w = d;
    for (int win : {1, d.T - 1, d.T, d.T + 1, INT_MAX}) {
        w.window = win;
        g_calls.clear();
        CHECK(fwd(w) == FA_OK && g_calls.size() == 1);
        CHECK(g_last.window == (win >= d.T ? 0 : win));
    }
    // the largest accepted length
    Dims big;
    big.B = 1; big.H = 1; big.HKV = 1; big.dt = FA_DTYPE_F32; big.D = 8; big.T = 1 << 30;
    g_calls.clear();
    CHECK(fwd(big) == FA_OK && g_calls.size() == 1 && g_last.T == (1 << 30));
    g_calls.clear();
    CHECK(dkdv(d) == FA_OK && g_calls.size() == 1 && g_calls[0] == "dkdv_b16");
    // full backward: the Dvec workspace comes from the library's workspace cache.  Without a
    // device that fails and nothing is launched (FA_ERR_HIP); with one, dQ+Dvec then dK/dV run.
    g_calls.clear();
    const fa_status_t s = bwd(d);
    if (s == FA_OK) {
        CHECK(g_calls.size() == 2 && g_calls[0] == "dq_b16_fused_d" && g_calls[1] == "dkdv_b16");
    } else {
        CHECK(s == FA_ERR_HIP);
        CHECK(g_calls.empty());
    }
    // no-allocation backward: the fixed scratch replaces the workspace cache (which has no
    // device to allocate on here), so the two passes run and both see the scratch as Dvec
    g_calls.clear();
    CHECK(flash_attn_bwd_noalloc(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), (float*)P(6),
                                 (float*)P(7), (float*)P(8), d.B, d.T, d.H, d.HKV, d.D, d.scale,
                                 d.causal, d.window, d.dt, nullptr) == FA_OK);
    CHECK(g_calls.size() == 3 && g_calls[0] == "scratch" && g_calls[1] == "dq_b16_fused_d" &&
          g_calls[2] == "dkdv_b16");
    CHECK(g_last.Dvec == fa::g_fake_scratch && fa::g_scratch_request == (size_t)d.B * d.H * d.T);
    g_calls.clear();
    CHECK(flash_attn_bwd_noalloc(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), (float*)P(6),
                                 (float*)P(7), (float*)P(8), d.B, d.T, d.H, d.HKV, d.D, d.scale,
                                 d.causal, d.window, FA_DTYPE_F32, nullptr) == FA_OK);
    CHECK(g_calls.size() == 4 && g_calls[1] == "preprocess" && g_calls[3] == "dkdv_f32");
    // beyond the scratch: refused before anything is looked up or launched
    g_calls.clear();
    CHECK(flash_attn_bwd_noalloc(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), (float*)P(6),
                                 (float*)P(7), (float*)P(8), 2, FA_NOALLOC_MAX_DVEC / 16 + 1, 8,
                                 2, 64, d.scale, 1, 0, d.dt, nullptr) == FA_ERR_UNSUPPORTED);
    CHECK(flash_attn_bwd_noalloc(P(0), P(1), P(2), P(3), (const float*)P(4), P(5), nullptr,
                                 (float*)P(7), (float*)P(8), d.B, d.T, d.H, d.HKV, d.D, d.scale,
                                 d.causal, d.window, d.dt, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(g_calls.empty());
    // strided, Tq != Tk
    fa_layout_t lq{(int64_t)d.H * 24 * d.D, d.D, (int64_t)24 * d.D};
    fa_layout_t lk{(int64_t)d.HKV * 56 * d.D, d.D, (int64_t)56 * d.D};
    g_calls.clear();
    CHECK(flash_attn_fwd_strided(P(0), P(1), P(2), P(3), (float*)P(4), d.B, 24, 56, d.H, d.HKV,
                                 d.D, d.scale, 1, 5, d.dt, nullptr, lq, lk) == FA_OK);
    CHECK(g_calls.size() == 1 && g_last.T == 24 && g_last.Tk == 56 && g_last.window == 5 &&
          g_last.lq.h == 24 * d.D && g_last.lk.b == lk.batch);
    g_calls.clear();
    CHECK(flash_attn_qk_norm_rope(P(0), 8 * 64, 64, (const float*)P(1), (const float*)P(2), 64,
                                  P(3), P(4), 16, 4, 64, 64, 0, 1, FA_DTYPE_BF16, nullptr) ==
          FA_OK);
    CHECK(g_calls.size() == 1 && g_calls[0] == "rope");
    g_calls.clear();
    CHECK(flash_attn_mfma_rate_probe(P(0), (float*)P(1), 0, 10, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_mfma_rate_probe(P(0), (float*)P(1), 8, 0, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_mfma_rate_probe(MIS, (float*)P(1), 8, 10, nullptr) == FA_ERR_INVALID_ARG);
    CHECK(g_calls.empty());
    CHECK(flash_attn_mfma_rate_probe(P(0), (float*)P(1), 8, 10, nullptr) == FA_OK);
    CHECK(g_calls.size() == 1 && g_calls[0] == "mfma_probe");
}

// Visibility of (row r, key c) by the definition in flash_attn.h.
bool vis(int r, int c, int Tq, int Tk, int causal, int window) {
    const int64_t p = (int64_t)r + Tk - Tq;
    return r < Tq && c < Tk && (!causal || c <= p) && (window == 0 || c >= p - window + 1);
}

void test_classifier() {
    long blocks = 0;
    for (int Tq = 1; Tq <= 37; Tq += 3)
        for (int Tk = 1; Tk <= 41; Tk += 4)
            for (int bq : {1, 4, 16, 32})
                for (int bk : {1, 8, 16})
                    for (int causal = 0; causal <= 1; ++causal)
                        for (int window : {0, 1, 5, 17, 40, INT_MAX})
                            for (int i = 0; i * bq < Tq; ++i) {
                                int lo = -1, hi = -1;
                                CHECK(flash_attn_kv_block_range_qk(Tq, Tk, bq, bk, causal, window,
                                                                   i, &lo, &hi) == FA_OK);
                                for (int j = 0; j * bk < Tk; ++j) {
                                    int nvis = 0, nin = 0;
                                    for (int r = i * bq; r < i * bq + bq && r < Tq; ++r)
                                        for (int c = j * bk; c < j * bk + bk; ++c) {
                                            nvis += vis(r, c, Tq, Tk, causal, window);
                                            nin += c < Tk;
                                        }
                                    const int want = nvis == 0 ? 0
                                                   : (nvis == nin && j * bk + bk <= Tk) ? 1
                                                                                        : 2;
                                    const int got = flash_attn_block_class_qk(Tq, Tk, bq, bk,
                                                                              causal, window, i, j);
                                    CHECK(got == want);
                                    if (nvis) CHECK(j >= lo && j < hi);
                                    ++blocks;
                                }
                            }
    // argument guards: huge or negative indices are refused, never overflow
    int off = 0, lo = 0, hi = 0;
    CHECK(flash_attn_block_class(100, 64, 64, 1, 0, INT_MAX, 0, &off) == -1);
    CHECK(flash_attn_block_class(100, INT_MAX, 64, 1, 0, 2, 0, &off) == -1);
    CHECK(flash_attn_block_class(100, 64, 64, 1, -1, 0, 0, &off) == -1);
    CHECK(flash_attn_block_class_qk(100, 100, 64, INT_MAX, 1, 0, 0, 3) == -1);
    CHECK(flash_attn_kv_block_range(100, 64, 64, 1, 0, INT_MAX, &lo, &hi) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_kv_block_range(100, 64, 64, 1, 0, 0, nullptr, &hi) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_kv_block_range_qk(INT_MAX, 1, 1 << 20, 1, 1, 0, 1 << 10, &lo, &hi) ==
          FA_ERR_INVALID_ARG);
    int bq = 0, bk = 0;
    CHECK(flash_attn_default_tiles(FA_DTYPE_BF16, 128, 1, &bq, &bk) == FA_OK && bq > 0 && bk > 0);
    CHECK(flash_attn_default_tiles(FA_DTYPE_BF16, 128, 3, &bq, &bk) == FA_ERR_INVALID_ARG);
    CHECK(flash_attn_default_tiles(FA_DTYPE_F32, 8, 0, nullptr, &bk) == FA_ERR_INVALID_ARG);
    printf("classifier blocks checked %ld\n", blocks);
}

}  // namespace

int main() {
    test_validation();
    test_dispatch();
    test_classifier();
    for (int s = -1; s <= 4; ++s) CHECK(flash_attn_status_string((fa_status_t)s) != nullptr);
    if (g_fail) {
        printf("abi-asan FAILED %d checks\n", g_fail);
        return 1;
    }
    printf("abi-asan ok\n");
    return 0;
}
