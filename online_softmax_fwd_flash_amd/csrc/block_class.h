// Block classification for tiled causal / sliding-window attention, shared by every kernel
// and by the host-side query entry points, so host tests see exactly what the device does.
//
// A block covers query rows [r0, r1) and keys [c0, c1) of a T x T problem.  A query row r
// sees key c when (no causal or c <= r) and (no window or c >= r - W + 1) and c < T.
//   SKIP    nothing in the block is visible (never computed),
//   FULL    every in-range element is visible and no key is past T (no mask test),
//   PARTIAL anything else (per-element test).  Rows >= T are never stored, so they do not
//           force a mask.
// Causal whole-block skipping and mask-only-on-the-diagonal follow the Graphcore page
// "flash_attention_qkv_packed.cpp" (doBlock / doMask conditions of its loops) and the forge
// page "flash_attention.metal" (forward kernel: causal key bound, diagonal-only mask, window
// block skip).  For non-square tiles the mask of a block depends only on off = r0 - c0:
// keep c' <= r' + off (causal) and c' >= r' + off - W + 1 (window), in block-local indices.
#pragma once

#ifndef FA_HD
#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif
#endif

namespace fa {

enum BlockClass : int { kSkip = 0, kFull = 1, kPartial = 2 };

FA_HD int block_class(int T, int r0, int r1, int c0, int c1, bool causal, int window) {
    if (r1 > T) r1 = T;
    if (r0 >= r1 || c0 >= T || c0 >= c1) return kSkip;
    const int R = r1 - 1;                      // last in-range row
    const int C = (c1 < T ? c1 : T) - 1;       // last in-range key
    // any visible pair: exists r in [r0,R] with [r-W+1, r] meeting [c0, C]
    if (causal && c0 > R) return kSkip;
    if (window > 0 && C < r0 - window + 1) return kSkip;
    bool full = (c1 <= T);
    if (causal && C > r0) full = false;
    if (window > 0 && c0 < R - window + 1) full = false;
    return full ? kFull : kPartial;
}

// Key-block range [lo, hi) (blocks of bk keys) that rows [r0, r1) may see.
FA_HD void kv_block_range(int T, int r0, int r1, int bk, bool causal, int window, int& lo,
                          int& hi) {
    if (r1 > T) r1 = T;
    if (r0 >= r1) { lo = hi = 0; return; }
    int first = (window > 0 && r0 - window + 1 > 0) ? r0 - window + 1 : 0;
    int last = causal ? r1 - 1 : T - 1;
    lo = first / bk;
    hi = last / bk + 1;
}

// Query-block range [lo, hi) (blocks of bq rows) whose rows may see keys [c0, c1).
FA_HD void q_block_range(int T, int c0, int c1, int bq, bool causal, int window, int& lo,
                         int& hi) {
    if (c1 > T) c1 = T;
    if (c0 >= c1) { lo = hi = 0; return; }
    int first = causal ? c0 : 0;
    int last = (window > 0 && c1 - 1 + window - 1 < T - 1) ? c1 - 1 + window - 1 : T - 1;
    if (first > last) { lo = hi = 0; return; }
    lo = first / bq;
    hi = last / bq + 1;
}

// Per-element keep test in global indices (used inside PARTIAL blocks).
FA_HD bool visible(int r, int c, int T, bool causal, int window) {
    return c < T && (!causal || c <= r) && (window <= 0 || c >= r - window + 1);
}

}  // namespace fa
