// Block classification for tiled causal / sliding-window attention, shared by every kernel
// and by the host-side query entry points, so host tests see exactly what the device does.
//
// A block covers query rows [r0, r1) and keys [c0, c1).  In a T x T problem a query row r
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

// Query rows and keys may number differently (Tq, Tk).  Query row r then sits at key position
// r + Tk - Tq (the rows are the last Tq positions, as when the keys start with a prefix), and
// the rules above apply to that position: row r sees key c when c < Tk and (no causal or
// c <= r + Tk - Tq) and (no window or c >= r + Tk - Tq - W + 1).  With Tq = Tk this is the
// square rule.  Rows whose position is negative (Tq > Tk, causal) see no key.

FA_HD int block_class(int Tq, int Tk, int r0, int r1, int c0, int c1, bool causal, int window) {
    if (r1 > Tq) r1 = Tq;
    if (r0 >= r1 || c0 >= Tk || c0 >= c1) return kSkip;
    const int dq = Tk - Tq;
    const int p0 = r0 + dq, P = r1 - 1 + dq;   // first and last row position
    const int C = (c1 < Tk ? c1 : Tk) - 1;     // last in-range key
    // any visible pair: exists p in [p0, P] with [p-W+1, p] meeting [c0, C]
    if (causal && c0 > P) return kSkip;
    if (window > 0 && C < p0 - window + 1) return kSkip;
    bool full = (c1 <= Tk);
    if (causal && C > p0) full = false;
    if (window > 0 && c0 < P - window + 1) full = false;
    return full ? kFull : kPartial;
}

// Key-block range [lo, hi) (blocks of bk keys) that rows [r0, r1) may see.
FA_HD void kv_block_range(int Tq, int Tk, int r0, int r1, int bk, bool causal, int window,
                          int& lo, int& hi) {
    if (r1 > Tq) r1 = Tq;
    lo = hi = 0;
    if (r0 >= r1) return;
    const int dq = Tk - Tq;
    const int p0 = r0 + dq, P = r1 - 1 + dq;
    const int first = (window > 0 && p0 - window + 1 > 0) ? p0 - window + 1 : 0;
    const int last = causal ? (P < Tk - 1 ? P : Tk - 1) : Tk - 1;
    if (last < first) return;
    lo = first / bk;
    hi = last / bk + 1;
}

// Query-block range [lo, hi) (blocks of bq rows) whose rows may see keys [c0, c1).
FA_HD void q_block_range(int Tq, int Tk, int c0, int c1, int bq, bool causal, int window,
                         int& lo, int& hi) {
    if (c1 > Tk) c1 = Tk;
    lo = hi = 0;
    if (c0 >= c1) return;
    const int dq = Tk - Tq;
    // row positions p = r + dq that see some key of [c0, c1): p >= c0 (causal) and
    // p <= c1 - 1 + W - 1 (window), with r in [0, Tq)
    int first = causal ? c0 - dq : 0;
    int last = (window > 0) ? c1 - 1 + window - 1 - dq : Tq - 1;
    if (first < 0) first = 0;
    if (last > Tq - 1) last = Tq - 1;
    if (first > last) return;
    lo = first / bq;
    hi = last / bq + 1;
}

// floor(a / b) for b > 0 and any a.
FA_HD int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Key blocks j (keys [j*bk, j*bk + bk)) that are FULL for rows [r0, r1), as [lo, hi) (empty
// when hi <= lo): every key in range (c1 <= Tk), before the causal bound of the first row
// and inside the window of the last row.  Inside it block_class returns kFull; the kernels
// call block_class only outside it.
FA_HD void full_kv_block_range(int Tq, int Tk, int r0, int r1, int bk, bool causal, int window,
                               int& lo, int& hi) {
    if (r1 > Tq) r1 = Tq;
    lo = hi = 0;
    if (r0 >= r1) return;
    const int dq = Tk - Tq;
    const int p0 = r0 + dq, P = r1 - 1 + dq;
    int h = Tk / bk;                                          // (j + 1) bk <= Tk
    if (causal) {                                             // (j + 1) bk - 1 <= p0
        const int hc = floor_div(p0 + 1, bk);
        if (hc < h) h = hc;
    }
    int l = 0;
    if (window > 0 && P - window + 1 > 0) l = (P - window + 1 + bk - 1) / bk;   // j bk >= P - W + 1
    if (h > l) {
        lo = l;
        hi = h;
    }
}

// Query blocks i (rows [i*bq, i*bq + bq)) that are FULL for keys [c0, c1), as [lo, hi): the
// transposed form for key-owned passes.
FA_HD void full_q_block_range(int Tq, int Tk, int c0, int c1, int bq, bool causal, int window,
                              int& lo, int& hi) {
    lo = hi = 0;
    if (c0 >= c1 || c1 > Tk) return;
    const int dq = Tk - Tq;
    int l = 0;
    if (causal && c1 - 1 - dq > 0) l = (c1 - 1 - dq + bq - 1) / bq;   // i bq + dq >= c1 - 1
    int h = (Tq + bq - 1) / bq;                                          // i bq < Tq
    if (window > 0 && Tq > c0 + window - dq) {                           // last row inside
        const int hw = floor_div(c0 + window - dq, bq);                  // (i + 1) bq <= c0 + W - dq
        if (hw < h) h = hw;
    }
    if (h > l) {
        lo = l;
        hi = h;
    }
}

// Per-element keep test in global indices (used inside PARTIAL blocks).
FA_HD bool visible(int r, int c, int Tq, int Tk, bool causal, int window) {
    const int p = r + Tk - Tq;
    return r < Tq && c < Tk && (!causal || c <= p) && (window <= 0 || c >= p - window + 1);
}

// Number of keys row r sees, as the interval [lo, lo + n) (n = 0 when none): the kernels'
// per-lane form of the rule, one unsigned compare per element.
FA_HD void row_keys(int r, int Tq, int Tk, bool causal, int window, int& lo, int& n) {
    const int p = r + Tk - Tq;
    lo = window > 0 ? p - window + 1 : 0;
    if (lo < 0) lo = 0;
    int hi = causal ? p : Tk - 1;
    if (hi > Tk - 1) hi = Tk - 1;
    n = hi >= lo ? hi - lo + 1 : 0;
}

// Query rows that see key c, as [lo, lo + n): the transposed form for key-owned passes.
FA_HD void key_rows(int c, int Tq, int Tk, bool causal, int window, int& lo, int& n) {
    const int dq = Tk - Tq;
    lo = causal ? c - dq : 0;
    if (lo < 0) lo = 0;
    int hi = window > 0 ? c - dq + window - 1 : Tq - 1;
    if (hi > Tq - 1) hi = Tq - 1;
    n = (c < Tk && hi >= lo) ? hi - lo + 1 : 0;
}

}  // namespace fa
