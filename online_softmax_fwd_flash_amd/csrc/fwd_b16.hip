// 16-bit forward attention for gfx950 (bf16 or fp16 I/O, D in {64, 128}): MFMA 16x16x32 with
// fp32 accumulation, online softmax in registers, O and one log-sum-exp per query row stored.
//
// Method (prior art, other hardware): forge "flash_attention.metal", header comment and the
// forward kernel (online-softmax update, m from -FLT_MAX, K/V staged per block through
// on-chip memory, causal key bound, window block skip, diagonal-only mask, l == 0 guard);
// Graphcore "flash_attention_qkv_packed.cpp", flashAttentionQKVPackedWithStash (block skip /
// mask conditions, L = m + log l stash).
//
// gfx950 design
//  * Workgroup = 4 waves = 128 query rows of one (b, h); wave w owns 32 rows; three
//    workgroups per CU, so one workgroup's barrier waits are covered by the others' work.
//    Key blocks of 32 go HBM -> LDS by LDS-DMA (buffer_load ... lds, 16 bytes per lane): no
//    staging registers and no LDS write instructions.  Two stages: block j + 1 is fetched
//    while block j is computed; one barrier per block, which does not wait for that fetch.
//  * All products are 16x16x32 MFMAs (on N(0, 1) operands the chip sustains about a third
//    more FLOP/s on this shape than on 32x32x16 under its power limit).  A wave's 32 rows are
//    two 16-row query tiles, so each lane holds two query rows (n and 16 + n).
//  * K and V tiles keep padded rows (D + 16 elements; each row's pad slots get copies of a
//    valid chunk): the 16-byte K operand reads and the V^T transpose reads are then free of
//    bank conflicts.
//  * Scores are formed transposed, S^T = K Q^T: the accumulator column (lane % 16) is a query
//    row, so each query's max / sum are in-lane plus two exchanges across the four 16-lane
//    rows.
//  * P^T (rounded to the element type, RNE) feeds O^T += V^T P^T straight from the
//    accumulator registers: lane row g holds keys 4g .. 4g + 3 of each 16-key tile, so its
//    entries of the block's two key tiles are the 8 keys it supplies for a 32-key k-step; the
//    V^T operand in that key order comes from the row-major V tile through two LDS transpose
//    reads (ds_read_b64_tr_b16) per MFMA, so V needs no transposed copy.
//  * The running max is rescaled lazily: O and l are only rescaled when some row's max grew
//    by more than 2^8 (the stale max keeps every exp2 argument below 8, so nothing overflows
//    and the final O / l and L = m*scale + ln l are exact up to rounding).
//  * Work order: longest key ranges (last query tiles) first; with GQA the query heads of one
//    KV head are placed on the same XCD (workgroup ids congruent mod 8) at the same time so
//    they share its K/V in that XCD's L2.
//  * Scalar and vector overhead per block is kept small, since a SIMD issues at most one
//    instruction of each kind per 4-cycle slot: each wave computes once the range of key
//    blocks that are FULL for its rows and runs the class test only outside it, and the
//    diagonal mask is a real branch (keep_branch) rather than selects on every block.
#include "common.h"
#include "kernels.h"
#include "stage_b16.h"

namespace fa {

namespace {

constexpr int kBQ = 128, kBK = 32, kThreads = 256;
constexpr int kWgs = 3;         // workgroups per CU
static_assert(kBQ == kB16FwdBq && kBK == kB16FwdBk, "forward tiling differs from kernels.h");

template <int D>
struct Bf16Fwd {
    static constexpr int DS = D / 32;          // 32-wide k-steps of S^T = K Q^T
    static constexpr int DT = D / 16;          // 16-row tiles of O^T
    static constexpr int NW = kThreads / 64;
    // K and V tiles with padded rows of D + 16 elements: the 16-byte K operand reads (16 rows
    // x 2 adjacent chunks per 32 lanes) and the V^T transpose reads (4 rows x 32 bytes per
    // 16 lanes) are then free of bank conflicts
    using PadT = Pad<D, 2>;
    static constexpr int ROWB = PadT::ROWB;
    static constexpr int PIECES = kBK * ROWB / 1024;          // 1 KB LDS-DMA pieces per tile
    static constexpr int KMAX = (PIECES + NW - 1) / NW;       // pieces per wave and tile (at most)
    static constexpr int TILEB = PIECES * 1024;
    static constexpr int STAGEB = 2 * TILEB;                  // K tile then V tile
    static_assert(PIECES * 1024 == kBK * ROWB, "tile must be whole pieces");
};

// LDS-DMA of key block jb into stage buffer `stage`: wave wu fills pieces wu, wu + NW, ... of
// the K tile and the same pieces of the V tile (same layout, so the same source offsets).
template <int D>
__device__ __forceinline__ void fwd_issue(const Buf& kb, const Buf& vb, const uint32_t* off,
                                          char* stage, int wu, uint32_t ld_bytes, int jb,
                                          int last) {
    using C = Bf16Fwd<D>;
    const int soff = __builtin_amdgcn_readfirstlane((int)((uint32_t)jb * kBK * ld_bytes));
    // pieces wu + i*NW exist for every wave except possibly the last one (last: this wave's
    // last piece exists; a wave-uniform value)
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i)
        if (i < C::KMAX - 1 || last) {
            dma_piece(kb, stage + (wu + i * C::NW) * 1024, off[i], soff);
            dma_piece(vb, stage + C::TILEB + (wu + i * C::NW) * 1024, off[i], soff);
        }
}

}  // namespace

// Loop-invariant values of one wave's walk over its key blocks.
template <int D>
struct FwdCtx {
    using C = Bf16Fwd<D>;
    Buf kbuf, vbuf;
    uint32_t off[C::KMAX];                   // LDS-DMA source offsets of this lane's pieces
    uint32_t kp;                             // K operand reads: stage-0 LDS address
    uint32_t vp;                             // V^T operand transpose reads: stage-0 address
    uint32_t ldk_b;                          // key row stride (bytes)
    int wu;                                  // wave index (uniform)
    int last;                                // this wave fills the last piece (uniform)
    int jhi, jf0, jf1;                       // block range end; FULL blocks [jf0, jf1)
    int T, Tk, wr0, window;
    bool cz;
    int g;                                   // lane row (lane / 16)
    int q[2];                                // this lane's two query rows
    int klo[2], kn[2];                       // keys each of them may see: [klo, klo + kn)
    float c;                                 // scale * log2(e)
    float inv8c;                             // 8 / c: rescale threshold above the running max
    __device__ __forceinline__ FwdCtx(const Buf& k, const Buf& v) : kbuf(k), vbuf(v) {}
};

// Online-softmax state of one wave: Q^T operands, O^T accumulators, and per query row (two
// per lane, tile qh) the running max m (raw score units), the rescale threshold thr = m + 8/c,
// m*c (clamped finite) and the lane's part of the running sum.
template <class E, int D>
struct FwdState {
    using C = Bf16Fwd<D>;
    typename E::v8 qreg[2][C::DS];
    f32x4 oacc[C::DT][2];
    float m[2], thr[2], mc[2], lsum[2];
};

// One key block j, staged in LDS stage STG (a compile-time constant, so every LDS address is
// a per-lane base plus an immediate offset).  Issues the next block's LDS-DMA into the other
// stage after the barrier.
template <class E, int D, int STG>
__device__ __forceinline__ void fwd_block(FwdState<E, D>& st, const FwdCtx<D>& x, char* sm,
                                          int j) {
    using C = Bf16Fwd<D>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    // scalar block test before the wait, only outside the FULL range
    int cls = kFull;
    if (j < x.jf0 || j >= x.jf1) {
        keep_branch();
        cls = block_class(x.T, x.Tk, x.wr0, x.wr0 + 32, j * kBK, j * kBK + kBK, x.cz, x.window);
    }
    wait_vmcnt<0>();   // block j's pieces, the only ones in flight
    // all pieces visible; every wave is done with the other stage (block j - 1)
    lds_barrier();
    if (j + 1 < x.jhi)
        fwd_issue<D>(x.kbuf, x.vbuf, x.off, sm + (STG ^ 1) * C::STAGEB, x.wu, x.ldk_b, j + 1, x.last);
    if (cls == kSkip) return;
    // S^T tiles [kt][qh]: entry r of lane (n, g) is key j*BK + 16*kt + 4g + r of query row
    // wr0 + 16*qh + n
    f32x4 s[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) s[kt][qh] = f32x4{0.f, 0.f, 0.f, 0.f};
    V8 ka[C::DS][2];
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
            ka[ds][kt] = lds_load<V8>(x.kp + STG * C::STAGEB + 16 * kt * C::ROWB + 64 * ds);
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) s[kt][qh] = mfma16x16x32(ka[ds][kt], st.qreg[qh][ds], s[kt][qh]);
    if (cls == kPartial) {
        keep_branch();
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k0 = j * kBK + 16 * kt + 4 * x.g + r;
                    if ((unsigned)(k0 - x.klo[qh]) >= (unsigned)x.kn[qh]) s[kt][qh][r] = -INFINITY;
                }
        }
    }
    // block max of each query row: three-input maxima over the lane's 8 entries, then the
    // other three 16-lane rows'
    float mx[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        const f32x4 &a = s[0][qh], &b = s[1][qh];
        const float t = vmax(vmax(vmax(a[0], a[1]), a[2]), vmax(vmax(a[3], b[0]), b[1]));
        mx[qh] = rows4_max(vmax(vmax(b[2], b[3]), t));
    }
    // lazy rescale: only when some row's block max passed its threshold (the first visible
    // key of a row always does: thr starts at -inf).  Otherwise the stale max keeps every
    // exp2 argument below 8.
    if (__any(mx[0] > st.thr[0] || mx[1] > st.thr[1])) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            const float mnew = vmax(st.m[qh], mx[qh]);
            const float corr = fast_exp2((st.m[qh] - mnew) * x.c);
            st.m[qh] = mnew;
            st.thr[qh] = mnew + x.inv8c;
            st.mc[qh] = vmax(mnew * x.c, kNegMax);   // finite even while m = -FLT_MAX
            st.lsum[qh] *= corr;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) st.oacc[dt][qh] *= corr;
        }
    }
    // P^T operand of query tile qh: element e is key 4g + e (e < 4) or 16 + 4g + e - 4, the
    // lane's own entries, in the key order of the V^T transpose reads
    V8 pb[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[kt][qh][r] = fast_exp2(fmaf(s[kt][qh][r], x.c, -st.mc[qh]));
        const f32x4 &a = s[0][qh], &b = s[1][qh];
        st.lsum[qh] += ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pb[qh][e] = (typename E::s)a[e];
            pb[qh][4 + e] = (typename E::s)b[e];
        }
    }
    // O^T += V^T P^T: the V^T operand of column tile dt (16 columns of V over the block's 32
    // keys) from two transpose reads.  At D = 128 the wave's priority is raised while it issues
    // these, so its MFMA chain is not interleaved with the other waves' softmax work (2-5%
    // faster; at D = 64, where the vector port is the limit, 2% slower).
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
        const uint32_t pv = x.vp + STG * C::STAGEB + 32 * dt;
        const V4 lo = lds_load_tr4<E>(pv);
        const V4 hi = lds_load_tr4<E>(pv + 16 * C::ROWB);
        V8 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            av[e] = lo[e];
            av[4 + e] = hi[e];
        }
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) st.oacc[dt][qh] = mfma16x16x32(av, pb[qh], st.oacc[dt][qh]);
    }
    if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
}

template <class E, int D>
__global__ __launch_bounds__(kThreads, kWgs) void fwd_b16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ L, int B,
    int T, int Tk, int H, int HKV, float scale, int causal, int window, int nqt, int xcd_group,
    Layout lq, Layout lk) {
    using C = Bf16Fwd<D>;
    using V8 = typename E::v8;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

    int qt, b, h;
    decode_q_work(blockIdx.x, nqt, B, H, HKV, xcd_group, qt, b, h);
    const int hk = h / (H / HKV);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)

    FwdCtx<D> x(head_buf<D>(K + b * lk.b + hk * lk.h, ldk, Tk),
                head_buf<D>(V + b * lk.b + hk * lk.h, ldk, Tk));
    x.wr0 = qt * kBQ + __builtin_amdgcn_readfirstlane(w) * 32;   // wave-uniform: scalar block tests
    x.ldk_b = (uint32_t)(ldk * 2);
    x.cz = causal != 0;
    x.T = T;
    x.Tk = Tk;
    x.window = window;
    x.g = g;
    x.c = scale * kLog2e;
    x.inv8c = 8.0f / x.c;
    x.q[0] = x.wr0 + n;
    x.q[1] = x.wr0 + 16 + n;
    row_keys(x.q[0], T, Tk, x.cz, window, x.klo[0], x.kn[0]);
    row_keys(x.q[1], T, Tk, x.cz, window, x.klo[1], x.kn[1]);

    FwdState<E, D> st;
    // Q^T operands: lane (n, g) holds Q[q][32*ds + 8g .. +7] of its two rows (zero past T)
    {
        const Buf qbuf = head_buf<D>(Q + b * lq.b + h * lq.h, ldq, T);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            const uint32_t off = (uint32_t)x.q[qh] * (uint32_t)(ldq * 2) + 16 * g;
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds)
                st.qreg[qh][ds] = __builtin_bit_cast(V8, qbuf.load16(off + ds * 64));
        }
    }
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) st.oacc[dt][qh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        st.m[qh] = kNegMax;
        st.thr[qh] = -INFINITY;
        st.mc[qh] = kNegMax;
        st.lsum[qh] = 0.f;
    }

    int jlo;
    kv_block_range(T, Tk, qt * kBQ, qt * kBQ + kBQ, kBK, x.cz, window, jlo, x.jhi);
    // key blocks that are FULL for this wave's rows
    full_kv_block_range(T, Tk, x.wr0, x.wr0 + 32, kBK, x.cz, window, x.jf0, x.jf1);

    // LDS-DMA source offsets of this lane in its wave's pieces of a K / V tile
    x.wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i) x.off[i] = dma_src_offset_padded<D, 2>(w + i * C::NW, lane, x.ldk_b);
    // LDS read bases inside a stage.  K operand: row n at byte 16g (k-steps 64 bytes apart,
    // key tiles 16 rows apart).  V^T operand: lane (j, g) addresses row 4g + j/4 at column
    // 4*(j%4) (column tiles 32 bytes apart; the second read 16 rows further).
    char* sm = reinterpret_cast<char*>(smem);
    x.kp = pinned_lds_addr(lds_addr(sm + n * C::ROWB + 16 * g));
    x.vp = pinned_lds_addr(lds_addr(sm + C::TILEB + (4 * g + (n >> 2)) * C::ROWB + 8 * (n & 3)));

    x.last = __builtin_amdgcn_readfirstlane((int)(x.wu + (C::KMAX - 1) * C::NW < C::PIECES));
    if (jlo < x.jhi) fwd_issue<D>(x.kbuf, x.vbuf, x.off, sm, x.wu, x.ldk_b, jlo, x.last);

    // blocks alternate between the two LDS stages: two per trip, stage 0 then stage 1
    int j = jlo;
    for (; j + 1 < x.jhi; j += 2) {
        fwd_block<E, D, 0>(st, x, sm, j);
        fwd_block<E, D, 1>(st, x, sm, j + 1);
    }
    if (j < x.jhi) fwd_block<E, D, 0>(st, x, sm, j);

    // the row sums over the four 16-lane rows; L and 1/l per query row
    float inv[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        const float lsum = rows4_sum(st.lsum[qh]);
        inv[qh] = lsum > 0.f ? 1.f / lsum : 0.f;
        if (g == 0 && x.q[qh] < T)
            L[((int64_t)b * H + h) * T + x.q[qh]] = lsum > 0.f ? st.m[qh] * scale + fast_log2(lsum) * kLn2 : 0.f;
    }
    // O leaves through LDS, so that every store instruction writes whole rows: each wave puts
    // its 32 x D tile, row-major, in its part of the two stages (free once every wave is past
    // its last block), then reads it back 16 bytes per lane, D/8 lanes per row.  Row stride
    // D + 8 elements: the 8-byte writes of 16 rows at 4 adjacent columns hit distinct banks.
    lds_barrier();
    constexpr uint32_t OROW = 2 * D + 16;
    static_assert(kThreads / 64 * 32 * OROW <= 2 * C::STAGEB, "O tiles must fit the stages");
    const uint32_t ot = lds_addr(sm) + (uint32_t)w * 32 * OROW;
    // tile (dt, qh), entry r of lane (n, g): O^T[16*dt + 4g + r][query row 16*qh + n]
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            u32x2 wv;
            wv[0] = pack2<E>(st.oacc[dt][qh][0] * inv[qh], st.oacc[dt][qh][1] * inv[qh]);
            wv[1] = pack2<E>(st.oacc[dt][qh][2] * inv[qh], st.oacc[dt][qh][3] * inv[qh]);
            *(__attribute__((address_space(3))) u32x2*)(ot + (16 * qh + n) * OROW + 2 * (16 * dt + 4 * g)) = wv;
        }
    // lane l: row RPI*i + l/LPR of the wave's 32, elements 8*(l%LPR) .. +7 (rows past T not stored)
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int RPI = 64 / LPR;               // rows per instruction
    const int rr = lane / LPR, ch = lane % LPR;
    uint16_t* Ow = O + b * lq.b + h * lq.h + 8 * ch;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = RPI * i + rr;
        const u32x4 v = lds_load<u32x4>(ot + row * OROW + 16 * ch);
        if (x.wr0 + row < T) *reinterpret_cast<u32x4*>(Ow + (int64_t)(x.wr0 + row) * ldq) = v;
    }
}

namespace {

template <class E, int D>
hipError_t launch_fwd_b16_t(const AttnArgs& a) {
    using C = Bf16Fwd<D>;
    const int nqt = (a.T + kBQ - 1) / kBQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    const int xcd_group = xcd_group_for(nqt, a.B, a.H, a.HKV);
    const size_t lds = 2 * C::STAGEB;
    static std::atomic<bool> attr_set[kMaxDeviceSlots];
    hipError_t e = allow_dynamic_lds((const void*)fwd_b16_kernel<E, D>, lds, attr_set);
    if (e != hipSuccess) return e;
    log_launch("fwd_b16_kernel", ElemName<E>::value, D, grid, kThreads, lds, a.B, a.T, a.Tk,
               a.H, a.HKV, a.causal, a.window);
    hipLaunchKernelGGL((fwd_b16_kernel<E, D>), dim3(grid), dim3(kThreads), lds, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.Oout, a.L, a.B, a.T, a.Tk, a.H, a.HKV, a.scale, a.causal,
                       a.window, nqt, xcd_group, a.lq, a.lk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_b16(const AttnArgs& a) {
    if (a.f16) {
        if (a.D == 64) return launch_fwd_b16_t<F16, 64>(a);
        if (a.D == 128) return launch_fwd_b16_t<F16, 128>(a);
    } else {
        if (a.D == 64) return launch_fwd_b16_t<Bf16, 64>(a);
        if (a.D == 128) return launch_fwd_b16_t<Bf16, 128>(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
