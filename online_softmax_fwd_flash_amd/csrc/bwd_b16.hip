// 16-bit backward attention for gfx950 (bf16 or fp16 I/O, D in {64, 128}): a dK/dV pass and a
// separate dQ pass on MFMA with fp32 accumulation; P is recomputed from the stored
// log-sum-exp, never stored.
// Gradients are written once, in fp32, without atomics, so results are deterministic.
//
// Method (prior art, other hardware): forge "flash_attention.metal", backward section and the
// kernels flash_attn_bwd_dq / flash_attn_bwd_dv / flash_attn_bwd_dk (P = exp(s*scale - L),
// dS = P (dP - D), dQ / dK carry one factor of scale, dK / dV summed over a KV head's query
// heads, key-owned accumulation without atomics, window bounds of the query loop);
// teeny-kernels "flash_attn2.rs", backward_dq and backward_dkv doc comments (the same
// formulas); Graphcore "flash_attention_qkv_packed.cpp", flashAttentionQKVPackedGrad
// (key-chunk-outer loop with dV += P^T dO, dP = dO V^T, dS, dK += dS^T Q).
//
// dK/dV pass (16x16x32 MFMA).  Workgroup = 4 waves x 32 keys of one (b, kv head), two
// workgroups per CU; it walks every (query head of the group, 32-row query block) pair that
// sees its keys, last query block first.  Q, dO (row-major, padded rows) and L, D of a block
// reach LDS by LDS-DMA, double-buffered.  S = Q K^T and dP = dO V^T keep a key per
// accumulator column, so P and dS leave the accumulators already in the A-operand layout of
// dV += P^T dO and dK += dS^T Q; the B operands of those (dO and Q with rows in the
// accumulator's order) come from the row-major tiles through LDS transpose reads.
//
// In both passes the dP accumulators start at D of their query rows (dK/dV: with -V as the
// operand, so the MFMAs leave D - dP; dQ: at -D, leaving dP - D), so dS = P (dP - D) costs one
// multiply per score; the per-block class test runs only outside each wave's precomputed range
// of FULL blocks, and the diagonal mask is a branch.
//
// dQ pass (16x16x32 MFMA; on N(0, 1) operands the chip sustains about a third more FLOP/s on
// this shape than on 32x32x16 under its power limit).  Workgroup = 4 waves x 32 query rows
// (two 16-row tiles per wave) of one (b, h), two workgroups per CU at D = 128, walking its key
// blocks of 64; K and V reach LDS by LDS-DMA (padded rows, double-buffered).  S^T = K Q^T and
// dP^T = V dO^T keep a query per accumulator column, so L and D are per-lane values and each
// lane's dS^T entries of two stacked 16-key tiles form its B operand of dQ^T += K^T dS^T
// directly; the K^T operand comes from the same K tile through transpose reads in that key
// order.
#include "common.h"
#include "kernels.h"
#include "stage_b16.h"

namespace fa {

namespace {

constexpr float kBigLse = 3.0e38f;   // L of a padding row: exp2(s*c - big) = 0

}  // namespace

// ------------------------------------------------------------------------------ dK / dV
// 16x16x32 MFMAs: S = Q K^T puts 16 keys on the accumulator columns and 4 query rows per lane,
// so P and dS of two 16-row blocks concatenate into the A operand of dV += P^T dO and
// dK += dS^T Q (32 query rows per k-step), whose B operands come from the same row-major
// Q / dO tiles through LDS transpose reads.
namespace {

// The staged (query head, query block) pair: Q and dO tiles of 32 rows, and their L and D.
template <int D>
struct DkdvStage {
    static constexpr int NW = 4, NT = 256;
    static constexpr int BQ = 32;                     // query rows per staged block
    static constexpr int QB16 = BQ / 16, KKS = BQ / 32;   // 16-row blocks, 32-row k-steps
    static constexpr int DS = D / 32;                 // 32-wide k-steps of S and dP
    static constexpr int NDB = D / 16;                // 16-wide column blocks of dK / dV
    // Padded row (elements).  Row-major Q / dO tiles serve both operand reads: 16-byte reads
    // of 16 rows x 2 column groups per half-wave (A of S, dP) and 8-byte transpose reads of
    // 16 rows x 8 dwords per wave (B of dV, dK); both are conflict-free at a row stride of
    // D + 16 elements.  The tiles reach LDS by LDS-DMA (the pad slots get copies).
    using PadT = Pad<D, 2>;
    static constexpr int LDN = PadT::ROWB / 2;
    static constexpr int TPIECES = BQ * PadT::ROWB / 1024;   // 1 KB pieces per tile
    static constexpr int OFF_DO = TPIECES * 1024;             // bytes
    static constexpr int OFF_L = 2 * OFF_DO;                  // 64 floats of L, then 64 of D
    static constexpr int STAGE = OFF_L + 2 * 256;             // bytes per stage
    static constexpr int QW = NW / 2;                         // waves per tile
    static constexpr int PMAX = (TPIECES + QW - 1) / QW;      // pieces per wave (at most)
    static_assert(TPIECES * 1024 == BQ * PadT::ROWB, "tile must be whole pieces");
};

// LDS-DMA of the stage of query block i2 of head h2 (the group's h2-th query head) into
// buffer `buf`.  The first half of the waves fill the Q tile (pieces w, w + NW/2, ...),
// the second half the dO tile; wave 0 also moves the block's L values, wave 1 its D values.
// Q / dO rows reach LDS through one descriptor for the whole KV group when the group's heads
// lie inside each row (row stride >= (rep - 1) * head stride + D, as in [B, T, H, D]): rows
// past T are then beyond its end for every head.  Otherwise ([B, H, T, D]: the next head
// follows row T - 1) each block gets a descriptor of its own head's rows.
struct QdoSrc {
    Buf q, o;                    // group descriptors (grp)
    const uint16_t *Qg, *dOg;    // first head of the group
    int64_t ldq, qh;             // row and head strides (elements)
    bool grp;
};

template <int D>
__device__ __forceinline__ void dkdv_issue(char* sm, const QdoSrc& qs, const float* Lg,
                                             const float* Dg, const uint32_t* voff, int w,
                                             int h2, int i2, int T, int buf) {
    using C = DkdvStage<D>;
    char* st = sm + buf * C::STAGE;
    const uint32_t rows = (uint32_t)i2 * C::BQ * (uint32_t)(qs.ldq * 2);
    const int tso = __builtin_amdgcn_readfirstlane(
        (int)(qs.grp ? rows + (uint32_t)(h2 * qs.qh * 2) : rows));
    const int wq = w % C::QW;
    char* dst = st + (w / C::QW) * C::OFF_DO;
    const Buf src = qs.grp ? (w < C::QW ? qs.q : qs.o)
                           : head_buf<D>((w < C::QW ? qs.Qg : qs.dOg) + h2 * qs.qh, qs.ldq, T);
    // pieces wq + QW*i exist for every wave except possibly the last one
#pragma unroll
    for (int i = 0; i < C::PMAX; ++i)
        if (i < C::PMAX - 1 || wq + C::QW * i < C::TPIECES)
            dma_piece(src, dst + (wq + C::QW * i) * 1024, voff[i], tso);
    if (w < 2) {
        const int rso = __builtin_amdgcn_readfirstlane(i2 * C::BQ * 4);
        // rows past T read as 0
        const Buf rb(w == 0 ? Lg + (int64_t)h2 * T : Dg + (int64_t)h2 * T, (uint32_t)T * 4u);
        dma_dwords(rb, st + C::OFF_L + w * 256, voff[C::PMAX], rso);
    }
}

}  // namespace

// Workgroup = 4 waves x 32 keys (two 16-key halves per wave) of one (b, kv head), two
// workgroups per CU.  Every A operand read from the Q / dO tiles and every transpose-read B
// operand of dV / dK feeds both key halves, so a wave moves about 40% fewer LDS bytes per MFMA
// than with 16 keys per wave (measured 16% faster at B=4 H=32 HKV=8 T=4096 D=128 than 16 keys
// per wave at three workgroups per CU), and the workgroup stages each Q / dO block for 128
// keys (half the barriers and L2 -> LDS traffic per FLOP).  K of the wave's keys stays in
// registers; -V of the workgroup's 128 keys is staged in LDS once (negated while staged), the
// B operand of D - dP = D - dO V^T; the dK and dV accumulators take 128 registers per wave.
namespace {

template <int D>
struct DkdvCfg : DkdvStage<D> {
    using Base = DkdvStage<D>;
    static constexpr int KH = 2;                          // 16-key halves per wave
    static constexpr int KPW = 16 * KH, BKW = Base::NW * KPW;
    // workgroups per CU: at D = 64 the registers (168) and LDS (41 KB) allow three
    static constexpr int WGS = D == 64 ? 3 : 2;
    // column blocks of the dV / dK products whose B operands are read before the softmax
    // arithmetic, which then hides the reads' latency (more would spill at D = 128)
    static constexpr int HOIST = D == 128 ? 2 : 4;
    static constexpr int VOFF = 2 * Base::STAGE;          // -V tile: BKW rows, padded
    static constexpr int LDS = VOFF + BKW * Base::PadT::ROWB;
};

template <int D>
struct DkdvCtx {
    using C = DkdvCfg<D>;
    QdoSrc qs;
    const float *Lg, *Dg;
    uint32_t voff[C::PMAX + 1];
    // per-lane LDS read bases in stage 0 (the dO tile is OFF_DO after the Q tile): A-operand
    // row n at column 8g; transpose-read row 4g + j/4 at column 4*(j%4) (j = lane % 16); L / D
    // of rows 4g .. 4g + 3 (D 256 bytes after L)
    uint32_t aq, tr, ld;
    uint32_t va;           // -V operand reads: row w*32 + n of the -V tile at column 8g
    int w, rep, niter, if0, if1, T, Tk, kw0, window, g;
    int qlo[C::KH], qn[C::KH];   // query rows that see this lane's key of each half
    bool cz;
    float c;
    __device__ __forceinline__ DkdvCtx(const QdoSrc& q) : qs(q) {}
};

template <class E, int D>
struct DkdvState {
    using C = DkdvCfg<D>;
    typename E::v8 kreg[C::KH][C::DS];
    f32x4 dka[C::KH][C::NDB], dva[C::KH][C::NDB];
};

// One (query head h2, query block i) pair, staged in LDS stage STG (a compile-time constant:
// every LDS address is a pinned per-lane base plus an immediate offset).  (h2n, in) is the
// pair after it, whose LDS-DMA goes into the other stage after the barrier.
//
// The dP accumulators start at +D with -V as operand, so the MFMAs leave D - dP; P (D - dP)
// is then -dS and dK accumulates -dS^T Q, negated again (with the scale) at the store.  Each
// negation is exact, so the stored dK equals the one from dS itself bit for bit.
template <class E, int D, int STG>
__device__ __forceinline__ void dkdv_block(DkdvState<E, D>& st, const DkdvCtx<D>& x, char* sm,
                                           int it, int i, int h2n, int in) {
    using C = DkdvCfg<D>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    using S16 = typename E::s;
    const int qr0 = i * C::BQ;
    int cls = kFull;
    if (i < x.if0 || i >= x.if1) {
        keep_branch();
        cls = block_class(x.T, x.Tk, qr0, qr0 + C::BQ, x.kw0, x.kw0 + C::KPW, x.cz, x.window);
    }
    wait_vmcnt<0>();   // this stage's pieces, the only loads in flight
    // every wave's pieces are visible; every wave is done with the other stage
    lds_barrier();
    if (it + 1 < x.niter) dkdv_issue<D>(sm, x.qs, x.Lg, x.Dg, x.voff, x.w, h2n, in, x.T, STG ^ 1);
    if (cls == kSkip) return;
    constexpr uint32_t SO = STG * C::STAGE;
    // S and D - dP of both key halves; entry r of lane (n, g): row 16qb + 4g + r, key 16h + n
    f32x4 sc[C::KH][C::QB16], dp[C::KH][C::QB16];
#pragma unroll
    for (int qb = 0; qb < C::QB16; ++qb) {
        const f32x4 d4 = lds_load<f32x4>(x.ld + SO + 256 + qb * 64);
#pragma unroll
        for (int h = 0; h < C::KH; ++h) {
            sc[h][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[h][qb] = d4;
        }
    }
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
        V8 aq[C::QB16], ao[C::QB16], vb[C::KH];
#pragma unroll
        for (int qb = 0; qb < C::QB16; ++qb) {
            const uint32_t off = SO + 2 * (qb * 16 * C::LDN + ds * 32);
            aq[qb] = lds_load<V8>(x.aq + off);
            ao[qb] = lds_load<V8>(x.aq + C::OFF_DO + off);
        }
#pragma unroll
        for (int h = 0; h < C::KH; ++h) vb[h] = lds_load<V8>(x.va + 2 * (16 * h * C::LDN + ds * 32));
#pragma unroll
        for (int qb = 0; qb < C::QB16; ++qb)
#pragma unroll
            for (int h = 0; h < C::KH; ++h) {
                sc[h][qb] = mfma16x16x32(aq[qb], st.kreg[h][ds], sc[h][qb]);
                dp[h][qb] = mfma16x16x32(ao[qb], vb[h], dp[h][qb]);
            }
    }
    auto tr_b = [&](int kk, int db, V8& bo, V8& bq) {
        const uint32_t off = SO + 2 * (32 * kk * C::LDN + 16 * db);
        const V4 ol = lds_load_tr4<E>(x.tr + C::OFF_DO + off);
        const V4 oh = lds_load_tr4<E>(x.tr + C::OFF_DO + off + 32 * C::LDN);
        const V4 ql = lds_load_tr4<E>(x.tr + off);
        const V4 qh = lds_load_tr4<E>(x.tr + off + 32 * C::LDN);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bo[e] = ol[e];
            bo[4 + e] = oh[e];
            bq[e] = ql[e];
            bq[4 + e] = qh[e];
        }
    };
    V8 bo[4], bq[4];
#pragma unroll
    for (int u = 0; u < C::HOIST; ++u) tr_b(0, u, bo[u], bq[u]);
    // rows past T have L = D = 0 and zero Q / dO: they add nothing
#pragma unroll
    for (int qb = 0; qb < C::QB16; ++qb) {
        const f32x4 l4 = lds_load<f32x4>(x.ld + SO + qb * 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ml = -l4[r] * kLog2e;
#pragma unroll
            for (int h = 0; h < C::KH; ++h) sc[h][qb][r] = fast_exp2(fmaf(sc[h][qb][r], x.c, ml));
        }
    }
    if (cls == kPartial) {
        keep_branch();
#pragma unroll
        for (int h = 0; h < C::KH; ++h)
#pragma unroll
            for (int qb = 0; qb < C::QB16; ++qb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int qi = qr0 + qb * 16 + 4 * x.g + r;
                    if ((unsigned)(qi - x.qlo[h]) >= (unsigned)x.qn[h]) sc[h][qb][r] = 0.f;
                }
    }
    V8 pp[C::KH], pd[C::KH];
#pragma unroll
    for (int h = 0; h < C::KH; ++h)
#pragma unroll
        for (int qb = 0; qb < C::QB16; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pp[h][4 * qb + r] = (S16)sc[h][qb][r];
                pd[h][4 * qb + r] = (S16)(sc[h][qb][r] * dp[h][qb][r]);   // -dS
            }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int d0 = 0; d0 < C::NDB; d0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (d0 > 0 || u >= C::HOIST) tr_b(0, d0 + u, bo[u], bq[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int h = 0; h < C::KH; ++h) {
                st.dva[h][d0 + u] = mfma16x16x32(pp[h], bo[u], st.dva[h][d0 + u]);
                st.dka[h][d0 + u] = mfma16x16x32(pd[h], bq[u], st.dka[h][d0 + u]);
            }
    }
    __builtin_amdgcn_s_setprio(0);
}

}  // namespace

template <class E, int D>
__global__ __launch_bounds__(256, DkdvCfg<D>::WGS) void dkdv_b16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ L, const float* __restrict__ Dv, float* __restrict__ dK,
    float* __restrict__ dV, int B, int T, int Tk, int H, int HKV, float scale, int causal,
    int window, Layout lq, Layout lk, int g16) {
    using C = DkdvCfg<D>;
    using V8 = typename E::v8;
    static_assert(C::BQ == 32 && C::KKS == 1, "one 32-row k-step per query block");
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
    char* sm = reinterpret_cast<char*>(smem);

    // longest query ranges (first key blocks under causal) first
    const int BG = B * HKV;
    const int kt = (int)(blockIdx.x / BG);
    const int bg = blockIdx.x % BG;
    const int b = bg / HKV, hk = bg % HKV, rep = H / HKV;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int n = lane & 15, g = lane >> 4;
    const int kw0 = kt * C::BKW + w * C::KPW;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)

    // -V of the workgroup's keys into LDS, row-major with padded rows (zeros past Tk)
    {
        const Buf vb = head_buf<D>(V + b * lk.b + hk * lk.h, ldk, Tk);
        constexpr int CPR = D / 8;   // 16-byte chunks per row
        const u32x4 sign = {0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
#pragma unroll
        for (int e = threadIdx.x; e < C::BKW * CPR; e += 256) {
            const int r = e / CPR, ch = e % CPR;
            const u32x4 v = vb.load16((uint32_t)(kt * C::BKW + r) * (uint32_t)(ldk * 2) + 16 * ch) ^ sign;
            *(__attribute__((address_space(3))) u32x4*)(lds_addr(sm) + C::VOFF + r * C::PadT::ROWB + 16 * ch) = v;
        }
    }

    const uint32_t ldq_b = (uint32_t)(ldq * 2);
    const uint16_t* Qg = Q + b * lq.b + (int64_t)hk * rep * lq.h;
    const uint16_t* dOg = dO + b * lq.b + (int64_t)hk * rep * lq.h;
    const uint32_t gspan = (uint32_t)(((int64_t)(rep - 1) * lq.h + (int64_t)(T - 1) * ldq + D) * 2);
    DkdvCtx<D> x(QdoSrc{Buf(Qg, gspan), Buf(dOg, gspan), Qg, dOg, ldq, lq.h,
                          ldq >= (int64_t)(rep - 1) * lq.h + D});
    x.Lg = L + ((int64_t)b * H + (int64_t)hk * rep) * T;
    x.Dg = Dv + ((int64_t)b * H + (int64_t)hk * rep) * T;
    x.w = w;
    x.rep = rep;
    x.T = T;
    x.Tk = Tk;
    x.kw0 = kw0;
    x.window = window;
    x.g = g;
    x.cz = causal != 0;
    x.c = scale * kLog2e;
#pragma unroll
    for (int h = 0; h < C::KH; ++h) key_rows(kw0 + 16 * h + n, T, Tk, x.cz, window, x.qlo[h], x.qn[h]);

    DkdvState<E, D> st;
    {
        const Buf kb = head_buf<D>(K + b * lk.b + hk * lk.h, ldk, Tk);
#pragma unroll
        for (int h = 0; h < C::KH; ++h) {
            const uint32_t off = (uint32_t)(kw0 + 16 * h + n) * (uint32_t)(ldk * 2) + 16 * g;
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds)
                st.kreg[h][ds] = __builtin_bit_cast(V8, kb.load16(off + ds * 64));
        }
    }
#pragma unroll
    for (int h = 0; h < C::KH; ++h)
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) st.dka[h][i] = st.dva[h][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    int ilo, ihi;
    q_block_range(T, Tk, kt * C::BKW, kt * C::BKW + C::BKW, C::BQ, x.cz, window, ilo, ihi);
    full_q_block_range(T, Tk, kw0, kw0 + C::KPW, C::BQ, x.cz, window, x.if0, x.if1);
    x.niter = rep * (ihi - ilo);
#pragma unroll
    for (int i = 0; i < C::PMAX; ++i)
        x.voff[i] = dma_src_offset_padded<D, 2>(w % C::QW + C::QW * i, lane, ldq_b);
    x.voff[C::PMAX] = 4u * (uint32_t)lane;
    {
        const int j = lane & 15;
        x.aq = pinned_lds_addr(lds_addr(sm + 2 * (n * C::LDN + 8 * g)));
        x.tr = pinned_lds_addr(lds_addr(sm + 2 * ((4 * g + (j >> 2)) * C::LDN + 4 * (j & 3))));
        x.ld = pinned_lds_addr(lds_addr(sm + C::OFF_L + 16 * g));
        x.va = pinned_lds_addr(lds_addr(sm + C::VOFF + (w * C::KPW + n) * C::PadT::ROWB + 16 * g));
    }
    __syncthreads();   // the -V tile is complete

    // (query head, query block) pairs, heads innermost.  Under causal masking the first half
    // of the key tiles walks its query blocks from the last one down and the second half from
    // its first one up.  Workgroups start in key-tile order, the first half at once and each
    // later one on the slot an earlier one frees (tile nkt - 1 - k after tile k, which sees as
    // many fewer blocks as the later one sees more), on the XCD of its (b, kv head) group.  So
    // at any moment the first-half tiles of a group read the same query block, and so do its
    // second-half tiles, which shares each block through that XCD's L2.
    const int nkt = (Tk + C::BKW - 1) / C::BKW;
    const int di = (x.cz && 2 * kt >= nkt) ? 1 : -1;
    int h2n = 0, in = di > 0 ? ilo : ihi - 1;
    if (x.niter > 0) dkdv_issue<D>(sm, x.qs, x.Lg, x.Dg, x.voff, w, h2n, in, T, 0);
    int it = 0;
    for (; it + 1 < x.niter; it += 2) {
        int i = in;
        if (++h2n == rep) {
            h2n = 0;
            in += di;
        }
        dkdv_block<E, D, 0>(st, x, sm, it, i, h2n, in);
        i = in;
        if (++h2n == rep) {
            h2n = 0;
            in += di;
        }
        dkdv_block<E, D, 1>(st, x, sm, it + 1, i, h2n, in);
    }
    if (it < x.niter) {
        const int i = in;
        if (++h2n == rep) {
            h2n = 0;
            in += di;
        }
        dkdv_block<E, D, 0>(st, x, sm, it, i, h2n, in);
    }

    // entry r of lane (n, g) in block db of half h: key kw0 + 16h + 4g + r, column db*16 + n.
    // dka holds -dK / scale.  Stored as float32, or (g16) rounded to the element type.
    const float nscale = -scale;
    const int64_t kbase = b * lk.b + hk * lk.h;
#pragma unroll
    for (int h = 0; h < C::KH; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kk = kw0 + 16 * h + 4 * g + r;
            if (kk < Tk) {
                const int64_t row = kbase + (int64_t)kk * ldk + n;
                if (g16) {
                    typename E::s* dKh = reinterpret_cast<typename E::s*>(dK) + row;
                    typename E::s* dVh = reinterpret_cast<typename E::s*>(dV) + row;
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) {
                        dKh[db * 16] = (typename E::s)opaque(st.dka[h][db][r] * nscale);
                        dVh[db * 16] = (typename E::s)opaque(st.dva[h][db][r]);
                    }
                } else {
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) {
                        dK[row + db * 16] = st.dka[h][db][r] * nscale;
                        dV[row + db * 16] = st.dva[h][db][r];
                    }
                }
            }
        }
}

// ------------------------------------------------------------------------------ dQ
namespace {

template <int D, int NW>
struct DqCfg {
    static constexpr int NT = NW * 64;
    static constexpr int BQ = NW * 32;   // NW waves x 32 query rows
    static constexpr int BK = 64;        // keys per staged block
    static constexpr int DS = D / 32;    // 32-column k-steps of S^T and dP^T
    static constexpr int DT = D / 16;    // 16-column tiles of dQ^T
    // Row-major K and V tiles with padded rows of D + 16 elements (LDS-DMA fills the pad
    // slots with copies).  K and V are read 16 bytes per lane as A operands of S^T and dP^T
    // (16 consecutive rows at four consecutive 16-byte chunks), and K through transpose reads
    // as the A operand of dQ^T += K^T dS^T (4 rows x 32 bytes per 16 lanes): at this stride
    // neither has LDS bank conflicts (measured; D + 8 and D + 24 give 3 conflict cycles per
    // LDS instruction).
    using PadT = Pad<D, 2>;
    static constexpr int LDN = PadT::ROWB / 2;                // elements per row
    static constexpr int TPIECES = BK * PadT::ROWB / 1024;    // 1 KB pieces per tile
    static constexpr int OFF_V = TPIECES * 1024;              // bytes
    static constexpr int STAGE = 2 * OFF_V;                   // bytes per stage
    static constexpr int TW = NW / 2;                         // waves per tile
    static constexpr int PMAX = (TPIECES + TW - 1) / TW;      // pieces per wave (at most)
    static_assert(TPIECES * 1024 == BK * PadT::ROWB, "tile must be whole pieces");
};

// LDS-DMA of key block jb into stage buffer `st`: the first half of the waves fill the K
// tile (pieces w, w + NW/2, ...), the second half the V tile.
template <int D, int NW>
__device__ __forceinline__ void dq_issue(char* st, const Buf& kbuf, const Buf& vbuf,
                                         const uint32_t* voff, int w, uint32_t ldk_b, int jb) {
    using C = DqCfg<D, NW>;
    const int soff = __builtin_amdgcn_readfirstlane((int)((uint32_t)jb * C::BK * ldk_b));
    const int wt = w % C::TW;
    char* dst = st + (w / C::TW) * C::OFF_V;
    const Buf& src = w < C::TW ? kbuf : vbuf;
    // pieces wt + TW*i exist for every wave except possibly the last one
#pragma unroll
    for (int i = 0; i < C::PMAX; ++i)
        if (i < C::PMAX - 1 || wt + C::TW * i < C::TPIECES)
            dma_piece(src, dst + (wt + C::TW * i) * 1024, voff[i], soff);
}

}  // namespace

template <class E, int D, int NW, bool FUSE_D>
__global__ __launch_bounds__(NW * 64, 8 / NW) void dq_b16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ L, float* __restrict__ Dv,
    float* __restrict__ dQ, int B, int T, int Tk, int H, int HKV, float scale, int causal,
    int window, int nqt, int xcd_group, Layout lq, Layout lk, int g16) {
    using C = DqCfg<D, NW>;
    using V8 = typename E::v8;
    using S16 = typename E::s;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];
    char* sm = reinterpret_cast<char*>(smem);

    int qt, b, h;
    decode_q_work(blockIdx.x, nqt, B, H, HKV, xcd_group, qt, b, h);
    const int hk = h / (H / HKV);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int n = lane & 15, g = lane >> 4;
    const int wr0 = qt * C::BQ + w * 32;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)
    const uint32_t ldk_b = (uint32_t)(ldk * 2);
    const Buf kbuf = head_buf<D>(K + b * lk.b + hk * lk.h, ldk, Tk);
    const Buf vbuf = head_buf<D>(V + b * lk.b + hk * lk.h, ldk, Tk);
    const bool cz = causal != 0;
    const float c = scale * kLog2e;

    // the wave's 32 query rows are two 16-row tiles: lane (n, g) holds query rows wr0 + n and
    // wr0 + 16 + n, and qrow is each one's element offset in Q, O, dO and dQ
    int qq[2];
    int64_t qrow[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        qq[qh] = wr0 + 16 * qh + n;
        qrow[qh] = b * lq.b + (int64_t)qq[qh] * ldq + h * lq.h;
    }

    // B operands of S^T = K Q^T and dP^T = V dO^T: lane (n, g) holds Q / dO[q][32*ds + 8g ..]
    V8 qreg[2][C::DS], oreg[2][C::DS];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const int64_t at = qrow[qh] + ds * 32 + 8 * g;
            qreg[qh][ds] = __builtin_bit_cast(V8, qq[qh] < T ? *reinterpret_cast<const u32x4*>(Q + at) : z);
            oreg[qh][ds] = __builtin_bit_cast(V8, qq[qh] < T ? *reinterpret_cast<const u32x4*>(dO + at) : z);
        }
    float l2[2], dq_i[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
        l2[qh] = qq[qh] < T ? L[((int64_t)b * H + h) * T + qq[qh]] * kLog2e : kBigLse;
    if constexpr (FUSE_D) {
        // D_i = sum_d dO[i][d] O[i][d]: this lane's 8*DS columns, then the other three 16-lane
        // rows' (rows past T load zeros and give 0)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            float s = 0.f;
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds) {
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 o = qq[qh] < T ? *reinterpret_cast<const u32x4*>(O + qrow[qh] + ds * 32 + 8 * g) : z;
                s = dot8<E>(o, __builtin_bit_cast(u32x4, oreg[qh][ds]), s);
            }
            dq_i[qh] = rows4_sum(s);
            if (g == 0 && qq[qh] < T) Dv[((int64_t)b * H + h) * T + qq[qh]] = dq_i[qh];
        }
    } else {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) dq_i[qh] = qq[qh] < T ? Dv[((int64_t)b * H + h) * T + qq[qh]] : 0.f;
    }
    // keys each query row may see: [klo, klo + kn)
    int klo[2], kn[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) row_keys(qq[qh], T, Tk, cz, window, klo[qh], kn[qh]);
    // dQ^T accumulators: tile (dt, qh), entry r of lane (n, g): column 16*dt + 4g + r of query
    // row wr0 + 16*qh + n
    f32x4 dqa[C::DT][2];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) dqa[dt][qh] = f32x4{0.f, 0.f, 0.f, 0.f};

    int jlo, jhi;
    kv_block_range(T, Tk, qt * C::BQ, qt * C::BQ + C::BQ, C::BK, cz, window, jlo, jhi);
    int jf0, jf1;   // key blocks that are FULL for this wave's rows
    full_kv_block_range(T, Tk, wr0, wr0 + 32, C::BK, cz, window, jf0, jf1);
    uint32_t voff[C::PMAX];
#pragma unroll
    for (int i = 0; i < C::PMAX; ++i)
        voff[i] = dma_src_offset_padded<D, 2>(w % C::TW + C::TW * i, lane, ldk_b);

    if (jlo < jhi) dq_issue<D, NW>(sm, kbuf, vbuf, voff, w, ldk_b, jlo);
    for (int j = jlo; j < jhi; ++j) {
        const int stg = (j - jlo) & 1;
        // scalar block test before the wait, only outside the FULL range
        int cls = kFull;
        if (j < jf0 || j >= jf1) {
            keep_branch();
            cls = block_class(T, Tk, wr0, wr0 + 32, j * C::BK, j * C::BK + C::BK, cz, window);
        }
        wait_vmcnt<0>();   // block j's pieces, the only loads in flight
        // every wave's pieces are visible; every wave is done with the other stage
        lds_barrier();
        if (j + 1 < jhi) dq_issue<D, NW>(sm + (stg ^ 1) * C::STAGE, kbuf, vbuf, voff, w, ldk_b, j + 1);
        if (cls == kSkip) continue;
        const uint16_t* Kn = reinterpret_cast<const uint16_t*>(sm + stg * C::STAGE);
        const uint16_t* Vn = reinterpret_cast<const uint16_t*>(sm + stg * C::STAGE + C::OFF_V);
        // the two 32-key halves in turn: S^T and dP^T, the softmax arithmetic, then dQ^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // tiles [kt][qh] of S^T and dP^T: entry r of lane (n, g) is key
            // j*64 + 32*kb + 16*kt + 4g + r, query row wr0 + 16*qh + n.  dP^T starts at -D of
            // its query row, so the MFMAs leave dP^T - D.
            f32x4 sk[2][2], dk[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int qh = 0; qh < 2; ++qh) {
                    sk[kt][qh] = f32x4{0.f, 0.f, 0.f, 0.f};
                    dk[kt][qh] = f32x4{-dq_i[qh], -dq_i[qh], -dq_i[qh], -dq_i[qh]};
                }
            // A operands: 16 key rows of K / V at one 32-column k-step, 16 bytes per lane
#pragma unroll
            for (int ds = 0; ds < C::DS; ++ds) {
                V8 ak[2], av[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const int off = (kb * 32 + kt * 16 + n) * C::LDN + ds * 32 + 8 * g;
                    ak[kt] = *reinterpret_cast<const V8*>(Kn + off);
                    av[kt] = *reinterpret_cast<const V8*>(Vn + off);
                }
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int qh = 0; qh < 2; ++qh) {
                        sk[kt][qh] = mfma16x16x32(ak[kt], qreg[qh][ds], sk[kt][qh]);
                        dk[kt][qh] = mfma16x16x32(av[kt], oreg[qh][ds], dk[kt][qh]);
                    }
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sk[kt][qh][r] = fast_exp2(fmaf(sk[kt][qh][r], c, -l2[qh]));
            if (cls == kPartial) {
                keep_branch();
#pragma unroll
                for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int kk = j * C::BK + 32 * kb + 16 * kt + 4 * g + r;
                            if ((unsigned)(kk - klo[qh]) >= (unsigned)kn[qh]) sk[kt][qh][r] = 0.f;
                        }
            }
            // B operand of dQ^T += K^T dS^T for query tile qh: element e is key 32*kb + 4g + e
            // (e < 4) or 32*kb + 16 + 4g + e - 4, the lane's own entries
            V8 pd[2];
#pragma unroll
            for (int qh = 0; qh < 2; ++qh)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) pd[qh][4 * kt + r] = (S16)(sk[kt][qh][r] * dk[kt][qh][r]);
            // A operands K^T (16 columns of K over the same 32 keys) through transpose reads,
            // four column tiles at a time
#pragma unroll
            for (int dt0 = 0; dt0 < C::DT; dt0 += 4) {
                V8 at[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) at[u] = tr_operand16<E, C::LDN>(Kn, kb * 32, (dt0 + u) * 16, lane);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int qh = 0; qh < 2; ++qh) dqa[dt0 + u][qh] = mfma16x16x32(at[u], pd[qh], dqa[dt0 + u][qh]);
            }
        }
    }

    // tile (dt, qh) entry r: dQ[wr0 + 16*qh + n][16*dt + 4g + r]; float32, or (g16) rounded to
    // the element type.  One store instruction writes 64 contiguous bytes of each of 16 rows.
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        if (qq[qh] >= T) continue;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = dqa[dt][qh][r] * scale;
            const int64_t at = qrow[qh] + dt * 16 + 4 * g;
            if (g16) {
                u32x2 hv;
                hv[0] = pack2<E>(opaque(o[0]), opaque(o[1]));
                hv[1] = pack2<E>(opaque(o[2]), opaque(o[3]));
                *reinterpret_cast<u32x2*>(reinterpret_cast<S16*>(dQ) + at) = hv;
            } else {
                *reinterpret_cast<f32x4*>(dQ + at) = o;
            }
        }
    }
}

// ------------------------------------------------------------------------------ launchers
namespace {

template <class E, int D>
hipError_t launch_dkdv_b16_t(const AttnArgs& a) {
    using C = DkdvCfg<D>;
    static std::atomic<bool> set[kMaxDeviceSlots];
    const size_t lds = (size_t)C::LDS;
    hipError_t e = allow_dynamic_lds((const void*)dkdv_b16_kernel<E, D>, lds, set);
    if (e != hipSuccess) return e;
    const int nkt = (a.Tk + C::BKW - 1) / C::BKW;
    const unsigned grid = (unsigned)nkt * a.B * a.HKV;
    log_launch("dkdv_b16_kernel", ElemName<E>::value, D, grid, C::NT, lds, a.B, a.T, a.Tk, a.H,
               a.HKV, a.causal, a.window);
    hipLaunchKernelGGL((dkdv_b16_kernel<E, D>), dim3(grid), dim3(C::NT), lds, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, a.Lin, a.Dvec, a.dK, a.dV, a.B, a.T, a.Tk, a.H, a.HKV,
                       a.scale, a.causal, a.window, a.lq, a.lk, a.g16);
    return hipGetLastError();
}

constexpr int kDqWaves = 4;
static_assert(DqCfg<128, kDqWaves>::BQ == kB16DqBq && DqCfg<128, kDqWaves>::BK == kB16DqBk,
              "dQ tiling differs from kernels.h");
static_assert(DkdvCfg<128>::BQ == kB16DkdvBq && DkdvCfg<128>::BKW == kB16DkdvBk,
              "dK/dV tiling differs from kernels.h");

template <class E, int D, bool FUSE_D>
hipError_t launch_dq_b16_t(const AttnArgs& a) {
    using C = DqCfg<D, kDqWaves>;
    static std::atomic<bool> set[kMaxDeviceSlots];
    const size_t lds = 2 * (size_t)C::STAGE;
    hipError_t e = allow_dynamic_lds((const void*)dq_b16_kernel<E, D, kDqWaves, FUSE_D>, lds, set);
    if (e != hipSuccess) return e;
    const int nqt = (a.T + C::BQ - 1) / C::BQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    log_launch(FUSE_D ? "dq_b16_kernel(+Dvec)" : "dq_b16_kernel", ElemName<E>::value, D, grid,
               C::NT, lds, a.B, a.T, a.Tk, a.H, a.HKV, a.causal, a.window);
    hipLaunchKernelGGL((dq_b16_kernel<E, D, kDqWaves, FUSE_D>), dim3(grid), dim3(C::NT), lds,
                       a.stream, (const uint16_t*)a.Q, (const uint16_t*)a.K,
                       (const uint16_t*)a.V, (const uint16_t*)a.dO, (const uint16_t*)a.O, a.Lin,
                       a.Dvec, a.dQ, a.B, a.T, a.Tk, a.H, a.HKV, a.scale, a.causal, a.window, nqt,
                       xcd_group_for(nqt, a.B, a.H, a.HKV), a.lq, a.lk, a.g16);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dkdv_b16(const AttnArgs& a) {
    if (a.D == 64) return a.f16 ? launch_dkdv_b16_t<F16, 64>(a) : launch_dkdv_b16_t<Bf16, 64>(a);
    if (a.D == 128) return a.f16 ? launch_dkdv_b16_t<F16, 128>(a) : launch_dkdv_b16_t<Bf16, 128>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_dq_b16(const AttnArgs& a) {
    if (a.D == 64) return a.f16 ? launch_dq_b16_t<F16, 64, false>(a) : launch_dq_b16_t<Bf16, 64, false>(a);
    if (a.D == 128) return a.f16 ? launch_dq_b16_t<F16, 128, false>(a) : launch_dq_b16_t<Bf16, 128, false>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_dq_b16_fused_d(const AttnArgs& a) {
    if (a.O == nullptr) return hipErrorInvalidValue;
    if (a.D == 64) return a.f16 ? launch_dq_b16_t<F16, 64, true>(a) : launch_dq_b16_t<Bf16, 64, true>(a);
    if (a.D == 128) return a.f16 ? launch_dq_b16_t<F16, 128, true>(a) : launch_dq_b16_t<Bf16, 128, true>(a);
    return hipErrorInvalidValue;
}

}  // namespace fa
