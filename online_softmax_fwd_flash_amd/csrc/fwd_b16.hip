// 16-bit forward attention for gfx950 (bf16 or fp16 I/O, D in {64, 128}): MFMA 32x32x16 with
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
//  * The K tile keeps padded rows (D + 8 elements: 16-byte operand-row reads of consecutive
//    rows at one chunk are free of bank conflicts; each row's pad slot gets a copy of a valid
//    chunk); the V tile is unpadded with XOR-swizzled 16-byte chunks for its transpose reads
//    (8 rows x 4 chunks per wave).
//  * Scores are formed transposed, S^T = K Q^T: the accumulator column (lane % 32) is a query
//    row, so each query's max / sum are in-lane plus one exchange between wave halves.
//  * P^T (rounded to the element type, RNE) feeds O^T += V^T P^T straight from the
//    accumulator registers.  The
//    accumulator gives lane half g the keys 8*(r/4) + 4g + r%4 of each 32-key group; the
//    V^T operand in that key order comes from the row-major V tile through two LDS
//    transpose reads (ds_read_b64_tr_b16) per MFMA, so V needs no transposed copy.
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
constexpr int kNH = kBK / 32;   // 32-key halves of a key block
constexpr int kWgs = 3;         // workgroups per CU
static_assert(kBQ == kB16FwdBq && kBK == kB16FwdBk, "forward tiling differs from kernels.h");

template <int D>
struct Bf16Fwd {
    static constexpr int DC = D / 16;          // 16-wide k-steps of S^T = K Q^T
    static constexpr int NDB = D / 32;         // 32-row blocks of O^T
    static constexpr int NW = kThreads / 64;
    // K tile padded (operand-row reads), V tile unpadded and swizzled (transpose reads)
    static constexpr int KROWB = Pad<D>::ROWB;
    static constexpr int VROWB = 2 * D;
    // LDS-DMA pieces of 1 KB (the K tile rounded up; slots past its last row take rows of
    // the next block, which nothing reads)
    static constexpr int KPIECES = (kBK * KROWB + 1023) / 1024;
    static constexpr int VPIECES = kBK * VROWB / 1024;
    static constexpr int KMAX = (KPIECES + NW - 1) / NW;      // K pieces per wave (at most)
    static constexpr int VPW = VPIECES / NW;                  // V pieces per wave
    static constexpr int KTILEB = KPIECES * 1024;
    static constexpr int STAGEB = KTILEB + VPIECES * 1024;    // K tile then V tile
    static_assert(VPW * NW == VPIECES, "V tile must split evenly over the waves");
};

// LDS-DMA of key block jb into stage buffer `stage`: wave wu fills K pieces wu, wu + NW, ...
// and V pieces [wu*VPW, +VPW).
template <int D>
__device__ __forceinline__ void fwd_issue(const Buf& kb, const Buf& vb, const uint32_t* koff,
                                          const uint32_t* voff, char* stage, int wu,
                                          uint32_t ld_bytes, int jb, int klast) {
    using C = Bf16Fwd<D>;
    const int soff = __builtin_amdgcn_readfirstlane((int)((uint32_t)jb * kBK * ld_bytes));
    // pieces wu + i*NW exist for every wave except possibly the last one (klast: this wave's
    // last piece exists; a wave-uniform value)
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i)
        if (i < C::KMAX - 1 || klast)
            dma_piece(kb, stage + (wu + i * C::NW) * 1024, koff[i], soff);
    char* vbase = stage + C::KTILEB + wu * C::VPW * 1024;
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) dma_piece(vb, vbase + i * 1024, voff[i], soff);
}

}  // namespace

// Loop-invariant values of one wave's walk over its key blocks.
template <int D>
struct FwdCtx {
    using C = Bf16Fwd<D>;
    Buf kbuf, vbuf;
    uint32_t koff[C::KMAX], voff[C::VPW];   // LDS-DMA source offsets of this lane's pieces
    uint32_t kp;                             // K operand reads: stage-0 LDS address
    uint32_t vp[C::NDB];                     // V^T operand transpose reads: stage-0 addresses
    uint32_t ldk_b;                          // key row stride (bytes)
    int wu;                                  // wave index (uniform)
    int klast;                               // this wave fills the last K piece (uniform)
    int jhi, jf0, jf1;                       // block range end; FULL blocks [jf0, jf1)
    int T, Tk, wr0, window;
    bool cz;
    int klo, kn;                             // keys this lane's query row sees
    int g;                                   // lane half
    float c;                                 // scale * log2(e)
    float inv8c;                             // 8 / c: rescale threshold above the running max
    __device__ __forceinline__ FwdCtx(const Buf& k, const Buf& v) : kbuf(k), vbuf(v) {}
};

// Online-softmax state of one wave: Q^T operands, O^T accumulators, and per query row the
// running max m (raw score units), the rescale threshold thr = m + 8/c, m*c (clamped finite)
// and the running sum.
template <class E, int D>
struct FwdState {
    using C = Bf16Fwd<D>;
    typename E::v8 qreg[C::DC];
    f32x16 oacc[C::NDB];
    float m, thr, mc, lsum;
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
        fwd_issue<D>(x.kbuf, x.vbuf, x.koff, x.voff, sm + (STG ^ 1) * C::STAGEB, x.wu, x.ldk_b,
                     j + 1, x.klast);
    if (cls == kSkip) return;
    // S^T for the block's 32-key halves: entry r of lane (n, g) in s[hk] is key
    // j*BK + 32*hk + 8*(r/4) + 4g + r%4 of query n
    f32x16 s[kNH];
#pragma unroll
    for (int hk = 0; hk < kNH; ++hk)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[hk][r] = 0.f;
    V8 ka[C::DC][kNH];
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk)
            ka[dc][hk] = lds_load<V8>(x.kp + STG * C::STAGEB + 32 * dc + 32 * hk * C::KROWB);
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk) s[hk] = mfma32x32x16(ka[dc][hk], st.qreg[dc], s[hk]);
    // schedule: the first DC K reads up front, then one read per MFMA, so the LDS
    // latency hides behind the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, C::DC, 0);
#pragma unroll
    for (int i = 0; i < (kNH * C::DC) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, (kNH * C::DC) / 2, 0);
    if (cls == kPartial) {
        keep_branch();
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int k0 = j * kBK + 32 * hk + 8 * (r >> 2) + 4 * x.g + (r & 3);
                if ((unsigned)(k0 - x.klo) >= (unsigned)x.kn) s[hk][r] = -INFINITY;
            }
    }
    // block max of each query row: three-input maxima over the lane's 16 * kNH entries, then
    // the other wave half's
    float mx;
    {
        float t[kNH];
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk) {
            const f32x16& v = s[hk];
            const float a0 = vmax(vmax(v[0], v[1]), v[2]), a1 = vmax(vmax(v[3], v[4]), v[5]);
            const float a2 = vmax(vmax(v[6], v[7]), v[8]), a3 = vmax(vmax(v[9], v[10]), v[11]);
            const float a4 = vmax(vmax(v[12], v[13]), v[14]);
            t[hk] = vmax(vmax(vmax(a0, a1), a2), vmax(vmax(a3, a4), v[15]));
        }
        mx = t[0];
#pragma unroll
        for (int hk = 1; hk < kNH; ++hk) mx = vmax(mx, t[hk]);
    }
    mx = halves_max(mx);
    // lazy rescale: only when some row's block max passed its threshold (the first visible
    // key of a row always does: thr starts at -inf).  Otherwise the stale max keeps every
    // exp2 argument below 8.
    if (__any(mx > st.thr)) {
        const float mnew = vmax(st.m, mx);
        const float corr = fast_exp2((st.m - mnew) * x.c);
        st.m = mnew;
        st.thr = mnew + x.inv8c;
        st.mc = vmax(mnew * x.c, kNegMax);   // finite even while m = -FLT_MAX
        st.lsum *= corr;
#pragma unroll
        for (int i = 0; i < C::NDB; ++i) st.oacc[i] *= corr;
    }
    float ps[kNH];
#pragma unroll
    for (int hk = 0; hk < kNH; ++hk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[hk][r] = fast_exp2(fmaf(s[hk][r], x.c, -st.mc));
        // pairwise sum: a dependency chain of 4 adds instead of 16
        float t4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t4[i] = (s[hk][i] + s[hk][4 + i]) + (s[hk][8 + i] + s[hk][12 + i]);
        ps[hk] = (t4[0] + t4[1]) + (t4[2] + t4[3]);
    }
#pragma unroll
    for (int hk = 0; hk < kNH; ++hk) st.lsum += ps[hk];
    // P^T operand of 16-key quarter kh: element e <-> accumulator entry 8*(kh % 2) + e of
    // s[kh / 2]
    V8 pb[2 * kNH];
#pragma unroll
    for (int kh = 0; kh < 2 * kNH; ++kh)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kh][e] = (typename E::s)s[kh >> 1][8 * (kh & 1) + e];
#pragma unroll
    for (int kh = 0; kh < 2 * kNH; ++kh)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
            const uint32_t pv = x.vp[db] + STG * C::STAGEB + 16 * kh * C::VROWB;
            const V4 lo = lds_load_tr4<E>(pv);
            const V4 hi = lds_load_tr4<E>(pv + 8 * C::VROWB);
            V8 av;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                av[e] = lo[e];
                av[4 + e] = hi[e];
            }
            st.oacc[db] = mfma32x32x16(av, pb[kh], st.oacc[db]);
        }
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
    const int n = lane & 31, g = lane >> 5;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)

    FwdCtx<D> x(head_buf<D>(K + b * lk.b + hk * lk.h, ldk, Tk),
                head_buf<D>(V + b * lk.b + hk * lk.h, ldk, Tk));
    x.wr0 = qt * kBQ + __builtin_amdgcn_readfirstlane(w) * 32;   // wave-uniform: scalar block tests
    const int q = x.wr0 + n;
    x.ldk_b = (uint32_t)(ldk * 2);
    x.cz = causal != 0;
    x.T = T;
    x.Tk = Tk;
    x.window = window;
    x.g = g;
    x.c = scale * kLog2e;
    x.inv8c = 8.0f / x.c;
    // keys this query row may see: [klo, klo + kn)
    row_keys(q, T, Tk, x.cz, window, x.klo, x.kn);

    FwdState<E, D> st;
    // Q^T operand: lane (n, g) holds Q[q][16*dc + 8*g .. +7] (zero past T)
    {
        const Buf qbuf = head_buf<D>(Q + b * lq.b + h * lq.h, ldq, T);
        const uint32_t off = (uint32_t)q * (uint32_t)(ldq * 2) + 16 * g;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
            st.qreg[dc] = __builtin_bit_cast(V8, qbuf.load16(off + dc * 32));
    }
#pragma unroll
    for (int i = 0; i < C::NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[i][r] = 0.f;
    st.m = kNegMax;
    st.thr = -INFINITY;
    st.mc = kNegMax;
    st.lsum = 0.f;

    int jlo;
    kv_block_range(T, Tk, qt * kBQ, qt * kBQ + kBQ, kBK, x.cz, window, jlo, x.jhi);
    // key blocks that are FULL for this wave's rows
    full_kv_block_range(T, Tk, x.wr0, x.wr0 + 32, kBK, x.cz, window, x.jf0, x.jf1);

    // LDS-DMA source offsets of this lane in its wave's pieces of a K / V tile
    x.wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i) x.koff[i] = dma_src_offset_padded<D>(w + i * C::NW, lane, x.ldk_b);
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) x.voff[i] = dma_src_offset_swz<D>(w * C::VPW + i, lane, x.ldk_b);
    // LDS read offsets inside a stage.  K operand: rows n and 32 + n, chunk 2*dc + g (padded
    // rows: consecutive k-steps are 32 bytes apart).  V^T operand via transpose reads: lane
    // 16*cq + jj reads 8 bytes of row 16*kh + 4*(cq/2) + jj/4 (and 8 rows further) at
    // column 32*db + 16*(cq%2) + 4*(jj%4).
    char* sm = reinterpret_cast<char*>(smem);
    x.kp = pinned_lds_addr(lds_addr(sm + n * C::KROWB + 16 * g));
    {
        const int jj = lane & 15, cq = lane >> 4;
        const int vr = 4 * (cq >> 1) + (jj >> 2);
        const int vx = Swz<D>::v(vr) >> 2;
        const int lo2 = 2 * (cq & 1) + ((jj & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
            x.vp[db] = pinned_lds_addr(lds_addr(sm + C::KTILEB + vr * C::VROWB +
                                                16 * (4 * (db ^ vx) + lo2) + 8 * (jj & 1)));
    }

    x.klast = __builtin_amdgcn_readfirstlane((int)(x.wu + (C::KMAX - 1) * C::NW < C::KPIECES));
    if (jlo < x.jhi) fwd_issue<D>(x.kbuf, x.vbuf, x.koff, x.voff, sm, x.wu, x.ldk_b, jlo, x.klast);

    // blocks alternate between the two LDS stages: two per trip, stage 0 then stage 1
    int j = jlo;
    for (; j + 1 < x.jhi; j += 2) {
        fwd_block<E, D, 0>(st, x, sm, j);
        fwd_block<E, D, 1>(st, x, sm, j + 1);
    }
    if (j < x.jhi) fwd_block<E, D, 0>(st, x, sm, j);

    float lsum = st.lsum + swap_halves(st.lsum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (g == 0 && q < T)
        L[((int64_t)b * H + h) * T + q] = lsum > 0.f ? st.m * scale + fast_log2(lsum) * kLn2 : 0.f;
    // O leaves through LDS, so that every store instruction writes whole rows: each wave puts
    // its 32 x D tile, row-major, in its quarter of the two stages (free once every wave is
    // past its last block), then reads it back 16 bytes per lane, 16 lanes per row.  Row
    // stride D + 8 elements: the 8-byte writes of 32 rows at one column hit distinct banks.
    lds_barrier();
    constexpr uint32_t OROW = 2 * D + 16;
    static_assert(kThreads / 64 * 32 * OROW <= 2 * C::STAGEB, "O tiles must fit the stages");
    const uint32_t ot = lds_addr(sm) + (uint32_t)w * 32 * OROW;
    // lane (n, g), entry r of block db: O^T[db*32 + 8*(r/4) + 4g + r%4][query n]
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            u32x2 wv;
            wv[0] = pack2<E>(st.oacc[db][4 * t4 + 0] * inv, st.oacc[db][4 * t4 + 1] * inv);
            wv[1] = pack2<E>(st.oacc[db][4 * t4 + 2] * inv, st.oacc[db][4 * t4 + 3] * inv);
            *(__attribute__((address_space(3))) u32x2*)(ot + n * OROW + 2 * (db * 32 + 8 * t4 + 4 * g)) = wv;
        }
    // lane l: row 4i + l/16 of the wave's 32, elements 8*(l%16) .. +7 (rows past T not stored)
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
