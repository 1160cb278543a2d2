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
                                          uint32_t ld_bytes, int jb) {
    using C = Bf16Fwd<D>;
    const int soff = __builtin_amdgcn_readfirstlane((int)((uint32_t)jb * kBK * ld_bytes));
    // pieces wu + i*NW exist for every wave except possibly the last one
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i)
        if (i < C::KMAX - 1 || wu + i * C::NW < C::KPIECES)
            dma_piece(kb, stage + (wu + i * C::NW) * 1024, koff[i], soff);
    char* vbase = stage + C::KTILEB + wu * C::VPW * 1024;
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) dma_piece(vb, vbase + i * 1024, voff[i], soff);
}

}  // namespace

template <class E, int D>
__global__ __launch_bounds__(kThreads, kWgs) void fwd_b16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ L, int B,
    int T, int Tk, int H, int HKV, float scale, int causal, int window, int nqt, int xcd_group,
    Layout lq, Layout lk) {
    using C = Bf16Fwd<D>;
    using V8 = typename E::v8;
    using V4 = typename E::v4;
    extern __shared__ __attribute__((aligned(1024))) uint16_t smem[];

    int qt, b, h;
    decode_q_work(blockIdx.x, nqt, B, H, HKV, xcd_group, qt, b, h);
    const int hk = h / (H / HKV);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int wr0 = qt * kBQ + __builtin_amdgcn_readfirstlane(w) * 32;   // wave-uniform: scalar block tests
    const int q = wr0 + n;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)
    const uint32_t ldk_b = (uint32_t)(ldk * 2);
    const Buf kbuf = head_buf<D>(K + b * lk.b + hk * lk.h, ldk, Tk);
    const Buf vbuf = head_buf<D>(V + b * lk.b + hk * lk.h, ldk, Tk);
    const bool cz = causal != 0;
    const float c = scale * kLog2e;
    // keys this query row may see: [klo, klo + kn)
    int klo, kn;
    row_keys(q, T, Tk, cz, window, klo, kn);

    // Q^T operand: lane (n, g) holds Q[q][16*dc + 8*g .. +7] (zero past T)
    V8 qreg[C::DC];
    {
        const Buf qbuf = head_buf<D>(Q + b * lq.b + h * lq.h, ldq, T);
        const uint32_t off = (uint32_t)q * (uint32_t)(ldq * 2) + 16 * g;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) qreg[dc] = __builtin_bit_cast(V8, qbuf.load16(off + dc * 32));
    }
    f32x16 oacc[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m = kNegMax, lsum = 0.f;

    int jlo, jhi;
    kv_block_range(T, Tk, qt * kBQ, qt * kBQ + kBQ, kBK, cz, window, jlo, jhi);
    int jf0, jf1;   // key blocks that are FULL for this wave's rows
    full_kv_block_range(T, Tk, wr0, wr0 + 32, kBK, cz, window, jf0, jf1);

    // LDS-DMA source offsets of this lane in its wave's pieces of a K / V tile
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t koff[C::KMAX], voff[C::VPW];
#pragma unroll
    for (int i = 0; i < C::KMAX; ++i) koff[i] = dma_src_offset_padded<D>(w + i * C::NW, lane, ldk_b);
#pragma unroll
    for (int i = 0; i < C::VPW; ++i) voff[i] = dma_src_offset_swz<D>(w * C::VPW + i, lane, ldk_b);
    // LDS read offsets inside a stage.  K operand: rows n and 32 + n, chunk 2*dc + g (padded
    // rows: consecutive k-steps are 32 bytes apart).  V^T operand via transpose reads: lane
    // 16*cq + jj reads 8 bytes of row 16*kh + 4*(cq/2) + jj/4 (and 8 rows further) at
    // column 32*db + 16*(cq%2) + 4*(jj%4).
    const uint32_t kaddr = (uint32_t)(n * C::KROWB + 16 * g);
    uint32_t vaddr[C::NDB];
    {
        const int jj = lane & 15, cq = lane >> 4;
        const int vr = 4 * (cq >> 1) + (jj >> 2);
        const int vx = Swz<D>::v(vr) >> 2;
        const int lo2 = 2 * (cq & 1) + ((jj & 3) >> 1);
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
            vaddr[db] = (uint32_t)(C::KTILEB + vr * C::VROWB + 16 * (4 * (db ^ vx) + lo2) +
                                   8 * (jj & 1));
    }

    char* sm = reinterpret_cast<char*>(smem);
    if (jlo < jhi) fwd_issue<D>(kbuf, vbuf, koff, voff, sm, wu, ldk_b, jlo);

    for (int j = jlo; j < jhi; ++j) {
        const int stg = (j - jlo) & 1;
        // scalar block test before the wait, only outside the FULL range
        int cls = kFull;
        if (j < jf0 || j >= jf1) {
            keep_branch();
            cls = block_class(T, Tk, wr0, wr0 + 32, j * kBK, j * kBK + kBK, cz, window);
        }
        wait_vmcnt<0>();   // block j's pieces, the only ones in flight
        // all pieces visible; every wave is done with the other stage (block j - 1)
        lds_barrier();
        if (j + 1 < jhi) fwd_issue<D>(kbuf, vbuf, koff, voff, sm + (stg ^ 1) * C::STAGEB, wu, ldk_b, j + 1);
        if (cls == kSkip) continue;
        const char* sb = sm + stg * C::STAGEB;
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
                ka[dc][hk] = *reinterpret_cast<const V8*>(sb + kaddr + 32 * dc + 32 * hk * C::KROWB);
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
            for (int hk = 0; hk < kNH; ++hk) s[hk] = mfma32x32x16(ka[dc][hk], qreg[dc], s[hk]);
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
                    const int k0 = j * kBK + 32 * hk + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((unsigned)(k0 - klo) >= (unsigned)kn) s[hk][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = vmax(mx, vmax(s[hk][r], s[hk][r + 1]));
        mx = halves_max(mx);
        const float mnew = vmax(m, mx);
        // a row whose max is still the -FLT_MAX start rescales on its first visible key
        // (bitwise operators: one vector-compare sequence, no branches)
        if (__any((mnew > m) & ((m == kNegMax) | ((mnew - m) * c > 8.0f)))) {
            const float corr = fast_exp2((m - mnew) * c);
            m = mnew;
            lsum *= corr;
#pragma unroll
            for (int i = 0; i < C::NDB; ++i) oacc[i] *= corr;
        }
        const float mc = vmax(m * c, kNegMax);   // finite even while m = -FLT_MAX
        float ps[kNH];
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[hk][r] = fast_exp2(fmaf(s[hk][r], c, -mc));
            // pairwise sum: a dependency chain of 4 adds instead of 16
            float t4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) t4[i] = (s[hk][i] + s[hk][4 + i]) + (s[hk][8 + i] + s[hk][12 + i]);
            ps[hk] = (t4[0] + t4[1]) + (t4[2] + t4[3]);
        }
#pragma unroll
        for (int hk = 0; hk < kNH; ++hk) lsum += ps[hk];
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
                const char* pv = sb + vaddr[db] + 16 * kh * C::VROWB;
                const V4 lo = lds_read_tr4e<E>(reinterpret_cast<const uint16_t*>(pv));
                const V4 hi = lds_read_tr4e<E>(reinterpret_cast<const uint16_t*>(pv + 8 * C::VROWB));
                V8 av;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[e] = lo[e];
                    av[4 + e] = hi[e];
                }
                oacc[db] = mfma32x32x16(av, pb[kh], oacc[db]);
            }
    }

    lsum += swap_halves(lsum);
    if (q >= T) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t* Oq = O + b * lq.b + (int64_t)q * ldq + h * lq.h;
    // lane (n, g), entry r of block db: O^T[db*32 + 8*(r/4) + 4g + r%4][query n]
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            u32x2 wv;
            wv[0] = pack2<E>(oacc[db][4 * t4 + 0] * inv, oacc[db][4 * t4 + 1] * inv);
            wv[1] = pack2<E>(oacc[db][4 * t4 + 2] * inv, oacc[db][4 * t4 + 3] * inv);
            *reinterpret_cast<u32x2*>(Oq + db * 32 + 8 * t4 + 4 * g) = wv;
        }
    if (g == 0)
        L[((int64_t)b * H + h) * T + q] = lsum > 0.f ? m * scale + fast_log2(lsum) * kLn2 : 0.f;
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
