// bf16 forward attention for gfx950 (D in {64, 128}): bf16 MFMA 32x32x16 with fp32
// accumulation, online softmax in registers, O and one log-sum-exp per query row stored.
//
// Method (prior art, other hardware): forge "flash_attention.metal", header comment and the
// forward kernel (online-softmax update, m from -FLT_MAX, K/V staged per block through
// on-chip memory, causal key bound, window block skip, diagonal-only mask, l == 0 guard);
// Graphcore "flash_attention_qkv_packed.cpp", flashAttentionQKVPackedWithStash (block skip /
// mask conditions, L = m + log l stash).
//
// gfx950 design
//  * Workgroup = 4 waves = 128 query rows of one (b, h); wave w owns 32 rows.  Key blocks of
//    64 are double-buffered in LDS (one barrier per block); the next block's global loads are
//    issued before the current block's MFMAs so their latency hides behind them.
//  * Scores are formed transposed, S^T = K Q^T: the accumulator column (lane % 32) is a query
//    row, so each query's max / sum are in-lane plus one exchange between wave halves.
//  * P^T (bf16, RNE) feeds O^T += V^T P^T straight from the accumulator registers.  The
//    accumulator gives lane half g the keys 8*(r/4) + 4g + r%4 of each 32-key group; the
//    V^T operand in that key order comes from the row-major V tile through two LDS
//    transpose reads (ds_read_b64_tr_b16) per MFMA, so V needs no transposed copy.
//  * The running max is rescaled lazily: O and l are only rescaled when some row's max grew
//    by more than 2^8 (the stale max keeps every exp2 argument below 8, so nothing overflows
//    and the final O / l and L = m*scale + ln l are exact up to rounding).
//  * Work order: longest key ranges (last query tiles) first; with GQA the query heads of one
//    KV head are placed on the same XCD (workgroup ids congruent mod 8) at the same time so
//    they share its K/V in that XCD's L2.
#include "common.h"
#include "kernels.h"
#include "stage_bf16.h"

namespace fa {

namespace {

constexpr int kBQ = 128, kBK = 64, kThreads = 256;
static_assert(kBQ == kBf16FwdBq && kBK == kBf16FwdBk, "forward tiling differs from kernels.h");

template <int D>
struct Bf16Fwd {
    static constexpr int DC = D / 16;          // 16-wide k-steps of S^T = K Q^T
    static constexpr int NDB = D / 32;         // 32-row blocks of O^T
    // Both tiles row-major [key][d].  K rows are read 16 bytes per lane, 32 rows per
    // half-wave: an odd stride in 16-byte units (D + 8 elements) is conflict-free on the
    // 128-bank LDS.  V is read through transpose reads of 8 rows x 16 dwords per wave: a
    // stride of 16 x odd dwords (D + 32 elements) is conflict-free.
    using KTile = RowChunks<kBK, D, kThreads, D + 8>;
    using VTile = RowChunks<kBK, D, kThreads, D + 32>;
    static constexpr int KLD = KTile::LDN;
    static constexpr int VLD = VTile::LDN;
    static constexpr int KBUF = kBK * KLD;
    static constexpr int VBUF = kBK * VLD;
    static constexpr int BUF = KBUF + VBUF;    // one stage, bf16 elements
};

template <int D>
struct Stage {
    typename Bf16Fwd<D>::KTile k;
    typename Bf16Fwd<D>::VTile v;
    __device__ __forceinline__ void load(const Buf& kb, const Buf& vb, uint32_t ld_bytes, int j) {
        k.load(kb, ld_bytes, j * kBK);
        v.load(vb, ld_bytes, j * kBK);
    }
    __device__ __forceinline__ void store(uint16_t* buf) const {
        k.store(buf);
        v.store(buf + Bf16Fwd<D>::KBUF);
    }
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ L, int B,
    int T, int H, int HKV, float scale, int causal, int window, int nqt, int xcd_group) {
    using C = Bf16Fwd<D>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    int qt, b, h;
    decode_q_work(blockIdx.x, nqt, B, H, HKV, xcd_group, qt, b, h);
    const int hk = h / (H / HKV);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int wr0 = qt * kBQ + w * 32;
    const int q = wr0 + n;
    const int64_t ldq = (int64_t)H * D, ldk = (int64_t)HKV * D;
    const uint32_t ldk_b = (uint32_t)(ldk * 2);
    const Buf kbuf = rows_buf(K + (int64_t)b * T * ldk + (int64_t)hk * D, ldk, T);
    const Buf vbuf = rows_buf(V + (int64_t)b * T * ldk + (int64_t)hk * D, ldk, T);
    const bool cz = causal != 0;
    const float c = scale * kLog2e;
    // keys this query row may see: [klo, khi]
    const int klo = window > 0 ? q - window + 1 : 0;
    const int khi = cz ? q : T - 1;

    // Q^T operand: lane (n, g) holds Q[q][16*dc + 8*g .. +7] (zero past T)
    bf16x8 qreg[C::DC];
    {
        const Buf qbuf = rows_buf(Q + (int64_t)b * T * ldq + (int64_t)h * D, ldq, T);
        const uint32_t off = (uint32_t)q * (uint32_t)(ldq * 2) + 16 * g;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) qreg[dc] = __builtin_bit_cast(bf16x8, qbuf.load16(off + dc * 32));
    }
    f32x16 oacc[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
    float m = kNegMax, lsum = 0.f;

    int jlo, jhi;
    kv_block_range(T, qt * kBQ, qt * kBQ + kBQ, kBK, cz, window, jlo, jhi);

    Stage<D> st;
    if (jlo < jhi) {
        st.load(kbuf, vbuf, ldk_b, jlo);
        st.store(smem);
    }
    __syncthreads();

    for (int j = jlo; j < jhi; ++j) {
        const uint16_t* buf = smem + ((j - jlo) & 1) * C::BUF;
        const bool more = j + 1 < jhi;
        const int cls = block_class(T, wr0, wr0 + 32, j * kBK, j * kBK + kBK, cz, window);
        if (cls != kSkip) {
            const uint16_t* Ks = buf;
            const uint16_t* Vs = buf + C::KBUF;
            f32x16 s0, s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
            for (int dc = 0; dc < C::DC; ++dc) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(Ks + n * C::KLD + dc * 16 + 8 * g);
                const bf16x8 a1 =
                    *reinterpret_cast<const bf16x8*>(Ks + (32 + n) * C::KLD + dc * 16 + 8 * g);
                s0 = mfma32x32x16(a0, qreg[dc], s0);
                s1 = mfma32x32x16(a1, qreg[dc], s1);
            }
            // next block's K/V global loads fly while this block's softmax and P V run
            if (more) st.load(kbuf, vbuf, ldk_b, j + 1);
            if (cls == kPartial) {
                // entry r of lane (n, g): key j*64 + 32*half + 8*(r/4) + 4g + r%4
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int k0 = j * kBK + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((unsigned)(k0 - klo) > (unsigned)(khi - klo)) s0[r] = -INFINITY;
                    if ((unsigned)(k0 + 32 - klo) > (unsigned)(khi - klo)) s1[r] = -INFINITY;
                }
            }
            float mx = vmax(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = vmax(mx, vmax(s0[r], s1[r]));
            mx = vmax(mx, swap_halves(mx));
            const float mnew = vmax(m, mx);
            // a row whose max is still the -FLT_MAX start rescales on its first visible key
            if (__any(mnew > m && (m == kNegMax || (mnew - m) * c > 8.0f))) {
                const float corr = fast_exp2((m - mnew) * c);
                m = mnew;
                lsum *= corr;
#pragma unroll
                for (int i = 0; i < C::NDB; ++i) oacc[i] *= corr;
            }
            const float mc = vmax(m * c, kNegMax);   // finite even while m = -FLT_MAX
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s0[r] = fast_exp2(fmaf(s0[r], c, -mc));
                s1[r] = fast_exp2(fmaf(s1[r], c, -mc));
                ps0 += s0[r];
                ps1 += s1[r];
            }
            lsum += ps0 + ps1;
            // P^T operand: 8 keys per 16-key half, element e <-> accumulator entry 8*half + e
            bf16x8 pb[4];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pb[hf][e] = (__bf16)s0[8 * hf + e];
                    pb[2 + hf][e] = (__bf16)s1[8 * hf + e];
                }
#pragma unroll
            for (int kh = 0; kh < 4; ++kh)
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const bf16x8 a = tr_operand32<C::VLD>(Vs, 16 * kh, 32 * db, lane);
                    oacc[db] = mfma32x32x16(a, pb[kh], oacc[db]);
                }
        } else if (more) {
            st.load(kbuf, vbuf, ldk_b, j + 1);
        }
        if (more) st.store(smem + ((j + 1 - jlo) & 1) * C::BUF);
        __syncthreads();
    }

    lsum += swap_halves(lsum);
    if (q >= T) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint16_t* Oq = O + ((int64_t)b * T + q) * ldq + (int64_t)h * D;
    // lane (n, g), entry r of block db: O^T[db*32 + 8*(r/4) + 4g + r%4][query n]
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            u32x2 wv;
            wv[0] = pack_bf16x2(oacc[db][4 * t4 + 0] * inv, oacc[db][4 * t4 + 1] * inv);
            wv[1] = pack_bf16x2(oacc[db][4 * t4 + 2] * inv, oacc[db][4 * t4 + 3] * inv);
            *reinterpret_cast<u32x2*>(Oq + db * 32 + 8 * t4 + 4 * g) = wv;
        }
    if (g == 0)
        L[((int64_t)b * H + h) * T + q] = lsum > 0.f ? m * scale + fast_log2(lsum) * kLn2 : 0.f;
}

namespace {

template <int D>
hipError_t launch_fwd_bf16_t(const AttnArgs& a) {
    using C = Bf16Fwd<D>;
    const int nqt = (a.T + kBQ - 1) / kBQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    const int xcd_group = xcd_group_for(nqt, a.B, a.H, a.HKV);
    const size_t lds = 2 * C::BUF * sizeof(uint16_t);
    static bool attr_set[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!attr_set[dev]) {
        e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set[dev] = true;
    }
    hipLaunchKernelGGL((fwd_bf16_kernel<D>), dim3(grid), dim3(kThreads), lds, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (uint16_t*)a.Oout, a.L, a.B, a.T, a.H, a.HKV, a.scale, a.causal,
                       a.window, nqt, xcd_group);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const AttnArgs& a) {
    if (a.D == 64) return launch_fwd_bf16_t<64>(a);
    if (a.D == 128) return launch_fwd_bf16_t<128>(a);
    return hipErrorInvalidValue;
}

}  // namespace fa
