// bf16 backward attention for gfx950 (D in {64, 128}): a dK/dV pass and a separate dQ pass,
// both on bf16 MFMA 32x32x16 with fp32 accumulation; P is recomputed from the stored
// log-sum-exp, never stored.  Gradients are written once, in fp32, without atomics, so
// results are deterministic.
//
// Method (prior art, other hardware): forge "flash_attention.metal", backward section and the
// kernels flash_attn_bwd_dq / flash_attn_bwd_dv / flash_attn_bwd_dk (P = exp(s*scale - L),
// dS = P (dP - D), dQ / dK carry one factor of scale, dK / dV summed over a KV head's query
// heads, key-owned accumulation without atomics, window bounds of the query loop);
// teeny-kernels "flash_attn2.rs", backward_dq and backward_dkv doc comments (the same
// formulas); Graphcore "flash_attention_qkv_packed.cpp", flashAttentionQKVPackedGrad
// (key-chunk-outer loop with dV += P^T dO, dP = dO V^T, dS, dK += dS^T Q).
//
// dK/dV pass.  Workgroup = NW waves x 32 keys of one (b, kv head); it walks every
// (query head of the group, 64-row query block) pair that sees its keys, Q / dO staged in
// LDS both row-major (operand of S = Q K^T and dP = dO V^T) and transposed (operand of
// dV += P^T dO and dK += dS^T Q, rows permuted to match the accumulator layout of P / dS).
// K and V of the wave's 32 keys stay in registers.  S = Q K^T puts the wave's keys on the
// accumulator columns, so P and dS leave the accumulator already in the layout the next two
// MFMAs take as their A operand.
//
// dQ pass.  Workgroup = 8 waves x 32 query rows of one (b, h) walking its key blocks of 64;
// K row-major and transposed plus V row-major in LDS.  S^T = K Q^T and dP^T = V dO^T keep a
// query per accumulator column, so L and D are per-lane scalars and dS^T feeds
// dQ^T += K^T dS^T directly, as P^T feeds O^T in the forward.
#include "common.h"
#include "kernels.h"
#include "stage_bf16.h"

namespace fa {

namespace {

constexpr float kBigLse = 3.0e38f;   // L of a padding row: exp2(s*c - big) = 0

// ------------------------------------------------------------------------------ dK / dV
template <int D, int NW>
struct DkdvCfg {
    static constexpr int NT = NW * 64;
    static constexpr int BQ = 64;                      // query rows per staged block
    static constexpr int KPW = 32;                     // keys per wave
    static constexpr int BKW = NW * KPW;               // keys per workgroup
    static constexpr int DC = D / 16;
    static constexpr int NDB = D / 32;
    using QTile = Blocks4x8<BQ, D, NT>;
    static constexpr int LDN = QTile::LDN, LDT = QTile::LDT;
    static constexpr int QN = BQ * LDN;                // elements of one natural tile
    static constexpr int QT = D * LDT;                 // elements of one transposed tile
    // stage layout (bf16 elements): Qn | dOn | Qt | dOt | L (BQ floats) | D (BQ floats)
    static constexpr int OFF_DON = QN, OFF_QT = 2 * QN, OFF_DOT = 2 * QN + QT;
    static constexpr int OFF_L = 2 * QN + 2 * QT;       // element offset of the float arrays
    static constexpr int STAGE = OFF_L + 4 * BQ;        // 2*BQ floats = 4*BQ bf16 slots
};

template <int D, int NW>
struct DkdvStage {
    using C = DkdvCfg<D, NW>;
    typename C::QTile q, go;
    float lv, dv;

    __device__ __forceinline__ void load(const uint16_t* Qh, const uint16_t* dOh,
                                         const float* Lh, const float* Dh, int64_t ldq, int i,
                                         int T) {
        const uint32_t ldb = (uint32_t)(ldq * 2);
        q.load(rows_buf(Qh, ldq, T), ldb, i * C::BQ);
        go.load(rows_buf(dOh, ldq, T), ldb, i * C::BQ);
        const int t = threadIdx.x;
        if (t < C::BQ) {
            const int row = i * C::BQ + t;
            lv = row < T ? Lh[row] * kLog2e : kBigLse;
            dv = row < T ? Dh[row] : 0.f;
        }
    }

    __device__ __forceinline__ void store(uint16_t* buf) const {
        q.store_natural(buf);
        go.store_natural(buf + C::OFF_DON);
        q.store_transposed(buf + C::OFF_QT);
        go.store_transposed(buf + C::OFF_DOT);
        const int t = threadIdx.x;
        if (t < C::BQ) {
            float* f = reinterpret_cast<float*>(buf + C::OFF_L);
            f[t] = lv;
            f[C::BQ + t] = dv;
        }
    }
};

}  // namespace

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ L, const float* __restrict__ Dv, float* __restrict__ dK,
    float* __restrict__ dV, int B, int T, int H, int HKV, float scale, int causal, int window) {
    using C = DkdvCfg<D, NW>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    // longest query ranges (first key blocks under causal) first; consecutive ids walk the
    // (b, kv head) groups, so a group's blocks keep landing on the same XCD
    const int BG = B * HKV;
    const int kt = (int)(blockIdx.x / BG);
    const int bg = blockIdx.x % BG;
    const int b = bg / HKV, hk = bg % HKV, rep = H / HKV;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int kw0 = kt * C::BKW + w * C::KPW;
    const int key = kw0 + n;
    const int64_t ldq = (int64_t)H * D, ldk = (int64_t)HKV * D;
    const bool cz = causal != 0;
    const float c = scale * kLog2e;
    // queries that see this lane's key: [qlo, qhi] (lanes of keys past T are never stored)
    const int qlo = cz ? key : 0;
    const int qhi = min(window > 0 ? key + window - 1 : T - 1, T - 1);

    // B operands of S = Q K^T and dP = dO V^T: lane (n, g) holds K/V[key][16*dc + 8g .. +7]
    bf16x8 kreg[C::DC], vreg[C::DC];
    {
        const uint16_t* Kk = K + ((int64_t)b * T + key) * ldk + (int64_t)hk * D + 8 * g;
        const uint16_t* Vk = V + ((int64_t)b * T + key) * ldk + (int64_t)hk * D + 8 * g;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            kreg[dc] = __builtin_bit_cast(bf16x8, key < T ? *reinterpret_cast<const u32x4*>(Kk + dc * 16) : z);
            vreg[dc] = __builtin_bit_cast(bf16x8, key < T ? *reinterpret_cast<const u32x4*>(Vk + dc * 16) : z);
        }
    }
    f32x16 dka[C::NDB], dva[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dka[i][r] = dva[i][r] = 0.f;

    int ilo, ihi;
    q_block_range(T, kt * C::BKW, kt * C::BKW + C::BKW, C::BQ, cz, window, ilo, ihi);
    const int nqb = ihi - ilo;
    const int niter = rep * nqb;

    const uint16_t* Qg = Q + (int64_t)b * T * ldq + (int64_t)hk * rep * D;
    const uint16_t* dOg = dO + (int64_t)b * T * ldq + (int64_t)hk * rep * D;
    const float* Lg = L + ((int64_t)b * H + (int64_t)hk * rep) * T;
    const float* Dg = Dv + ((int64_t)b * H + (int64_t)hk * rep) * T;

    DkdvStage<D, NW> st;
    if (niter > 0) {
        st.load(Qg, dOg, Lg, Dg, ldq, ilo, T);
        st.store(smem);
    }
    __syncthreads();

    for (int it = 0; it < niter; ++it) {
        const int i = ilo + it % nqb;
        const uint16_t* buf = smem + (it & 1) * C::STAGE;
        const bool more = it + 1 < niter;
        if (more) {
            const int h2 = (it + 1) / nqb, i2 = ilo + (it + 1) % nqb;
            st.load(Qg + h2 * D, dOg + h2 * D, Lg + (int64_t)h2 * T, Dg + (int64_t)h2 * T, ldq,
                    i2, T);
        }
        const uint16_t* Qn = buf;
        const uint16_t* dOn = buf + C::OFF_DON;
        const uint16_t* Qt = buf + C::OFF_QT;
        const uint16_t* dOt = buf + C::OFF_DOT;
        const float* Ls = reinterpret_cast<const float*>(buf + C::OFF_L);
        const float* Ds = Ls + C::BQ;

#pragma unroll 1
        for (int qs = 0; qs < C::BQ / 32; ++qs) {
            const int qr0 = i * C::BQ + qs * 32;
            const int cls = block_class(T, qr0, qr0 + 32, kw0, kw0 + 32, cz, window);
            if (cls == kSkip) continue;
            f32x16 sc, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = dp[r] = 0.f;
            // A operands of S and dP, four k-steps issued ahead of their MFMAs
#pragma unroll
            for (int d0 = 0; d0 < C::DC; d0 += 4) {
                bf16x8 aq[4], ao[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int off = (qs * 32 + n) * C::LDN + (d0 + u) * 16 + 8 * g;
                    aq[u] = *reinterpret_cast<const bf16x8*>(Qn + off);
                    ao[u] = *reinterpret_cast<const bf16x8*>(dOn + off);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    sc = mfma32x32x16(aq[u], kreg[d0 + u], sc);
                    dp = mfma32x32x16(ao[u], vreg[d0 + u], dp);
                }
            }
            // entry r of lane (n, g): query qr0 + 8*(r/4) + 4g + r%4, key kw0 + n
            bf16x8 pp[2], pd[2];
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(Ls + qs * 32 + 8 * t4 + 4 * g);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + qs * 32 + 8 * t4 + 4 * g);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = 4 * t4 + u;
                    sc[r] = fast_exp2(fmaf(sc[r], c, -l4[u]));
                    dp[r] = dp[r] - d4[u];
                }
            }
            if (cls == kPartial) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qi = qr0 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if ((unsigned)(qi - qlo) > (unsigned)(qhi - qlo)) sc[r] = 0.f;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                pp[r >> 3][r & 7] = (__bf16)sc[r];
                pd[r >> 3][r & 7] = (__bf16)(sc[r] * dp[r]);
            }
            // dV += P^T dO and dK += dS^T Q over the 32 rows, 16 per k-step
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                bf16x8 bo[C::NDB], bq[C::NDB];
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    const int off = (db * 32 + n) * C::LDT + qs * 32 + 16 * hf + 8 * g;
                    bo[db] = *reinterpret_cast<const bf16x8*>(dOt + off);
                    bq[db] = *reinterpret_cast<const bf16x8*>(Qt + off);
                }
#pragma unroll
                for (int db = 0; db < C::NDB; ++db) {
                    dva[db] = mfma32x32x16(pp[hf], bo[db], dva[db]);
                    dka[db] = mfma32x32x16(pd[hf], bq[db], dka[db]);
                }
            }
        }
        if (more) st.store(smem + ((it + 1) & 1) * C::STAGE);
        __syncthreads();
    }

    // entry r of lane (n, g) in block db: key kw0 + 8*(r/4) + 4g + r%4, column db*32 + n
    float* dKg = dK + (int64_t)b * T * ldk + (int64_t)hk * D;
    float* dVg = dV + (int64_t)b * T * ldk + (int64_t)hk * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kk = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (kk < T) {
#pragma unroll
            for (int db = 0; db < C::NDB; ++db) {
                dKg[(int64_t)kk * ldk + db * 32 + n] = dka[db][r] * scale;
                dVg[(int64_t)kk * ldk + db * 32 + n] = dva[db][r];
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
    static constexpr int BK = 64;     // keys per staged block
    static constexpr int DC = D / 16;
    static constexpr int NDB = D / 32;
    using KTile = Blocks4x8<BK, D, NT>;   // K: natural + transposed
    using VTile = RowChunks<BK, D, NT>;   // V: natural
    static constexpr int LDN = KTile::LDN, LDT = KTile::LDT;
    static constexpr int KN = BK * LDN, KT = D * LDT;
    static constexpr int OFF_VN = KN, OFF_KT = 2 * KN;
    static constexpr int STAGE = 2 * KN + KT;
};

template <int D, int NW>
struct DqStage {
    using C = DqCfg<D, NW>;
    typename C::KTile k;
    typename C::VTile v;
    __device__ __forceinline__ void load(const Buf& kb, const Buf& vb, uint32_t ldb, int j) {
        k.load(kb, ldb, j * C::BK);
        v.load(vb, ldb, j * C::BK);
    }
    __device__ __forceinline__ void store(uint16_t* buf) const {
        k.store_natural(buf);
        v.store(buf + C::OFF_VN);
        k.store_transposed(buf + C::OFF_KT);
    }
};

}  // namespace

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 1) void dq_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ L, const float* __restrict__ Dv, float* __restrict__ dQ, int B,
    int T, int H, int HKV, float scale, int causal, int window, int nqt, int xcd_group) {
    using C = DqCfg<D, NW>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    int qt, b, h;
    decode_q_work(blockIdx.x, nqt, B, H, HKV, xcd_group, qt, b, h);
    const int hk = h / (H / HKV);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 31, g = lane >> 5;
    const int wr0 = qt * C::BQ + w * 32;
    const int q = wr0 + n;
    const int64_t ldq = (int64_t)H * D, ldk = (int64_t)HKV * D;
    const uint32_t ldk_b = (uint32_t)(ldk * 2);
    const Buf kbuf = rows_buf(K + (int64_t)b * T * ldk + (int64_t)hk * D, ldk, T);
    const Buf vbuf = rows_buf(V + (int64_t)b * T * ldk + (int64_t)hk * D, ldk, T);
    const bool cz = causal != 0;
    const float c = scale * kLog2e;

    // B operands of S^T = K Q^T and dP^T = V dO^T: lane (n, g) holds Q/dO[q][16*dc + 8g ..]
    bf16x8 qreg[C::DC], oreg[C::DC];
    {
        const int64_t base = ((int64_t)b * T + q) * ldq + (int64_t)h * D + 8 * g;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qreg[dc] = __builtin_bit_cast(bf16x8, q < T ? *reinterpret_cast<const u32x4*>(Q + base + dc * 16) : z);
            oreg[dc] = __builtin_bit_cast(bf16x8, q < T ? *reinterpret_cast<const u32x4*>(dO + base + dc * 16) : z);
        }
    }
    const float l2 = q < T ? L[((int64_t)b * H + h) * T + q] * kLog2e : kBigLse;
    const float dq_i = q < T ? Dv[((int64_t)b * H + h) * T + q] : 0.f;
    // keys this query row may see: [klo, khi]
    const int klo = window > 0 ? q - window + 1 : 0;
    const int khi = cz ? q : T - 1;
    f32x16 dqa[C::NDB];
#pragma unroll
    for (int i = 0; i < C::NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[i][r] = 0.f;

    int jlo, jhi;
    kv_block_range(T, qt * C::BQ, qt * C::BQ + C::BQ, C::BK, cz, window, jlo, jhi);
    DqStage<D, NW> st;
    if (jlo < jhi) {
        st.load(kbuf, vbuf, ldk_b, jlo);
        st.store(smem);
    }
    __syncthreads();

    for (int j = jlo; j < jhi; ++j) {
        const uint16_t* buf = smem + ((j - jlo) & 1) * C::STAGE;
        const bool more = j + 1 < jhi;
        if (more) st.load(kbuf, vbuf, ldk_b, j + 1);
        const int cls = block_class(T, wr0, wr0 + 32, j * C::BK, j * C::BK + C::BK, cz, window);
        if (cls != kSkip) {
            const uint16_t* Kn = buf;
            const uint16_t* Vn = buf + C::OFF_VN;
            const uint16_t* Kt = buf + C::OFF_KT;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 sk, dk;
#pragma unroll
                for (int r = 0; r < 16; ++r) sk[r] = dk[r] = 0.f;
                // A operands of S^T and dP^T for this 32-key half, four k-steps ahead
#pragma unroll
                for (int d0 = 0; d0 < C::DC; d0 += 4) {
                    bf16x8 ak[4], av[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int off = (kb * 32 + n) * C::LDN + (d0 + u) * 16 + 8 * g;
                        ak[u] = *reinterpret_cast<const bf16x8*>(Kn + off);
                        av[u] = *reinterpret_cast<const bf16x8*>(Vn + off);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        sk = mfma32x32x16(ak[u], qreg[d0 + u], sk);
                        dk = mfma32x32x16(av[u], oreg[d0 + u], dk);
                    }
                }
                // entry r of lane (n, g): key j*64 + 32kb + 8*(r/4) + 4g + r%4, query q
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sk[r] = fast_exp2(fmaf(sk[r], c, -l2));
                    dk[r] = dk[r] - dq_i;
                }
                if (cls == kPartial) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = j * C::BK + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
                        if ((unsigned)(kk - klo) > (unsigned)(khi - klo)) sk[r] = 0.f;
                    }
                }
                bf16x8 pd[2];
#pragma unroll
                for (int r = 0; r < 16; ++r) pd[r >> 3][r & 7] = (__bf16)(sk[r] * dk[r]);
                // dQ^T += K^T dS^T over this half's 32 keys, 16 per k-step
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    bf16x8 at[C::NDB];
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db)
                        at[db] = *reinterpret_cast<const bf16x8*>(
                            Kt + (db * 32 + n) * C::LDT + kb * 32 + hf * 16 + 8 * g);
#pragma unroll
                    for (int db = 0; db < C::NDB; ++db) dqa[db] = mfma32x32x16(at[db], pd[hf], dqa[db]);
                }
            }
        }
        if (more) st.store(smem + ((j + 1 - jlo) & 1) * C::STAGE);
        __syncthreads();
    }

    if (q >= T) return;
    float* dQq = dQ + ((int64_t)b * T + q) * ldq + (int64_t)h * D;
    // entry r of block db: dQ^T[db*32 + 8*(r/4) + 4g + r%4][query n]
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            f32x4 o;
#pragma unroll
            for (int u = 0; u < 4; ++u) o[u] = dqa[db][4 * t4 + u] * scale;
            *reinterpret_cast<f32x4*>(dQq + db * 32 + 8 * t4 + 4 * g) = o;
        }
}

// ------------------------------------------------------------------------------ launchers
namespace {

template <typename Kern>
hipError_t allow_lds(Kern kern, size_t lds, bool* set_flags) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!set_flags[dev]) {
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)lds);
        if (e != hipSuccess) return e;
        set_flags[dev] = true;
    }
    return hipSuccess;
}

constexpr int kDkdvWaves = 4;

template <int D>
hipError_t launch_dkdv_bf16_t(const AttnArgs& a) {
    using C = DkdvCfg<D, kDkdvWaves>;
    static bool set[kMaxDevices] = {};
    const size_t lds = 2 * C::STAGE * sizeof(uint16_t);
    hipError_t e = allow_lds(dkdv_bf16_kernel<D, kDkdvWaves>, lds, set);
    if (e != hipSuccess) return e;
    const int nkt = (a.T + C::BKW - 1) / C::BKW;
    const unsigned grid = (unsigned)nkt * a.B * a.HKV;
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, kDkdvWaves>), dim3(grid), dim3(C::NT), lds, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, a.Lin, a.Dvec, a.dK, a.dV, a.B, a.T, a.H, a.HKV,
                       a.scale, a.causal, a.window);
    return hipGetLastError();
}

constexpr int kDqWaves = 8;

template <int D>
hipError_t launch_dq_bf16_t(const AttnArgs& a) {
    using C = DqCfg<D, kDqWaves>;
    static bool set[kMaxDevices] = {};
    const size_t lds = 2 * C::STAGE * sizeof(uint16_t);
    hipError_t e = allow_lds(dq_bf16_kernel<D, kDqWaves>, lds, set);
    if (e != hipSuccess) return e;
    const int nqt = (a.T + C::BQ - 1) / C::BQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    hipLaunchKernelGGL((dq_bf16_kernel<D, kDqWaves>), dim3(grid), dim3(C::NT), lds, a.stream,
                       (const uint16_t*)a.Q, (const uint16_t*)a.K, (const uint16_t*)a.V,
                       (const uint16_t*)a.dO, a.Lin, a.Dvec, a.dQ, a.B, a.T, a.H, a.HKV, a.scale,
                       a.causal, a.window, nqt, xcd_group_for(nqt, a.B, a.H, a.HKV));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dkdv_bf16(const AttnArgs& a) {
    if (a.D == 64) return launch_dkdv_bf16_t<64>(a);
    if (a.D == 128) return launch_dkdv_bf16_t<128>(a);
    return hipErrorInvalidValue;
}

hipError_t launch_dq_bf16(const AttnArgs& a) {
    if (a.D == 64) return launch_dq_bf16_t<64>(a);
    if (a.D == 128) return launch_dq_bf16_t<128>(a);
    return hipErrorInvalidValue;
}

}  // namespace fa
