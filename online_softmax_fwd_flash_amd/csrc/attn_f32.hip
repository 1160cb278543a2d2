// fp32 attention kernels for gfx950: forward, dK/dV and dQ, on the 16x16x4 fp32 MFMA
// (true fp32 products, fp32 accumulation).  Head dim D is a runtime multiple of 8 up to 128,
// padded to DP in {8, 16, 32, 64, 128} for the contractions over the head dim (S = Q K^T,
// dP = dO V^T); the products whose output has head-dim columns (O, dQ, dK, dV) come in
// 16-column MFMA blocks, so their operand tiles are staged at least 16 columns wide (zeros
// past D).  A workgroup's tiling (BQ query rows x BK keys per block) is a template parameter
// so the tilings the pages use (32 x 32, 64 x 16) run as such.
//
// Orientation.  Scores are formed transposed, S^T = K Q^T, so MFMA column n (lane l % 16) is a
// query row: a query's running max / sum live in its own lanes and only the four 16-lane
// groups of a wave exchange values.  P^T then feeds O^T += V^T P^T directly from the
// accumulator layout, and O^T keeps each query in its own lanes for the rescale.
//
// Method: the forge page "flash_attention.metal" (forward kernel: K/V staged through on-chip
// memory per block, online softmax with m from -FLT_MAX, causal key bound, window block skip,
// diagonal-only mask, l == 0 guard; backward kernels dQ / dV / dK) and the Graphcore page
// "flash_attention_qkv_packed.cpp" (block skip / mask conditions, log-sum-exp stash,
// key-chunk-outer backward).
#include "common.h"
#include "kernels.h"

// At least two waves per SIMD.  That caps a wave at 256 registers, so the compiler keeps MFMA
// results in ordinary VGPRs; with room for more it allocates them in AGPRs and copies every
// score to VGPRs for the softmax arithmetic, extra vector instructions that cost time here
// because the fp32 MFMA does not overlap with vector instructions (7-13% per kernel at D = 8
// and 64).
#define kTwoWavesPerSimd __attribute__((amdgpu_waves_per_eu(2)))

namespace fa {

namespace {

template <int DP>
struct F32Tile {
    static constexpr int KS = DP / 4;                // MFMA k-steps over the (padded) head dim
    static constexpr int DW = DP < 16 ? 16 : DP;     // staged columns (16-column output blocks)
    static constexpr int LD = DW + 4;                // padded LDS row (floats): conflict-free
    static constexpr int NDB = DW / 16;              // 16-wide blocks of O / dQ / dK / dV
};

// Keys staged per barrier pair in the query-owned passes (forward, dQ): several key blocks of
// BK when BK is small (each block keeps its own class test and online-softmax update, in the
// same order, so results do not change), as long as the K and V tiles fit static LDS.
template <int DP, int BK>
struct F32KeyStage {
    static constexpr int SB = (BK < 64 && DP <= 64) ? 64 : BK;
    static constexpr int NSB = SB / BK;   // key blocks per stage
};

// Stage rows [row0, row0 + ROWS) of a [*, ld] matrix (head slice at `base`) into LDS
// (ROWS x DW, zero outside [0, T) x [0, D)).  With ONES (DP < DW, so D = DP and column DP is
// padding) column DP holds 1 in every row instead.
template <int DP, int ROWS, int NT, bool ONES = false>
__device__ __forceinline__ void stage_rows(float* __restrict__ dst, const float* __restrict__ base,
                                           int64_t ld, int row0, int T, int D) {
    constexpr int C4 = F32Tile<DP>::DW / 4;
    static_assert(!ONES || (DP < F32Tile<DP>::DW && DP % 4 == 0), "no padding column");
    for (int e = threadIdx.x; e < ROWS * C4; e += NT) {
        const int r = e / C4, d = (e % C4) * 4;
        const int row = row0 + r;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (row < T && d < D) {
            // D is a multiple of 8, so a float4 never straddles D
            x = *reinterpret_cast<const f32x4*>(base + (int64_t)row * ld + d);
        }
        if (ONES && d == DP) x[0] = 1.f;
        *reinterpret_cast<f32x4*>(dst + r * F32Tile<DP>::LD + d) = x;
    }
}

// max(v[l], v[l ^ 16]) for every lane l, in VALU (v_permlane16_swap_b32 exchanges the odd
// 16-lane rows of one copy of v with the even rows of another: the two results hold v[l] and
// v[l ^ 16] in some order, and max does not care which)
__device__ __forceinline__ float rows16_max(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// The same ROWS x DP tile through registers: load() issues the global loads of the next block
// while the current one is computed, store() writes them to LDS after the next barrier.  Used
// by the dQ pass, where it measured 6.5% faster at 64 x 16 tiles, D = 64; the forward and
// dK/dV passes measured 1-2% slower with it (more registers, no latency left to hide).
template <int DP, int ROWS, int NT>
struct RowPrefetch {
    static constexpr int C4 = F32Tile<DP>::DW / 4;
    static constexpr int PER = (ROWS * C4 + NT - 1) / NT;   // float4 per thread
    f32x4 v[PER];
    __device__ __forceinline__ void load(const float* __restrict__ base, int64_t ld, int row0,
                                         int T, int D) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * NT;
            const int r = e / C4, d = (e % C4) * 4;
            const int row = row0 + r;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (e < ROWS * C4 && row < T && d < D) x = *reinterpret_cast<const f32x4*>(base + (int64_t)row * ld + d);
            v[i] = x;
        }
    }
    __device__ __forceinline__ void store(float* __restrict__ dst) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * NT;
            if (e < ROWS * C4)
                *reinterpret_cast<f32x4*>(dst + (e / C4) * F32Tile<DP>::LD + (e % C4) * 4) = v[i];
        }
    }
};


}  // namespace

// ------------------------------------------------------------------------------ forward
template <int DP, int BQ, int BK>
__global__ __launch_bounds__(BQ / 16 * 64) kTwoWavesPerSimd void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ L, int B, int T, int Tk, int H, int HKV, int D,
    float scale, int causal, int window, int nqt, Layout lq, Layout lk) {
    using Tl = F32Tile<DP>;
    constexpr int NW = BQ / 16, NT = NW * 64, KS = Tl::KS, LD = Tl::LD, NDB = Tl::NDB;
    constexpr int SB = F32KeyStage<DP, BK>::SB, NSB = F32KeyStage<DP, BK>::NSB;
    // When the V tile has a padding column (DP < DW, i.e. D = 8), that column holds ones, so
    // the PV products also leave each query's sum of P in O^T row DP: no per-score adds, and
    // the rescale of O covers the sum.
    constexpr bool kSumInPV = DP < Tl::DW;
    __shared__ __attribute__((aligned(16))) float Ks[SB * LD];
    __shared__ __attribute__((aligned(16))) float Vs[SB * LD];

    const int BH = B * H;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // longest key ranges first
    const int bh = blockIdx.x % BH;
    const int b = bh / H, h = bh % H, hk = h / (H / HKV);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int n = lane & 15, g = lane >> 4;
    const int wr0 = qt * BQ + w * 16;
    const int q = wr0 + n;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)
    const float* Qh = Q + b * lq.b + h * lq.h;
    const float* Kh = K + b * lk.b + hk * lk.h;
    const float* Vh = V + b * lk.b + hk * lk.h;

    // Q * scale * log2(e) (fp32: one rounding of 2^-24 relative), so S^T comes out of the
    // MFMAs in exp2 units
    const float c = scale * kLog2e;
    float qreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d = g * KS + s;
        qreg[s] = (q < T && d < D) ? Qh[(int64_t)q * ldq + d] * c : 0.f;
    }
    f32x4 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Running reference mc (exp2 units), lazily moved: the S^T MFMAs start from -mc, so their
    // results are the exp2 arguments themselves; O and the sum are rescaled only when a row's
    // block max passes mc + 8 (thr = 8 once the row has seen a key, -inf before, so the first
    // visible key always does), so every exp2 argument stays below 8.
    float mc = 0.f, thr = -INFINITY, lsum = 0.f;
    f32x4 negmc = {0.f, 0.f, 0.f, 0.f};
    const bool cz = causal != 0;

    int jlo, jhi;
    kv_block_range(T, Tk, qt * BQ, qt * BQ + BQ, BK, cz, window, jlo, jhi);
    // key blocks FULL for this wave's rows: the class test runs only outside them
    int jf0, jf1;
    full_kv_block_range(T, Tk, wr0, wr0 + 16, BK, cz, window, jf0, jf1);
    for (int j0 = jlo; j0 < jhi; j0 += NSB) {
        __syncthreads();
        stage_rows<DP, SB, NT>(Ks, Kh, ldk, j0 * BK, Tk, D);
        stage_rows<DP, SB, NT, kSumInPV>(Vs, Vh, ldk, j0 * BK, Tk, D);
        __syncthreads();
        // S^T of the staged key blocks (each block skipped or masked by its own class); one
        // online-softmax update for all of them
        int cls[NSB];
        f32x4 s[NSB][BK / 16];
#pragma unroll
        for (int jj = 0; jj < NSB; ++jj) {
            const int j = j0 + jj;
            cls[jj] = kFull;
            if (j >= jhi) {
                cls[jj] = kSkip;
            } else if (j < jf0 || j >= jf1) {
                keep_branch();
                cls[jj] = block_class(T, Tk, wr0, wr0 + 16, j * BK, j * BK + BK, cz, window);
            }
#pragma unroll
            for (int kb = 0; kb < BK / 16; ++kb) s[jj][kb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (cls[jj] == kSkip) continue;
#pragma unroll
            for (int kb = 0; kb < BK / 16; ++kb) {
                f32x4 a = negmc;
                const float* krow = Ks + (jj * BK + kb * 16 + n) * LD + g * KS;
#pragma unroll
                for (int st = 0; st < KS; ++st) a = mfma16x16x4f32(krow[st], qreg[st], a);
                s[jj][kb] = a;
            }
            if (cls[jj] == kPartial) {
#pragma unroll
                for (int kb = 0; kb < BK / 16; ++kb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = j * BK + kb * 16 + 4 * g + r;
                        if (!visible(q, key, T, Tk, cz, window)) s[jj][kb][r] = -INFINITY;
                    }
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < NSB; ++jj)
#pragma unroll
            for (int kb = 0; kb < BK / 16; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[jj][kb][r]);
        mx = halves_max(rows16_max(mx));
        if (__any(mx > thr)) {
            // d: how far the row's reference moves up (a row that has seen no key yet jumps
            // to this stage's max; its O and sum are still zero)
            const bool seen = thr > 0.f;
            const bool now = seen || mx > -INFINITY;
            const float d = seen ? fmaxf(mx, 0.f) : (now ? mx : 0.f);
            const float corr = seen ? fast_exp2(-d) : 0.f;
            mc += d;
            thr = now ? 8.f : -INFINITY;
            negmc = f32x4{-mc, -mc, -mc, -mc};
            if constexpr (!kSumInPV) lsum *= corr;
#pragma unroll
            for (int i = 0; i < NDB; ++i) oacc[i] *= corr;
#pragma unroll
            for (int jj = 0; jj < NSB; ++jj)
#pragma unroll
                for (int kb = 0; kb < BK / 16; ++kb) s[jj][kb] -= d;
        }
#pragma unroll
        for (int jj = 0; jj < NSB; ++jj) {
            if (cls[jj] == kSkip) continue;
#pragma unroll
            for (int kb = 0; kb < BK / 16; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(s[jj][kb][r]);
                    if constexpr (!kSumInPV) lsum += p;
                    const float* vrow = Vs + (jj * BK + kb * 16 + 4 * g + r) * LD + n;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        oacc[db] = mfma16x16x4f32(vrow[db * 16], p, oacc[db]);
                }
        }
    }

    if constexpr (kSumInPV) {
        // O^T row DP of query n: element DP % 4 of block DP / 16 in lane (n, (DP % 16) / 4)
        lsum = __shfl(oacc[DP / 16][DP % 4], 16 * ((DP % 16) / 4) + n, 64);
    } else {
        lsum += xor_shfl(lsum, 16);
        lsum += xor_shfl(lsum, 32);
    }
    if (q >= T) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* Oq = O + b * lq.b + (int64_t)q * ldq + h * lq.h;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + 4 * g;
        if (d < D) *reinterpret_cast<f32x4*>(Oq + d) = oacc[db] * inv;
    }
    if (g == 0)
        L[((int64_t)b * H + h) * T + q] = lsum > 0.f ? (mc + fast_log2(lsum)) * kLn2 : 0.f;
}

// ------------------------------------------------------------------------------ dK / dV
// Keys per workgroup: BK, or several key blocks of BK when BK < 64, so that a workgroup has
// four waves (a one-wave workgroup per 16-key block left one wave per SIMD, the Q / dO stage
// filling the LDS).  Each wave's 16 keys lie inside one BK block, and every query x key
// class test is per wave, so the BK blocking itself is unchanged.
template <int BK>
struct DkdvF32Keys {
    static constexpr int KW = BK < 64 ? 64 : BK;
};

// One workgroup per (b, kv head, KW keys); wave w owns keys [w*16, w*16+16) of them and loops
// over the query heads of the group and the query blocks that see them.
template <int DP, int BQ, int BK>
__global__ __launch_bounds__(DkdvF32Keys<BK>::KW / 16 * 64) kTwoWavesPerSimd void dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    float* __restrict__ dK, float* __restrict__ dV, int B, int T, int Tk, int H, int HKV, int D,
    float scale, int causal, int window, int nkt, Layout lq, Layout lk) {
    using Tl = F32Tile<DP>;
    constexpr int KW = DkdvF32Keys<BK>::KW;
    constexpr int NW = KW / 16, NT = NW * 64, KS = Tl::KS, LD = Tl::LD, NDB = Tl::NDB;
    __shared__ __attribute__((aligned(16))) float Qs[BQ * LD];
    __shared__ __attribute__((aligned(16))) float dOs[BQ * LD];
    __shared__ __attribute__((aligned(16))) float Ls[BQ];
    __shared__ __attribute__((aligned(16))) float Ds[BQ];

    const int BG = B * HKV;
    const int kt = (int)(blockIdx.x / BG);
    const int bg = blockIdx.x % BG;
    const int b = bg / HKV, hk = bg % HKV, rep = H / HKV;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int n = lane & 15, g = lane >> 4;
    const int kw0 = kt * KW + w * 16;
    const int key = kw0 + n;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)
    const float* Kh = K + b * lk.b + hk * lk.h;
    const float* Vh = V + b * lk.b + hk * lk.h;
    const bool cz = causal != 0;
    const float c = scale * kLog2e;

    // K * scale * log2(e) (fp32), so S comes out of the MFMAs in exp2 units; the S and dP
    // MFMAs start from -L*log2(e) and -Dvec of each query row, leaving P's exp2 argument and
    // dP - Dvec
    float kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d = g * KS + s;
        const bool ok = key < Tk && d < D;
        kreg[s] = ok ? Kh[(int64_t)key * ldk + d] * c : 0.f;
        vreg[s] = ok ? Vh[(int64_t)key * ldk + d] : 0.f;
    }
    f32x4 dka[NDB], dva[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dka[i] = dva[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    int ilo, ihi;
    q_block_range(T, Tk, kt * KW, kt * KW + KW, BQ, cz, window, ilo, ihi);
    // 16-row query blocks FULL for this wave's keys: the class test runs only outside them
    int if0, if1;
    full_q_block_range(T, Tk, kw0, kw0 + 16, 16, cz, window, if0, if1);
    for (int hh = 0; hh < rep; ++hh) {
        const int h = hk * rep + hh;
        const float* Qh = Q + b * lq.b + h * lq.h;
        const float* dOh = dO + b * lq.b + h * lq.h;
        const float* Lh = L + ((int64_t)b * H + h) * T;
        const float* Dh = Dv + ((int64_t)b * H + h) * T;
        for (int i = ilo; i < ihi; ++i) {
            __syncthreads();
            stage_rows<DP, BQ, NT>(Qs, Qh, ldq, i * BQ, T, D);
            stage_rows<DP, BQ, NT>(dOs, dOh, ldq, i * BQ, T, D);
            for (int e = threadIdx.x; e < BQ; e += NT) {
                const int row = i * BQ + e;
                Ls[e] = row < T ? -Lh[row] * kLog2e : 0.f;
                Ds[e] = row < T ? -Dh[row] : 0.f;
            }
            __syncthreads();
#pragma unroll 1
            for (int qs = 0; qs < BQ; qs += 16) {
                const int qr0 = i * BQ + qs;
                int cls = kFull;
                if (qr0 < if0 * 16 || qr0 >= if1 * 16) {
                    keep_branch();
                    cls = block_class(T, Tk, qr0, qr0 + 16, kw0, kw0 + 16, cz, window);
                }
                if (cls == kSkip) continue;
                // lane (n, g), element r: query qr0 + 4g + r, key kw0 + n
                f32x4 sc = *reinterpret_cast<const f32x4*>(Ls + qs + 4 * g);
                f32x4 dp = *reinterpret_cast<const f32x4*>(Ds + qs + 4 * g);
                const float* qrow = Qs + (qs + n) * LD + g * KS;
                const float* orow = dOs + (qs + n) * LD + g * KS;
#pragma unroll
                for (int st = 0; st < KS; ++st) {
                    sc = mfma16x16x4f32(qrow[st], kreg[st], sc);
                    dp = mfma16x16x4f32(orow[st], vreg[st], dp);
                }
                f32x4 p, ds;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float pr = fast_exp2(sc[r]);
                    if (cls == kPartial && !visible(qr0 + 4 * g + r, key, T, Tk, cz, window)) pr = 0.f;
                    p[r] = pr;
                    ds[r] = pr * dp[r];
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float* dorow = dOs + (qs + 4 * g + r) * LD + n;
                    const float* qcol = Qs + (qs + 4 * g + r) * LD + n;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        dva[db] = mfma16x16x4f32(p[r], dorow[db * 16], dva[db]);
                        dka[db] = mfma16x16x4f32(ds[r], qcol[db * 16], dka[db]);
                    }
                }
            }
        }
    }
    // lane (n, g), element r: key kw0 + 4g + r, column d = db*16 + n
    float* dKh = dK + b * lk.b + hk * lk.h;
    float* dVh = dV + b * lk.b + hk * lk.h;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kk = kw0 + 4 * g + r;
            if (kk < Tk && d < D) {
                dKh[(int64_t)kk * ldk + d] = dka[db][r] * scale;
                dVh[(int64_t)kk * ldk + d] = dva[db][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------ dQ
template <int DP, int BQ, int BK>
__global__ __launch_bounds__(BQ / 16 * 64) kTwoWavesPerSimd void dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ L, const float* __restrict__ Dv,
    float* __restrict__ dQ, int B, int T, int Tk, int H, int HKV, int D, float scale, int causal,
    int window, int nqt, Layout lq, Layout lk) {
    using Tl = F32Tile<DP>;
    constexpr int NW = BQ / 16, NT = NW * 64, KS = Tl::KS, LD = Tl::LD, NDB = Tl::NDB;
    constexpr int SB = F32KeyStage<DP, BK>::SB, NSB = F32KeyStage<DP, BK>::NSB;
    __shared__ __attribute__((aligned(16))) float Ks[SB * LD];
    __shared__ __attribute__((aligned(16))) float Vs[SB * LD];

    const int BH = B * H;
    const int qt = nqt - 1 - (int)(blockIdx.x / BH);
    const int bh = blockIdx.x % BH;
    const int b = bh / H, h = bh % H, hk = h / (H / HKV);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int n = lane & 15, g = lane >> 4;
    const int wr0 = qt * BQ + w * 16;
    const int q = wr0 + n;
    const int64_t ldq = lq.t, ldk = lk.t;   // row strides (elements)
    const float* Qh = Q + b * lq.b + h * lq.h;
    const float* dOh = dO + b * lq.b + h * lq.h;
    const float* Kh = K + b * lk.b + hk * lk.h;
    const float* Vh = V + b * lk.b + hk * lk.h;
    const bool cz = causal != 0;
    const float c = scale * kLog2e;

    // Q * scale * log2(e) (fp32), so S^T comes out of the MFMAs in exp2 units; the S^T and
    // dP^T MFMAs start from this lane's -L*log2(e) and -Dvec, leaving P's exp2 argument and
    // dP - Dvec
    float qreg[KS], doreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int d = g * KS + s;
        const bool ok = q < T && d < D;
        qreg[s] = ok ? Qh[(int64_t)q * ldq + d] * c : 0.f;
        doreg[s] = ok ? dOh[(int64_t)q * ldq + d] : 0.f;
    }
    const float l2 = q < T ? L[((int64_t)b * H + h) * T + q] * kLog2e : 0.f;
    const float dq_i = q < T ? Dv[((int64_t)b * H + h) * T + q] : 0.f;
    const f32x4 negl = {-l2, -l2, -l2, -l2}, negd = {-dq_i, -dq_i, -dq_i, -dq_i};
    f32x4 dqa[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqa[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    int jlo, jhi;
    kv_block_range(T, Tk, qt * BQ, qt * BQ + BQ, BK, cz, window, jlo, jhi);
    // 16-key blocks FULL for this wave's rows: the class test runs only outside them
    int kf0, kf1;
    full_kv_block_range(T, Tk, wr0, wr0 + 16, 16, cz, window, kf0, kf1);
    RowPrefetch<DP, SB, NT> pk, pv;
    if (jlo < jhi) {
        pk.load(Kh, ldk, jlo * BK, Tk, D);
        pv.load(Vh, ldk, jlo * BK, Tk, D);
    }
    for (int j0 = jlo; j0 < jhi; j0 += NSB) {
        __syncthreads();
        pk.store(Ks);
        pv.store(Vs);
        __syncthreads();
        if (j0 + NSB < jhi) {   // next stage's loads in flight while this one is computed
            pk.load(Kh, ldk, (j0 + NSB) * BK, Tk, D);
            pv.load(Vh, ldk, (j0 + NSB) * BK, Tk, D);
        }
        // the 16-key blocks of the staged key blocks j0 .. (up to jhi)
        const int nkb = ((jhi - j0 < NSB ? jhi - j0 : NSB) * BK) / 16;
#pragma unroll 1
        for (int kb = 0; kb < nkb; ++kb) {
            const int kc0 = j0 * BK + kb * 16;
            int cls = kFull;
            if (kc0 < kf0 * 16 || kc0 >= kf1 * 16) {
                keep_branch();
                cls = block_class(T, Tk, wr0, wr0 + 16, kc0, kc0 + 16, cz, window);
            }
            if (cls == kSkip) continue;
            f32x4 sc = negl, dp = negd;
            const float* krow = Ks + (kb * 16 + n) * LD + g * KS;
            const float* vrow = Vs + (kb * 16 + n) * LD + g * KS;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                sc = mfma16x16x4f32(krow[st], qreg[st], sc);
                dp = mfma16x16x4f32(vrow[st], doreg[st], dp);
            }
            // lane (n, g), element r: key kc0 + 4g + r, query q
            f32x4 ds;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pr = fast_exp2(sc[r]);
                if (cls == kPartial && !visible(q, kc0 + 4 * g + r, T, Tk, cz, window)) pr = 0.f;
                ds[r] = pr * dp[r];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float* kcol = Ks + (kb * 16 + 4 * g + r) * LD + n;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    dqa[db] = mfma16x16x4f32(kcol[db * 16], ds[r], dqa[db]);
            }
        }
    }
    if (q >= T) return;
    float* dQq = dQ + b * lq.b + (int64_t)q * ldq + h * lq.h;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + 4 * g;
        if (d < D) *reinterpret_cast<f32x4*>(dQq + d) = dqa[db] * scale;
    }
}

// ------------------------------------------------------------------------------ launchers
namespace {

template <int DP, int BQ, int BK>
hipError_t launch_fwd_f32_t(const AttnArgs& a) {
    const int nqt = (a.T + BQ - 1) / BQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    if (log_enabled()) {
        char nm[64];
        snprintf(nm, sizeof nm, "fwd_f32_kernel<DP=%d,BQ=%d,BK=%d>", DP, BQ, BK);
        log_launch(nm, "f32", a.D, grid, BQ / 16 * 64, 0, a.B, a.T, a.Tk, a.H, a.HKV, a.causal,
                   a.window);
    }
    hipLaunchKernelGGL((fwd_f32_kernel<DP, BQ, BK>), dim3(grid), dim3(BQ / 16 * 64), 0,
                       a.stream, (const float*)a.Q, (const float*)a.K, (const float*)a.V,
                       (float*)a.Oout, a.L, a.B, a.T, a.Tk, a.H, a.HKV, a.D, a.scale, a.causal,
                       a.window, nqt, a.lq, a.lk);
    return hipGetLastError();
}

template <int DP, int BQ, int BK>
hipError_t launch_dkdv_f32_t(const AttnArgs& a) {
    constexpr int KW = DkdvF32Keys<BK>::KW;
    const int nkt = (a.Tk + KW - 1) / KW;
    const unsigned grid = (unsigned)nkt * a.B * a.HKV;
    if (log_enabled()) {
        char nm[64];
        snprintf(nm, sizeof nm, "dkdv_f32_kernel<DP=%d,BQ=%d,BK=%d>", DP, BQ, BK);
        log_launch(nm, "f32", a.D, grid, KW / 16 * 64, 0, a.B, a.T, a.Tk, a.H, a.HKV, a.causal,
                   a.window);
    }
    hipLaunchKernelGGL((dkdv_f32_kernel<DP, BQ, BK>), dim3(grid), dim3(KW / 16 * 64), 0,
                       a.stream, (const float*)a.Q, (const float*)a.K, (const float*)a.V,
                       (const float*)a.dO, a.Lin, a.Dvec, a.dK, a.dV, a.B, a.T, a.Tk, a.H, a.HKV, a.D,
                       a.scale, a.causal, a.window, nkt, a.lq, a.lk);
    return hipGetLastError();
}

template <int DP, int BQ, int BK>
hipError_t launch_dq_f32_t(const AttnArgs& a) {
    const int nqt = (a.T + BQ - 1) / BQ;
    const unsigned grid = (unsigned)nqt * a.B * a.H;
    if (log_enabled()) {
        char nm[64];
        snprintf(nm, sizeof nm, "dq_f32_kernel<DP=%d,BQ=%d,BK=%d>", DP, BQ, BK);
        log_launch(nm, "f32", a.D, grid, BQ / 16 * 64, 0, a.B, a.T, a.Tk, a.H, a.HKV, a.causal,
                   a.window);
    }
    hipLaunchKernelGGL((dq_f32_kernel<DP, BQ, BK>), dim3(grid), dim3(BQ / 16 * 64), 0,
                       a.stream, (const float*)a.Q, (const float*)a.K, (const float*)a.V,
                       (const float*)a.dO, a.Lin, a.Dvec, a.dQ, a.B, a.T, a.Tk, a.H, a.HKV, a.D,
                       a.scale, a.causal, a.window, nqt, a.lq, a.lk);
    return hipGetLastError();
}

template <template <int, int, int> class Fn, int DP>
hipError_t by_tiles(const AttnArgs& a, int bq, int bk) {
    if (bq == 32 && bk == 32) return Fn<DP, 32, 32>::run(a);
    if (bq == 64 && bk == 16) return Fn<DP, 64, 16>::run(a);
    if (bq == 64 && bk == 64) return Fn<DP, 64, 64>::run(a);
    if (bq == 64 && bk == 32) return Fn<DP, 64, 32>::run(a);
    if (bq == 32 && bk == 16) return Fn<DP, 32, 16>::run(a);
    if (bq == 32 && bk == 64) return Fn<DP, 32, 64>::run(a);
    return hipErrorInvalidValue;
}

template <template <int, int, int> class Fn>
hipError_t by_dim(const AttnArgs& a, int bq, int bk) {
    if (a.D <= 8) return by_tiles<Fn, 8>(a, bq, bk);
    if (a.D <= 16) return by_tiles<Fn, 16>(a, bq, bk);
    if (a.D <= 32) return by_tiles<Fn, 32>(a, bq, bk);
    if (a.D <= 64) return by_tiles<Fn, 64>(a, bq, bk);
    return by_tiles<Fn, 128>(a, bq, bk);
}

template <int DP, int BQ, int BK> struct FwdF32 {
    static hipError_t run(const AttnArgs& a) { return launch_fwd_f32_t<DP, BQ, BK>(a); }
};
template <int DP, int BQ, int BK> struct DkdvF32 {
    static hipError_t run(const AttnArgs& a) { return launch_dkdv_f32_t<DP, BQ, BK>(a); }
};
template <int DP, int BQ, int BK> struct DqF32 {
    static hipError_t run(const AttnArgs& a) { return launch_dq_f32_t<DP, BQ, BK>(a); }
};

}  // namespace

bool f32_tiles_supported(int bq, int bk) {
    return (bq == 32 || bq == 64) && (bk == 16 || bk == 32 || bk == 64);
}

hipError_t launch_fwd_f32(const AttnArgs& a, int bq, int bk) { return by_dim<FwdF32>(a, bq, bk); }
hipError_t launch_dkdv_f32(const AttnArgs& a, int bq, int bk) {
    return by_dim<DkdvF32>(a, bq, bk);
}
hipError_t launch_dq_f32(const AttnArgs& a, int bq, int bk) { return by_dim<DqF32>(a, bq, bk); }

}  // namespace fa
