/*
 * flash_attn.h — C ABI of a fused, exact scaled-dot-product attention library for AMD MI355X
 * (gfx950), in the FlashAttention-2 style: forward with an online softmax that never writes
 * the T x T score matrix and stores one log-sum-exp per query row; backward that recomputes
 * the probabilities tile by tile from that log-sum-exp.
 *
 * Sources (web pages, cited by title and section):
 *   [forge]     "flash_attention.metal" (forge, S.-P. Boucher): header comment (what is stored,
 *               the online-softmax update, m starting at -FLT_MAX), FlashParams, the forward
 *               kernel flash_attn_fwd and the backward kernels flash_attn_bwd_dq / _dv / _dk.
 *   [ipu]       "flash_attention_qkv_packed.cpp" (Graphcore flash-attention-ipu):
 *               flashAttentionQKVPackedWithStash (forward with stored log-sum-exp),
 *               flashAttentionQKVPackedGrad (backward), getTriuOffsetSequence (causal masks
 *               of non-square blocks).
 *   [teeny]     "flash_attn2.rs" (teeny-kernels 0.2.0): forward, backward_dq, backward_dkv
 *               doc comments; the module comment on the tensor layout.
 *   [metal5]    "flashback.metal" (FlashMetal): backprop_attention, its batch and head
 *               offset arithmetic.
 *   [rope]      "qkv_rope.py" (modded-nanogpt): the fused QK-norm + rotary forward.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layouts (row-major, contiguous, as in [forge] forward kernel's address arithmetic):
 *    Q, O, dO, dQ : [B, T, H,   D]      K, V, dK, dV : [B, T, HKV, D]
 *    L, Dvec      : [B, H, T]  float32
 *  GQA: query head h reads KV head h / (H / HKV) ([forge] forward kernel); H % HKV == 0.
 *  scale multiplies q.k ([forge] flash_attn_fwd, [teeny] forward); must be finite and > 0.
 *  causal != 0 keeps keys j <= i (diagonal kept).  window > 0 keeps keys j >= i - window + 1
 *  (window counts keys including self; 0 = off; without causal it is a lower bound only),
 *  as in [forge] FlashParams and the per-row bounds of its kernels.  A window of T keys or
 *  more keeps every key, exactly as no window.
 *  L = m + ln(l) in natural-log units ([ipu] forward epilogue, [forge] forward epilogue);
 *  a row with no visible key gets O = 0 and L = 0 ([forge] forward epilogue guard).
 *  dtype selects the element type of Q, K, V, O and dO: FA_DTYPE_F32 (float),
 *  FA_DTYPE_BF16 (bfloat16) or FA_DTYPE_F16 (IEEE half, the 16-bit type of [ipu]'s op
 *  definition), the 16-bit types with fp32 accumulation.  L, Dvec, dQ, dK, dV are float32
 *  (flash_attn_bwd_grad16 aside).
 *
 *  Pointers are DEVICE pointers (HIP device memory of the current device), 16-byte aligned.
 *  The caller owns every buffer; the library keeps no pointer to them after a call returns.
 *  Calls are asynchronous on `stream` (0 = the null stream): they return after enqueueing,
 *  and errors raised while the kernels run surface at the caller's next synchronisation.
 *  Every output is overwritten (never accumulated into).
 *
 *  Errors: arguments are validated on the host before anything is enqueued.
 *    FA_ERR_INVALID_ARG  null pointer, B/T/H/HKV/D < 1, H % HKV != 0, window < 0,
 *                        scale not finite or <= 0, dtype not one of the values below,
 *                        misaligned pointer, size overflow (T or Tk above 2^30 rows,
 *                        B*T*H*D > 2^40 elements, or for bf16 the T rows of one head
 *                        spanning 2 GiB), an unusable layout (flash_attn_*_strided), tile
 *                        sizes that are not supported values;
 *    FA_ERR_UNSUPPORTED  a valid request this build has no kernel for (head dim);
 *    FA_ERR_HIP          a HIP runtime error while enqueueing (hipGetLastError) or while
 *                        taking the backward's workspace.
 *  No C++ exception crosses this interface.
 *
 *  Supported head dims: FA_DTYPE_F32: D a multiple of 8 in [8, 128];
 *                       FA_DTYPE_BF16, FA_DTYPE_F16: D in {64, 128}.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums span the whole int range (the _RANGE_ markers are not values to pass): any int a
 * caller puts in an fa_dtype_t is a valid object, and the library answers unknown values with
 * FA_ERR_INVALID_ARG. */
typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,
    FA_ERR_UNSUPPORTED = 2,
    FA_ERR_HIP = 3,
    FA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    FA_STATUS_RANGE_MAX_ = 2147483647
} fa_status_t;

typedef enum {
    FA_DTYPE_F32 = 0,
    FA_DTYPE_BF16 = 1,
    FA_DTYPE_F16 = 2,
    FA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    FA_DTYPE_RANGE_MAX_ = 2147483647
} fa_dtype_t;

/* Forward ([forge] flash_attn_fwd; [ipu] flashAttentionQKVPackedWithStash; [teeny] forward):
 * O = softmax(scale * Q K^T, masked) V per (b, h), and L = row log-sum-exp of the masked,
 * scaled scores.  Inputs Q, K, V (dtype); outputs O (dtype) and L (float32). */
fa_status_t flash_attn_fwd(const void* Q, const void* K, const void* V, void* O, float* L,
                           int B, int T, int H, int HKV, int D, float scale, int causal,
                           int window, fa_dtype_t dtype, hipStream_t stream);

/* Backward of the loss sum(O * dO) ([forge] backward kernels; [ipu]
 * flashAttentionQKVPackedGrad; [teeny] backward_dq / backward_dkv):
 *   Dvec_i = dO_i . O_i;  P = exp(scale * Q K^T - L) on visible entries;  dP = dO V^T;
 *   dS = P * (dP - Dvec);  dQ = scale dS K;  dK = scale dS^T Q;  dV = P^T dO,
 * dK and dV summed over the H/HKV query heads of each KV head.  O and L must be the forward's
 * outputs for the same inputs.  Outputs dQ, dK, dV are float32.  Runs flash_attn_bwd_dq_dvec
 * and then flash_attn_bwd_dkdv on `stream`.  The Dvec workspace (B*H*T floats) comes from a
 * per-device cache of at most 4 buffers that the library keeps until the process ends: a
 * call allocates (hipMalloc) only on a device's first calls and when a larger problem comes,
 * and never makes the host wait for the GPU except on such growth.  Reuse of a buffer that
 * another call may still read is ordered on the GPU (hipStreamWaitEvent), so calls on any
 * streams and host threads are safe; concurrent calls on one device take the cache's lock for
 * the few microseconds of their enqueueing.  Under stream capture the workspace is allocated
 * stream-ordered (hipMallocAsync / hipFreeAsync) instead, which a graph records as memory
 * nodes. */
fa_status_t flash_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                           const float* L, const void* dO, float* dQ, float* dK, float* dV,
                           int B, int T, int H, int HKV, int D, float scale, int causal,
                           int window, fa_dtype_t dtype, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): flash_attn_bwd without the per-call
 * workspace.  Same arguments, kernels and results (bit for bit) as flash_attn_bwd; the Dvec
 * workspace is instead a fixed array of FA_NOALLOC_MAX_DVEC floats (16 MiB) in device memory
 * that the library holds on each device it runs on until the process ends.  The call makes no
 * allocation (no hipMalloc / hipMallocAsync / hipFree) and enqueues only the two kernels.
 * B * H * T above FA_NOALLOC_MAX_DVEC returns FA_ERR_UNSUPPORTED before anything is enqueued.
 * Every call on one device shares that device's array: calls that may run at the same time on
 * one device (other streams, other host threads) race on it and must be ordered by the caller.
 * The array keeps the last call's contents; nothing in it needs clearing (each call writes
 * every Dvec value it reads).  The first call on a device looks up the array's address
 * (hipGetSymbolAddress); later calls reuse it. */
#define FA_NOALLOC_MAX_DVEC 4194304
fa_status_t flash_attn_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                                   const float* L, const void* dO, float* dQ, float* dK,
                                   float* dV, int B, int T, int H, int HKV, int D, float scale,
                                   int causal, int window, fa_dtype_t dtype, hipStream_t stream);

/* As flash_attn_fwd / flash_attn_bwd, with the block tiling forced: bq query rows by bk keys
 * per block (0, 0 = the library's choice).  FA_DTYPE_F32 accepts bq in {32, 64} and
 * bk in {16, 32, 64}; the 16-bit types accept (0, 0) or their one tiling.  The tiling decides
 * which blocks are skipped, computed without a mask, or masked (causal diagonal, window edge,
 * ragged T); results agree with the automatic tiling up to rounding order. */
fa_status_t flash_attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* L,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk);
fa_status_t flash_attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O,
                              const float* L, const void* dO, float* dQ, float* dK, float* dV,
                              int B, int T, int H, int HKV, int D, float scale, int causal,
                              int window, fa_dtype_t dtype, hipStream_t stream, int bq, int bk);

/* Element strides of a [B, T, heads, D] tensor view: `batch`, `row` and `head` are the
 * distances, in elements, from (b, t, h, 0) to (b + 1, t, h, 0), (b, t + 1, h, 0) and
 * (b, t, h + 1, 0); the D elements of a row are contiguous.  For a tensor of `heads` heads:
 *   contiguous [B, T, heads, D] (the layout of the entry points above): {T*heads*D, heads*D, D}
 *   [B, heads, T, D] ([metal5] backprop_attention) and [B*heads, T, D] ([teeny] module
 *   comment): {heads*T*D, D, T*D}
 *   each third of a packed [3, B*H, T, D] QKV buffer ([ipu] flashAttentionQKVPackedWithStash,
 *   whose qkv is 3 x G x L x D): the [B, H, T, D] strides, from that third's base pointer. */
typedef struct fa_layout {
    int64_t batch, row, head;
} fa_layout_t;

/* As flash_attn_fwd / flash_attn_bwd on strided views, and with T query rows and Tk keys
 * (Tk = T for the other entry points).  Q, O, dO and dQ follow q_layout (H heads, T rows),
 * K, V, dK and dV follow kv_layout (HKV heads, Tk rows), in elements of each tensor's own
 * type (so the float32 gradients take the same element strides as their 16-bit inputs); L
 * and Dvec stay [B, H, T] float32.  Default tiling.  A layout is rejected
 * (FA_ERR_INVALID_ARG) unless its strides are non-negative multiples of 16 bytes, row >= D,
 * distinct (b, t, head) never overlap, and, for the 16-bit types, one head's rows span under
 * 2 GiB.
 * Query and key lengths ([teeny] flash_attention2_forward, its n_ctx_q and n_ctx_k; no page
 * states a causal rule for them): query row i sits at key position i + Tk - T, the last T
 * positions, as when the keys start with a cached prefix.  causal keeps keys j <= i + Tk - T,
 * window keeps j >= i + Tk - T - window + 1; a row with no visible key gets O = 0 and L = 0
 * (when T > Tk under causal, the first T - Tk rows). */
fa_status_t flash_attn_fwd_strided(const void* Q, const void* K, const void* V, void* O,
                                   float* L, int B, int T, int Tk, int H, int HKV, int D,
                                   float scale, int causal, int window, fa_dtype_t dtype,
                                   hipStream_t stream, fa_layout_t q_layout,
                                   fa_layout_t kv_layout);
fa_status_t flash_attn_bwd_strided(const void* Q, const void* K, const void* V, const void* O,
                                   const float* L, const void* dO, float* dQ, float* dK,
                                   float* dV, int B, int T, int Tk, int H, int HKV, int D,
                                   float scale, int causal, int window, fa_dtype_t dtype,
                                   hipStream_t stream, fa_layout_t q_layout,
                                   fa_layout_t kv_layout);

/* As flash_attn_bwd_strided, with dQ, dK and dV written in the input's 16-bit type (dtype
 * FA_DTYPE_BF16 or FA_DTYPE_F16; FA_DTYPE_F32 is FA_ERR_INVALID_ARG) instead of float32:
 * each value is the float32 result of flash_attn_bwd_strided rounded to nearest-even, at the
 * same element strides.  Halves the gradient traffic; gradients of magnitude above ~4 lose
 * more than the bf16 path's absolute bound on float32 outputs, so it suits consumers that
 * keep 16-bit gradients anyway. */
fa_status_t flash_attn_bwd_grad16(const void* Q, const void* K, const void* V, const void* O,
                                  const float* L, const void* dO, void* dQ, void* dK, void* dV,
                                  int B, int T, int Tk, int H, int HKV, int D, float scale,
                                  int causal, int window, fa_dtype_t dtype, hipStream_t stream,
                                  fa_layout_t q_layout, fa_layout_t kv_layout);

/* Backward stage 1 ([ipu] flashAttentionQKVPackedGrad, its D = rowsum(O * grad) step;
 * [forge] backward section comment; [teeny] backward_dq): Dvec[b,h,i] = sum_d dO[b,i,h,d] *
 * O[b,i,h,d], accumulated in float32.  Dvec is a caller-owned [B,H,T] float32 buffer. */
fa_status_t flash_attn_bwd_preprocess(const void* O, const void* dO, float* Dvec, int B, int T,
                                      int H, int D, fa_dtype_t dtype, hipStream_t stream);

/* Backward stage 2 ([forge] flash_attn_bwd_dv / flash_attn_bwd_dk; [teeny] backward_dkv;
 * [ipu] flashAttentionQKVPackedGrad outer loop over key chunks): dK and dV, each key block
 * owned by one workgroup that loops over the query heads of its group and the query blocks
 * that see it, so every element is written once, without atomics.  Dvec from stage 1. */
fa_status_t flash_attn_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dvec, float* dK, float* dV, int B,
                                int T, int H, int HKV, int D, float scale, int causal,
                                int window, fa_dtype_t dtype, hipStream_t stream, int bq,
                                int bk);

/* Backward stage 3 ([forge] flash_attn_bwd_dq; [teeny] backward_dq): dQ, one query block per
 * workgroup looping over the key blocks it sees.  Dvec from stage 1. */
fa_status_t flash_attn_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
                              const float* L, const float* Dvec, float* dQ, int B, int T,
                              int H, int HKV, int D, float scale, int causal, int window,
                              fa_dtype_t dtype, hipStream_t stream, int bq, int bk);

/* Backward stages 1 and 3 in one pass ([ipu] flashAttentionQKVPackedGrad, its rowsum(O * grad)
 * step; [forge] flash_attn_bwd_dq; [teeny] backward_dq): dQ exactly as flash_attn_bwd_dq, and
 * Dvec[b,h,i] = sum_d dO[b,i,h,d] * O[b,i,h,d] (float32 accumulation) written to the
 * caller-owned [B,H,T] float32 buffer Dvec, which flash_attn_bwd_dkdv then reads.  bf16: one
 * kernel, each query block forming the Dvec values of its own rows from O and the dO rows it
 * loads anyway.  f32: stage 1 then stage 3.  O and dO are [B,T,H,D] like Q; bq, bk as for
 * flash_attn_bwd_dq. */
fa_status_t flash_attn_bwd_dq_dvec(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* L, float* Dvec, float* dQ, int B,
                                   int T, int H, int HKV, int D, float scale, int causal,
                                   int window, fa_dtype_t dtype, hipStream_t stream, int bq,
                                   int bk);

/* QK RMS-norm + rotary prologue ([rope] "qkv_rope.py": module docstring, qk_norm_rope_forward
 * and its forward kernel): from one packed QK projection qk [tokens, 2*heads, qk_dim] (query
 * heads first; element strides qk_stride_t per token and qk_stride_h per head, qk_dim
 * contiguous), each row x is normalised in fp32 as x * rsqrt(mean(x^2) + 2^-23) (no weight)
 * and mixed with its pair-swapped copy (elements 2i and 2i+1 exchanged) through per-token
 * float32 factor tables: y = factor1[t] * x + factor2[t] * swap(x) (tables [tokens, qk_dim],
 * row stride factor_stride_t elements; a rotation has factor1 = cos, factor2 = -sin / +sin on
 * even / odd elements).  Query rows go to out_q, key rows to out_k, both contiguous
 * [tokens, heads, qk_dim] in `dtype`.
 *   paired: logical head h of token t goes to token 2t + h / (heads/2), head h % (heads/2)
 *     (outputs [2*tokens, heads/2, qk_dim]); odd h read the second half of double-width
 *     tables [tokens, 2*qk_dim].  Needs an even head count; not with key_offset.
 *   key_offset: for key heads of tokens t > 0 the elements from rotary_dim on are the previous
 *     token's normalised row instead (rotary_dim even, <= qk_dim).
 * qk_dim in {16, 32, 64, 128, 256} (FA_ERR_UNSUPPORTED otherwise); dtype F32, BF16 or F16;
 * every pointer 16-byte aligned, strides multiples of 16 bytes, qk_stride_h >= qk_dim and
 * qk_stride_t >= (2*heads - 1) * qk_stride_h + qk_dim (a token's rows stored together). */
fa_status_t flash_attn_qk_norm_rope(const void* qk, int64_t qk_stride_t, int64_t qk_stride_h,
                                   const float* factor1, const float* factor2,
                                   int64_t factor_stride_t, void* out_q, void* out_k, int tokens,
                                   int heads, int qk_dim, int rotary_dim, int paired,
                                   int key_offset, fa_dtype_t dtype, hipStream_t stream);

/* ---- host-only helpers (no GPU needed) ---- */

/* Human-readable name of a status code (static string). */
const char* flash_attn_status_string(fa_status_t s);

/* Class of block (i, j) — query rows [i*bq, i*bq+bq) by keys [j*bk, j*bk+bk) of a T x T
 * problem — exactly as the kernels decide it: 0 = skipped (nothing visible), 1 = computed
 * without a mask (every in-range element visible), 2 = computed with the element mask
 * (causal diagonal, window edge, or keys past T).  *off receives i*bq - j*bk, from which the
 * kernels rebuild the mask (keep c <= r + off, c >= r + off - window + 1); this is the
 * quantity whose cycle [ipu] getTriuOffsetSequence enumerates (as off + 1).
 * Returns -1 on invalid arguments. */
int flash_attn_block_class(int T, int bq, int bk, int causal, int window, int i, int j,
                           int* off);

/* Key-block range [*j_lo, *j_hi) a query tile i loops over (same rule as the kernels). */
fa_status_t flash_attn_kv_block_range(int T, int bq, int bk, int causal, int window, int i,
                                      int* j_lo, int* j_hi);

/* The same two for T query rows against Tk keys (the rule of flash_attn_fwd_strided). */
int flash_attn_block_class_qk(int Tq, int Tk, int bq, int bk, int causal, int window, int i,
                              int j);
fa_status_t flash_attn_kv_block_range_qk(int Tq, int Tk, int bq, int bk, int causal, int window,
                                         int i, int* j_lo, int* j_hi);

/* Tiling the library picks for a dtype / head dim: pass 0 = forward, 1 = dK/dV, 2 = dQ.
 * *bq, *bk are the query and key block sizes of that pass. */
fa_status_t flash_attn_default_tiles(fa_dtype_t dtype, int D, int pass, int* bq, int* bk);

/* The layout check flash_attn_*_strided apply to each view: FA_OK if `layout` describes a
 * usable [B, T, heads, D] view of element type `dtype` (strides non-negative multiples of
 * 16 bytes, row >= D, no two (b, t, head) rows overlapping, and for bf16 one head's T rows
 * spanning under 2 GiB), FA_ERR_INVALID_ARG otherwise. */
fa_status_t flash_attn_check_layout(fa_layout_t layout, int B, int T, int heads, int D,
                                    fa_dtype_t dtype);

/* Measurement helper (not part of the attention path): a kernel of `grid` workgroups of 256
 * threads (four waves) in which every wave issues iters * 32 bf16 MFMA 16x16x32 operations
 * (16384 FLOP each; the shape the attention kernels use) on fixed operands, so the launch
 * performs grid * 4 * iters * 32 * 16384 FLOP.  `operands` holds 4096 bf16 values (lane l's 16-byte fragments at element offsets
 * (i*64 + l)*8, i < 8), loaded once per wave; their distribution decides the rate, since the
 * chip's power limit depends on the bits the MFMA units switch.  `out` receives grid * 256
 * floats (sums of the accumulators, so the work is not optimised away).  Device pointers,
 * 16-byte aligned; 1 <= grid <= 2^20, 1 <= iters <= 2^24. */
fa_status_t flash_attn_mfma_rate_probe(const void* operands, float* out, int grid, int iters,
                                       hipStream_t stream);

/* Library ABI version (major * 100 + minor). */
int flash_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
