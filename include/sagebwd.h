/*
 * sagebwd.h - C ABI of a SageBwd-style trainable INT8 attention for AMD MI355X (gfx950).
 *
 * The method (SageBwd article, "SageBwd: a trainable low-bit attention mechanism",
 * aitrends.kr article 8227):
 *   - QK-norm: every token vector of Q and K is RMS-normalised over the head dim, gain 1
 *     (article, QK-norm paragraph);
 *   - K-smoothing: the per-channel mean of the normalised keys over all N tokens of a head
 *     is subtracted right before quantisation (article, K-smoothing paragraph; the axis is
 *     fixed by the Q-smoothing paragraph's bias term (dS^T 1) mu_Q^T, a d-vector over tokens);
 *   - per-block INT8 quantisation (article, per-block kernels paragraph): one float32 scale
 *     per `blk` tokens x d channels, scale = absmax/127, codes = round-to-nearest-even of
 *     x * (127/absmax) clamped to [-127, 127]; an all-zero block has scale 0 and codes 0;
 *   - six of attention's seven matmuls in INT8 with int32 accumulation (forward QK^T, PV;
 *     backward recomputed QK^T, dV = P^T dO, dK = dS^T Q, dQ = dS K) and dP = dO V^T in the
 *     16-bit input type with float32 accumulation (article, precision-split paragraph);
 *   - a flash-style forward and backward that never writes the N x N scores to memory
 *     (TurboQuant blog, FlashAttention section);
 *   - optionally Q-smoothing (article, Q-smoothing paragraph, which names the bias term
 *     (dS^T 1) mu_Q^T): the queries' per-channel mean mu_Q over the N tokens of a head is
 *     subtracted before quantising Q; every score then gets back the per-key bias
 *     b_k = (K~ mu_Q)_k, taken from the dequantised K codes, b_k = Ks * (Kc_k . mu_Q); and dK
 *     gets dK_bias = (dS^T 1) mu_Q^T, with dS the dequantised dS codes of each tile summed
 *     over its queries. dQ is unchanged.
 *
 * In-kernel quantisation tiles (P~ in the forward, P and dS in the backward) use the same
 * absmax/127 rule in float32, except that the kernels take 127/absmax from the hardware
 * reciprocal and round x * (127/absmax) once (fused), so a code can differ from the rule's
 * by one at a near-tie; these codes stay inside the kernels:
 *   P~ (forward)   : SAGEBWD_FWD_TILE_Q query rows x blk keys; the online-softmax running
 *                    max moves once per such tile and P~ = exp(s - running max); the row
 *                    sum l accumulates P~ before quantisation.
 *   P  (backward)  : blk query rows (one query block) x SAGEBWD_BWD_P_TILE_K keys.
 *   dS (backward)  : blk query rows x SAGEBWD_BWD_DS_TILE_K keys.
 * Every tile lies inside one blk x blk block, so the block scales factor out of each
 * integer product. The tile shapes are compile-time constants of the kernels (the macros
 * below); the caller cannot choose them.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors), contiguous,
 *     16-byte aligned. Shapes are given in [B,H,N,d] order, last index fastest, except that
 *     the 16-bit tensors follow sagebwd_params.layout ([B,N,H,d] with SAGEBWD_LAYOUT_BNHD).
 *   - N need not be a multiple of blk: the last quantisation block of a head then holds
 *     N mod blk tokens (its absmax, and the means, cover those tokens only). The 16-bit
 *     tensors hold exactly N tokens per head; every array of the library's own (codes,
 *     scales, statistics, lse) holds Np = N rounded up to a multiple of blk, the tokens from
 *     N on being padding (codes 0, rstd 1, lse +inf; their other statistics are not
 *     meaningful). Padding tokens are never normalised, so eps = 0 is valid with any N.
 *   - The caller owns every buffer. The library allocates nothing, keeps no state between
 *     calls, never synchronises, and is re-entrant; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream). Calls sharing a workspace must be
 *     ordered on one stream.
 *   - Inputs are never written. Outputs are fully overwritten.
 *   - Argument errors are reported before anything is enqueued and before any HIP call.
 *     A failed launch returns SAGEBWD_ERR_HIP. Faults inside kernels surface at the
 *     caller's next synchronisation, as usual in HIP. NaN/Inf inputs give unspecified
 *     (but memory-safe) results. No exception crosses this boundary.
 *   - N == 0 (or B == 0 or H == 0) is valid and enqueues nothing.
 */
#ifndef SAGEBWD_H
#define SAGEBWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGEBWD_FWD_TILE_Q 32
#define SAGEBWD_BWD_P_TILE_K 16
#define SAGEBWD_BWD_DS_TILE_K 64
/* Q-Attn split: keys per forward tile (the online-softmax step; P~ is not quantised there) */
#define SAGEBWD_QATTN_FWD_TILE_K 64

typedef enum {
  SAGEBWD_OK = 0,
  SAGEBWD_ERR_NULL = -1,        /* a required pointer is NULL                               */
  SAGEBWD_ERR_SHAPE = -2,       /* negative size, N > 2^22, B*H > 2^24, or 3*B*H*ceil(N/blk)
                                   >= 2^31 (the prologue's workgroups)                      */
  SAGEBWD_ERR_UNSUPPORTED = -3, /* d or blk not in {64, 128}, unknown dtype, dq_mode or
                                   layout or fmt or split, eps < 0, qk_gain or
                                   normed_grads without qk_norm, normed_grads with qk_gain,
                                   q_smooth with FP8 or with the Q-Attn split               */
  SAGEBWD_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                         */
  SAGEBWD_ERR_WORKSPACE = -5,   /* workspace smaller than the *_workspace_bytes() figure    */
  SAGEBWD_ERR_HIP = -6,         /* a kernel launch failed                                   */
  SAGEBWD_ERR_SCRATCH = -7      /* the allocation-free entry point's static scratch is too
                                   small for the problem                                    */
} sagebwd_status;

typedef enum { SAGEBWD_FP16 = 0, SAGEBWD_BF16 = 1 } sagebwd_dtype;

typedef struct {
  int32_t B, H, N, d;   /* batch, heads, tokens, head dim (d in {64, 128})                  */
  int32_t blk;          /* quantisation block, tokens (64 or 128)                            */
  int32_t causal;       /* nonzero: key j is visible to query i iff j <= i                  */
  int32_t qk_norm;      /* nonzero: RMSNorm Q and K per token (gain 1 unless qk_gain)       */
  int32_t k_smooth;     /* nonzero: subtract K's per-channel mean before quantising         */
  float eps;            /* RMSNorm epsilon (>= 0), e.g. 1e-6; with eps = 0 an all-zero
                           token has no defined norm and its results are unspecified          */
  float sm_scale;       /* softmax scale; <= 0 selects 1/sqrt(d)                            */
  int32_t dtype;        /* sagebwd_dtype of Q, K, V, dO, O, dQ, dK, dV                       */
  int32_t dq_mode;      /* how the backward reduces dQ over key blocks (sagebwd_dq_mode)     */
  int32_t q_smooth;     /* nonzero: subtract Q's per-channel mean before quantising and add
                           the key bias / dK_bias terms back (see above)                    */
  int32_t layout;       /* sagebwd_layout of the 16-bit tensors Q, K, V, O, dO, dQ, dK, dV   */
  int32_t qk_gain;      /* nonzero (needs qk_norm): learnable QK-norm gains q_gain, k_gain
                           [H,d] float32, Q^ = g_Q o RMSNorm(Q) and K^ = g_K o RMSNorm(K) per
                           head and channel (SageBwd article, QK-norm paragraph: RMSNorm per
                           token, here with its weight); the backward also returns their
                           gradients dq_gain, dk_gain [H,d] (sums over batch and tokens)     */
  int32_t normed_grads; /* nonzero (with qk_norm, without qk_gain): the backward returns dQ,
                           dK with respect to the normalised Q^, K^ (before smoothing) and
                           leaves the RMSNorm backward to the caller                         */
  int32_t fmt;          /* sagebwd_fmt of the quantised products' codes (INT8 or FP8)         */
  int32_t split;        /* sagebwd_split: which of the seven products are quantised          */
} sagebwd_params;

/* Precision split of attention's seven products.
 * SAGEBWD_SPLIT_SAGEBWD (SageBwd article, precision-split paragraph): six products quantised
 *   (forward QK^T and PV; backward recomputed QK^T, dV = P^T dO, dK = dS^T Q, dQ = dS K),
 *   dP = dO V^T in the 16-bit input type.
 * SAGEBWD_SPLIT_QATTN (Full-Stack FP4 page, section 2.4, mixed-precision attention): the
 *   robust paths stay quantised, QK^T (forward and recomputed) and the dS products dK and dQ;
 *   the softmax-sensitive paths PV, P^T dO and dO V^T run on the 16-bit MFMA in the inputs'
 *   16-bit type (the page's BF16 is the bf16 inputs' type; fp16 inputs use fp16): P~ and P are
 *   rounded to it (nearest even) and V and dO enter with their own values, float32
 *   accumulation. The forward's key tile is SAGEBWD_QATTN_FWD_TILE_K keys (the running max
 *   moves once per tile and P~ = exp(s - running max) exactly, no lagging reference); the
 *   forward reads the raw V (sagebwd_forward's V argument) and ignores the V codes; the
 *   backward's P and dS tiles are as above, P only rounded. Not with q_smooth. */
typedef enum { SAGEBWD_SPLIT_SAGEBWD = 0, SAGEBWD_SPLIT_QATTN = 1 } sagebwd_split;

/* Code format of the quantised products. The SageBwd article's precision split names only
 * INT8 and FP16; FP8 attention is named by the Full-Stack FP4 page (section 1, problem
 * definition: attention kept in BF16 or FP8), and block-scaled FP8 training with the E4M3
 * format by the NVFP4 / Quartet 2 page. SAGEBWD_FMT_INT8:
 * codes in [-127, 127], scale absmax/127, int32 products (the method as described above).
 * SAGEBWD_FMT_FP8: OCP float8 e4m3fn codes (bias 7, subnormals kept, largest finite 448),
 * scale absmax/448, codes = e4m3 round-to-nearest-even of fl(x * (448/absmax)); the same
 * blocks, tiles, byte layouts and buffer sizes, products accumulated by the FP8 matrix
 * cores in float32 (not exactly). In-kernel tiles (P~, P, dS) round fl(x * 448/absmax) with
 * the hardware reciprocal. FP8 is not available with q_smooth (SAGEBWD_ERR_UNSUPPORTED). */
typedef enum { SAGEBWD_FMT_INT8 = 0, SAGEBWD_FMT_FP8 = 1 } sagebwd_fmt;

/* Memory layout of the 16-bit tensors (Q, K, V, O, dO, dQ, dK, dV; contiguous either way).
 * BHND is [B,H,N,d]; BNHD is [B,N,H,d], the layout a fused QKV projection produces, read and
 * written in place (no transposing copies). Every other tensor (codes, scales, statistics,
 * lse) keeps its documented [B,H,...] layout. */
typedef enum { SAGEBWD_LAYOUT_BHND = 0, SAGEBWD_LAYOUT_BNHD = 1 } sagebwd_layout;

/* dQ = dS K sums over every key block. SAGEBWD_DQ_SPILL writes each (64-query, blk-key) tile
 * of INT8 dS codes once to the workspace and contracts them with K in a query-major pass
 * (plain stores, O(N^2/2) bytes of scratch per head when causal). SAGEBWD_DQ_ATOMIC adds
 * each tile's float32 dQ contribution with atomics (O(N) scratch, but the atomic traffic is
 * (Np/blk) * Np * d * 4 bytes per head). SAGEBWD_DQ_AUTO picks SPILL while its scratch is at
 * most SAGEBWD_DQ_AUTO_SPILL_LIMIT bytes, else ATOMIC. Both give the same dQ up to float32
 * summation order. SPILL also needs one head's dS tiles (T * 64 * blk bytes, T below) under
 * 4 GiB: AUTO picks ATOMIC beyond that, and an explicit SPILL is rejected
 * (SAGEBWD_ERR_UNSUPPORTED from the backward, 0 from the workspace query). */
typedef enum { SAGEBWD_DQ_AUTO = 0, SAGEBWD_DQ_SPILL = 1, SAGEBWD_DQ_ATOMIC = 2 } sagebwd_dq_mode;
#define SAGEBWD_DQ_AUTO_SPILL_LIMIT (16ull << 30)

/* Bytes of scratch sagebwd_quant_prologue needs: the per-block channel sums of the
 * normalised keys, float32 [B,H,Np/blk,d], when k_smooth is on, then (256-byte aligned) those
 * of the normalised queries when q_smooth is on (0 when both are off). Returns 0 for
 * invalid params. */
size_t sagebwd_prologue_workspace_bytes(const sagebwd_params* p);

/* Quantisation prologue: QK-norm -> K-smoothing (and Q-smoothing) -> per-block INT8 codes
 * and scales. The codes, scales and statistics are the "quantised views" both passes reuse
 * (the Full-Stack FP4 page, section 2.4, reuses quantised Q, K, V between the passes).
 *   Q, K, V  in : dtype [B,H,N,d]
 *   Qc, Kc   out: int8 [B,H,Np,d]  codes of Q^ (of Q~ = Q^ - q_mean with q_smooth) and of
 *                                  K~ = K^ - mean (smoothed keys)
 *   Vtc      out: int8 [B,H,d,Np]  codes of V, stored TRANSPOSED (channel-major)
 *   Qs,Ks,Vs out: float32 [B,H,Np/blk]  block scales
 *   q_rstd, k_rstd out: float32 [B,H,Np]  1/sqrt(mean(x^2)+eps) per token (1 if !qk_norm)
 *   k_mean   out: float32 [B,H,d]  the subtracted mean (0 if !k_smooth)
 *   q_mean   out: float32 [B,H,d]  the subtracted query mean (q_smooth only; else ignored,
 *                                  may be NULL)
 *   kbias    out: float32 [B,H,Np] b_k = Ks * (Kc_k . q_mean), float32 sum over channels
 *                                  (q_smooth only; else ignored, may be NULL)
 *   q_gain, k_gain in: float32 [H,d]  QK-norm gains (qk_gain only; else ignored, may be NULL)
 *   workspace   : >= sagebwd_prologue_workspace_bytes(p) bytes (may be NULL if that is 0)
 * Bit-exact contract: per token, the d channels form 16 chunks of d/16 consecutive
 * channels; each chunk sums x*x in ascending channel order in float32, and ss is the
 * pairwise tree of the 16 chunk sums ((c0+c1), (c2+c3), ..., then pairs of those, down to
 * one); rstd = 1/sqrt(ss/d + eps) with correctly rounded float32 division and square
 * root; x^ = x*rstd (then x^ = x^*g[h][c] with qk_gain, one float32 product); the mean:
 * inside each block, token t joins group t mod 16, each group
 * sums its tokens in ascending order and the block sum is the same pairwise tree of the 16
 * group sums; the block sums are then added in ascending block order and divided by N;
 * K~ = K^ - mean; then the INT8 rule above. q_mean is taken the same way from Q^ (and
 * Q~ = Q^ - q_mean). kbias is not bit-specified (float32, any summation order). */
sagebwd_status sagebwd_quant_prologue(const sagebwd_params* p,
                                      const void* Q, const void* K, const void* V,
                                      int8_t* Qc, int8_t* Kc, int8_t* Vtc,
                                      float* Qs, float* Ks, float* Vs,
                                      float* q_rstd, float* k_rstd, float* k_mean,
                                      float* q_mean, float* kbias,
                                      const float* q_gain, const float* k_gain,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Allocation-free variant of sagebwd_quant_prologue, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, computation and outputs (bit for bit), without the workspace:
 * the prologue's scratch comes from a static device array of SAGEBWD_NOALLOC_SCRATCH_BYTES
 * bytes, which each GPU holds from the first call on it until the process ends. The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *   - Problems with sagebwd_prologue_workspace_bytes(p) > SAGEBWD_NOALLOC_SCRATCH_BYTES are
 *     rejected with SAGEBWD_ERR_SCRATCH, after the argument checks and before any HIP call
 *     (16 MiB covers e.g. B*H*ceil(N/blk)*d <= 4M, so K-smoothing at B*H = 32, N = 32768,
 *     d = 128, blk = 128 needs 1 MiB).
 *   - After the argument checks the call looks up the current device (and, if stream is not
 *     NULL, the stream's device, which must be the current one: else SAGEBWD_ERR_HIP with
 *     hipErrorInvalidDevice) and, on the first call per device, the array's device address.
 *   - Every call on one GPU shares that GPU's array. Calls ordered on one stream are safe;
 *     calls that may overlap in time on one GPU (other streams, unordered host threads) race
 *     on it and give undefined results. The kernels write every scratch byte they read
 *     within the same call, so nothing carries over from an earlier call. */
#define SAGEBWD_NOALLOC_SCRATCH_BYTES (16ull << 20)
sagebwd_status sagebwd_quant_prologue_noalloc(const sagebwd_params* p,
                                              const void* Q, const void* K, const void* V,
                                              int8_t* Qc, int8_t* Kc, int8_t* Vtc,
                                              float* Qs, float* Ks, float* Vs,
                                              float* q_rstd, float* k_rstd, float* k_mean,
                                              float* q_mean, float* kbias,
                                              const float* q_gain, const float* k_gain,
                                              void* stream);

/* Forward: O = softmax(sm_scale * Q^ K~^T [causal mask]) V with INT8 QK^T and PV.
 *   inputs : the prologue's Qc, Kc, Vtc, Qs, Ks, Vs, and its kbias with q_smooth (each
 *            score is then sm_scale * (Q~ K~^T + b_k); kbias ignored, may be NULL, without)
 *   V   in : dtype [B,H,N,d] (layout as Q): the raw values, read by the Q-Attn split's
 *            16-bit PV (Vtc and Vs are then ignored and may be NULL); ignored, may be NULL,
 *            with the SageBwd split
 *   O   out: dtype [B,H,N,d]
 *   lse out: float32 [B,H,Np], natural-log logsumexp of each row of the scaled scores
 *            (+inf for the padding rows from N on) */
sagebwd_status sagebwd_forward(const sagebwd_params* p,
                               const int8_t* Qc, const int8_t* Kc, const int8_t* Vtc,
                               const float* Qs, const float* Ks, const float* Vs,
                               const float* kbias, const void* V, void* O, float* lse, void* stream);

/* Bytes of scratch sagebwd_backward needs. Layout (each region starts on a 256-byte
 * boundary, in this order; "chunk" = 16 bytes):
 *   packets [B,H,Np/64] x P bytes     P = 17408 for d = 64, 33792 for d = 128: for each head
 *           and each 64-token tile, the tile's data in the order the key-block kernel copies
 *           it into LDS (r = token inside the tile, c = channel):
 *     [0, 64d)      Q codes [64][d]; chunk j of row r stored at chunk
 *                   j^(((r>>1)^((r>>4)<<2))&7) (d = 128) or j^((r>>1)&3) (d = 64)
 *     [64d, 192d)   dO [64][d], 16-bit; chunk j of row r stored at chunk j^(r&15) (d = 128)
 *                   or j^(r&7) (d = 64)
 *     [192d, 256d)  dO INT8 codes, channel-major [d][64]: token u of row c at byte
 *                   16*((u>>2)&3) + 4*(u>>4) + (u&3), then chunk j of row c stored at
 *                   chunk j^((c>>1)&3)
 *     [256d, +256)  lse * log2(e), float32 [64]
 *     [+256, +512)  D = rowsum(dO o O), float32 [64]
 *     [+512, +516)  the Q block scale; [+516, +520) the dO block scale (float32); padding
 * then, with dq_mode ATOMIC:
 *   dq_acc  float32 [B,H,Np,d]       dQ of the normalised queries, accumulated
 * or, with dq_mode SPILL (T = tiles per head = nb*nt - (blk/64)*nb*(nb-1)/2 when causal,
 * nb*nt otherwise, nb = Np/blk, nt = Np/64; tile (kb, t) of key block kb and query tile t has
 * index kb*nt - (blk/64)*kb*(kb-1)/2 + t - kb*blk/64 when causal, kb*nt + t otherwise):
 *   ktp     [B,H,Np/blk] x d*blk      K codes of each key block, channel-major [d][blk];
 *                                    chunk j of row c stored at chunk j^(c&7) (blk = 128)
 *                                    or j^((c>>1)&3) (blk = 64)
 *   dsp     [B,H,T] x 64*blk         INT8 dS codes of each tile, key-major [blk][64]:
 *                                    token u of the query tile at byte position
 *                                    16*((u>>2)&3) + 4*(u>>4) + (u&3) of the key's row,
 *                                    then chunk j of row k stored at chunk
 *                                    j^(((k>>1)^(k>>4))&3)
 *   dsm     float32 [B,H,T,blk/64]   per 64 keys of the tile (one dS scale tile):
 *                                    sm_scale * (dS tile scale) * (K block scale)
 * then, with qk_gain:
 *   gq      float32 [B,H,Np/64,d]    partial dq_gain of each 64-query tile
 *   gk      float32 [B,H,Np/blk,d]   partial dk_gain of each key block
 * Returns 0 for invalid params. */
size_t sagebwd_backward_workspace_bytes(const sagebwd_params* p);

/* Backward. Gradients are with respect to the RAW Q, K, V given to the prologue (the
 * RMSNorm backward is applied; K-smoothing adds no term because every row of dS sums to 0),
 * or with normed_grads with respect to the normalised Q^, K^.
 *   Q, K, V       in : dtype [B,H,N,d], the prologue's inputs
 *   Qc, Kc, Qs, Ks, q_rstd, k_rstd in: the prologue's outputs
 *   q_mean, kbias in : the prologue's outputs with q_smooth (ignored, may be NULL, without)
 *   q_gain, k_gain in : float32 [H,d], the prologue's gains with qk_gain (else ignored)
 *   O, lse        in : the forward's outputs
 *   dO            in : dtype [B,H,N,d]
 *   dQ, dK, dV    out: dtype [B,H,N,d]
 *   dq_gain, dk_gain out: float32 [H,d], the gains' gradients with qk_gain (else ignored,
 *                    may be NULL); float32 sums over tiles in a fixed order (deterministic)
 *   workspace        : >= sagebwd_backward_workspace_bytes(p) bytes, layout above */
sagebwd_status sagebwd_backward(const sagebwd_params* p,
                                const void* Q, const void* K, const void* V,
                                const int8_t* Qc, const int8_t* Kc,
                                const float* Qs, const float* Ks,
                                const float* q_rstd, const float* k_rstd,
                                const float* q_mean, const float* kbias,
                                const float* q_gain, const float* k_gain,
                                const void* O, const float* lse, const void* dO,
                                void* dQ, void* dK, void* dV,
                                float* dq_gain, float* dk_gain,
                                void* workspace, size_t workspace_bytes, void* stream);

/* One stage of sagebwd_backward, for callers that schedule or time the stages apart:
 *   part 0: D = rowsum(dO o O), dO codes/scales, the packets (and K^T codes or a zeroed
 *           dq_acc)
 *   part 1: the fused key-block kernel (S, P, dP, dS; dV, dK final; dQ^ accumulated)
 *   part 2: the dQ pass (dQ = dS K from the spilled tiles, or from dq_acc), RMSNorm
 *           backward, rounding to the dtype; with qk_gain also the gains' gradients
 * Arguments as for sagebwd_backward. Running parts 0, 1, 2 in order on one stream with the
 * same workspace is exactly sagebwd_backward; any other order gives undefined results.
 * part outside 0..2 -> SAGEBWD_ERR_UNSUPPORTED. */
sagebwd_status sagebwd_backward_part(const sagebwd_params* p, int32_t part,
                                     const void* Q, const void* K, const void* V,
                                     const int8_t* Qc, const int8_t* Kc,
                                     const float* Qs, const float* Ks,
                                     const float* q_rstd, const float* k_rstd,
                                     const float* q_mean, const float* kbias,
                                     const float* q_gain, const float* k_gain,
                                     const void* O, const float* lse, const void* dO,
                                     void* dQ, void* dK, void* dV,
                                     float* dq_gain, float* dk_gain,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* sagebwd_status_string(sagebwd_status s);

/* Detail of the last SAGEBWD_ERR_HIP returned on the calling host thread: the entry point
 * and the HIP runtime's error name and text for the enqueue that failed. The string is
 * owned by the library, stays valid until the next failing call on the same thread, and
 * is empty if no call on this thread has failed. Never NULL; makes no HIP call. */
const char* sagebwd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGEBWD_H */
