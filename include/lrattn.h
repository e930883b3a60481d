/*
 * lrattn.h - single-token decode attention over a per-head low-rank KV cache
 *            (gfx950 / MI355X, HIP).
 *
 * THE OPERATION
 *   WSVD page ("WSVD: Weighted Low-Rank Approximation for Fast and Efficient
 *   Execution of Low-Precision Vision-Language Models"), section 2.A: every
 *   head's key (and value) projection is factored per head with rank r, so
 *   the cache keeps a compact latent row per token and head, and each head's
 *   K (V) is rebuilt from its own latent times its own r x d factor.
 *   Section 2.C: the decode kernel fuses that rebuild with attention and Flash
 *   Decoding in one flow, keeping intermediates on chip.  AttentionPack page,
 *   section 2.C: the decompression is folded into the attention-score
 *   computation so less data crosses between HBM and on-chip memory.
 *
 *   For every sequence b < B and query head h < Hq, with kv-head
 *   g = h / (Hq / Hkv) and n = seq_lens[b]:
 *
 *     Lk[t] = L_K[b,g,t,:]           (times scales[0,b,g,t] for int8 latents)
 *     Lv[t] = L_V[b,g,t,:]           (times scales[1,b,g,t] for int8 latents)
 *     K[t]  = Lk[t] . B_K[g]         V[t] = Lv[t] . B_V[g]          t < n
 *     p     = softmax_t( softmax_scale * <q[b,h,:], K[t]> )
 *     out[b,h,:] = sum_t p[t] V[t]
 *
 *   The library never forms K or V.  By associativity it scores
 *   (q . B_K^T) . Lk[t] and projects (sum_t p[t] Lv[t]) . B_V, the same
 *   quantity, streaming 2r latent values per token and kv-head instead of 2d.
 *   Flash Decoding: the token axis is cut into num_splits partitions; each
 *   produces (reference max, exp-sum, unnormalized latent accumulator), and a
 *   second kernel merges the partitions of each (b, kv-head) with a
 *   log-sum-exp rule in fixed order and applies B_V.
 *
 * TENSORS (all row-major, contiguous, device memory of the stream's device)
 *   q        [B, Hq, d]            q_dtype       (F32, BF16 or F16)
 *   L_K, L_V [B, Hkv, T, r]        latent_dtype  (F32, BF16, F16 or I8)
 *   B_K, B_V [Hkv, r, d]           factor_dtype  (F32, BF16 or F16)
 *   scales   [2, B, Hkv, T] fp32   index 0 scales K latents, 1 scales V
 *                                  latents; required iff latent_dtype == I8,
 *                                  must be NULL otherwise
 *   seq_lens [B] int32             valid tokens per sequence, read on the
 *                                  device only.  Values above T are treated
 *                                  as T; values <= 0 produce a zero output row
 *                                  (attention over no tokens is undefined).
 *                                  Rows t >= seq_lens[b] are never read.
 *   out      [B, Hq, d]            out_dtype     (F32 or BF16)
 *   T is params.max_seq_len (the token stride of L_K, L_V and scales).
 *
 * SUPPORTED SHAPES
 *   head_dim d in {64, 128, 256}; rank r in {16, 32, 48, 64, 128} with
 *   r * sizeof(latent) <= 256 bytes (so r = 128 needs 1- or 2-byte latents);
 *   group Hq / Hkv in {1, 2, 4, 8}; batch and Hkv <= 65535.
 *   Anything else returns LRATTN_ERR_UNSUPPORTED before any device work.
 *
 * ALIGNMENT
 *   Every tensor pointer and the workspace must be 16-byte aligned.
 *
 * OWNERSHIP AND EXECUTION
 *   The caller owns every buffer, including the workspace (size from
 *   lrattn_workspace_size).  The library allocates nothing, frees nothing and
 *   keeps no pointer after a call returns.  Calls are asynchronous on
 *   `stream` (NULL = the null stream of the current device), never
 *   synchronize the host and read seq_lens only on the device, so they can be
 *   captured in a HIP graph.  The library holds no state: concurrent calls
 *   are safe as long as they do not share a workspace or output buffer.
 *
 * ERRORS
 *   Every entry point returns LRATTN_OK (0) or a negative lrattn_status.  All
 *   argument errors are detected on the host before anything is launched,
 *   and `out` and the workspace are left untouched.  LRATTN_ERR_HIP reports a
 *   failed launch (the HIP error is consumed from hipGetLastError).
 *
 * RESULTS
 *   Scores, softmax and accumulation run in fp32 on exactly-converted inputs.
 *   Where matrix cores take a product (q . B_K^T when q and B_K share a 2-byte
 *   format; the scores for bf16 latents with 4 or 8 query heads per kv-head
 *   and r a multiple of 32) the bf16/fp16 products are exact and summed in
 *   fp32, and q~ enters as three bf16 terms whose sum is q~ exactly.
 *   For a fixed num_splits, build and device, results are bitwise identical
 *   from run to run (fixed reduction order, no atomics).
 */
#ifndef LRATTN_H
#define LRATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* lrattn_stream;

typedef enum lrattn_dtype {
  LRATTN_F32 = 0,
  LRATTN_BF16 = 1,
  LRATTN_F16 = 2,
  LRATTN_I8 = 3
} lrattn_dtype;

typedef enum lrattn_status {
  LRATTN_OK = 0,
  LRATTN_ERR_NULL = -1,        /* a required pointer is NULL, or scales given for float latents */
  LRATTN_ERR_SHAPE = -2,       /* a size is <= 0, Hq not a multiple of Hkv, or sizes overflow */
  LRATTN_ERR_DTYPE = -3,       /* a dtype code outside lrattn_dtype, or not allowed for that tensor */
  LRATTN_ERR_UNSUPPORTED = -4, /* valid request outside the compiled shape set */
  LRATTN_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  LRATTN_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than lrattn_workspace_size */
  LRATTN_ERR_SPLITS = -7,      /* num_splits < 0 or > max_seq_len */
  LRATTN_ERR_HIP = -8,         /* a kernel launch failed */
  LRATTN_ERR_SCRATCH = -9      /* lrattn_decode_static: the records need more than
                                  LRATTN_STATIC_SCRATCH_BYTES */
} lrattn_status;

typedef struct lrattn_params {
  int32_t batch;         /* B */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv, divides Hq */
  int32_t head_dim;      /* d */
  int32_t rank;          /* r */
  int32_t max_seq_len;   /* T: token capacity (stride) of the latent cache */
  int32_t q_dtype;       /* lrattn_dtype of q */
  int32_t latent_dtype;  /* lrattn_dtype of L_K and L_V */
  int32_t factor_dtype;  /* lrattn_dtype of B_K and B_V */
  int32_t out_dtype;     /* lrattn_dtype of out: LRATTN_F32 or LRATTN_BF16 */
  float softmax_scale;   /* logit multiplier; <= 0 selects 1/sqrt(head_dim) */
  int32_t num_splits;    /* Flash-Decoding partitions over T per (b, kv-head);
                            0 lets the library choose (see lrattn_plan) */
} lrattn_params;

/* Library version: major * 10000 + minor * 100 + patch. */
int lrattn_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* lrattn_status_string(int status);

/*
 * Host-only.  Validates `p` and resolves the partition plan:
 * *num_splits = partitions per (b, kv-head) actually used, *split_tokens =
 * tokens per partition (partition i covers [i*split_tokens,
 * (i+1)*split_tokens) intersected with [0, seq_len)).  Either output may be
 * NULL.
 */
int lrattn_plan(const lrattn_params* p, int32_t* num_splits, int32_t* split_tokens);

/*
 * Host-only.  Name of the partition kernel that lrattn_partition (and
 * lrattn_decode) launches for `p`, as profilers list it: static text,
 * "partition_mfma_kernel" (bf16 latents, r a multiple of 32, 4 or 8 query
 * heads per kv-head: scores on the matrix cores) or "partition_kernel".
 * NULL when `p` is invalid or unsupported.
 */
const char* lrattn_partition_kernel(const lrattn_params* p);

/*
 * Partitions per head from which lrattn_decode (and lrattn_partition) forms
 * q . B_K^T once per query head in a small kernel ahead of the partition
 * kernel, instead of in the prologue of every partition's workgroup.  With
 * fewer partitions the absorption stays in the partition kernel.
 */
#define LRATTN_PRE_ABSORB_SPLITS 64

/*
 * Host-only.  Bytes of device workspace lrattn_decode needs for `p`:
 * B * Hq * num_splits * (r + 4) * 4 (one fp32 partial record per query head
 * and partition), rounded up to 256, plus, when num_splits >=
 * LRATTN_PRE_ABSORB_SPLITS, B * Hq * r * 4 for the absorbed queries, rounded
 * up to 256.
 */
int lrattn_workspace_size(const lrattn_params* p, size_t* bytes);

/*
 * The decode step: partition kernel then combine kernel, both on `stream`
 * (with at least LRATTN_PRE_ABSORB_SPLITS partitions per head, the query
 * absorption kernel first).
 * `workspace` holds workspace_bytes >= lrattn_workspace_size(p) bytes; its
 * contents on entry do not matter and are scratch afterwards.
 */
int lrattn_decode(const lrattn_params* p,
                  const void* q,
                  const void* L_K,
                  const void* L_V,
                  const void* B_K,
                  const void* B_V,
                  const float* scales,
                  const int32_t* seq_lens,
                  void* out,
                  void* workspace,
                  size_t workspace_bytes,
                  lrattn_stream stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * lrattn_decode with no workspace argument.  The partial records (and the
 * absorbed queries, when the plan has them) go to a static device buffer of
 * LRATTN_STATIC_SCRATCH_BYTES (16 MiB), one per
 * device, which the library holds from the first call on a device until the
 * process ends; the call allocates nothing.  Same operation, kernels, plan,
 * results (bitwise equal to lrattn_decode's for the same p) and argument
 * rules as lrattn_decode, plus:
 *   - a request whose lrattn_workspace_size exceeds LRATTN_STATIC_SCRATCH_BYTES
 *     returns LRATTN_ERR_SCRATCH before any device work (the five reference
 *     workloads need at most 8.6 MB: 4 x 40 heads x 256 partitions x r 48,
 *     and the absorbed queries);
 *   - the buffer used is the current device's: `stream` must belong to the
 *     current device (else LRATTN_ERR_UNSUPPORTED);
 *   - every call on one device shares that device's buffer, so calls that
 *     overlap in time on one device (different streams or threads without
 *     ordering) race and give undefined results; calls ordered on one
 *     stream are safe;
 *   - the first call on a device resolves the buffer's address
 *     (hipGetSymbolAddress); make it outside graph capture.
 */
#define LRATTN_STATIC_SCRATCH_BYTES (16u << 20)
int lrattn_decode_static(const lrattn_params* p,
                         const void* q,
                         const void* L_K,
                         const void* L_V,
                         const void* B_K,
                         const void* B_V,
                         const float* scales,
                         const int32_t* seq_lens,
                         void* out,
                         lrattn_stream stream);

/*
 * First half of lrattn_decode alone (for measurement and testing): absorb
 * q . B_K^T (in the partition kernel, or, with at least
 * LRATTN_PRE_ABSORB_SPLITS partitions per head, once per query head in a
 * kernel launched ahead of it), stream the latents, write one partial record
 * per (b, query head, non-empty partition) into the workspace.  Records of
 * partitions that lie past seq_len are not written.  The workspace is
 * lrattn_workspace_size(p) bytes, as for lrattn_decode.
 */
int lrattn_partition(const lrattn_params* p,
                     const void* q,
                     const void* L_K,
                     const void* L_V,
                     const void* B_K,
                     const float* scales,
                     const int32_t* seq_lens,
                     void* workspace,
                     size_t workspace_bytes,
                     lrattn_stream stream);

/*
 * Second half of lrattn_decode alone: merge the partial records left by
 * lrattn_partition (same p, seq_lens and workspace) and project through B_V.
 */
int lrattn_combine(const lrattn_params* p,
                   const void* B_V,
                   const int32_t* seq_lens,
                   void* out,
                   void* workspace,
                   size_t workspace_bytes,
                   lrattn_stream stream);

/*
 * Dense baseline on the same kernels: single-token decode attention over an
 * uncompressed cache, for comparison with the factored cache (the pages
 * measure their kernels against dense Flash Decoding: WSVD section 4,
 * FlashSVD's dense-cache path).  For every b, h with g = h / (Hq / Hkv):
 *   out[b,h,:] = sum_t softmax_t(scale * <q[b,h,:], K[b,g,t,:]>) V[b,g,t,:]
 *   K, V     [B, Hkv, T, d]  latent_dtype (int8 takes `scales` as above)
 * `p` is the same parameter block with rank == head_dim (else
 * LRATTN_ERR_SHAPE); factor_dtype is not used but must be a valid factor
 * code.  Workspace size, plan, alignment, ownership, seq_lens handling,
 * errors and determinism are those of lrattn_decode, with d * sizeof(K) <=
 * 256 bytes (d = 64, or d = 128 with 2- or 1-byte K and V).
 */
int lrattn_dense_decode(const lrattn_params* p,
                        const void* q,
                        const void* K,
                        const void* V,
                        const float* scales,
                        const int32_t* seq_lens,
                        void* out,
                        void* workspace,
                        size_t workspace_bytes,
                        lrattn_stream stream);

/*
 * Rebuilt (and optionally rotated) keys: the decode with K rebuilt on chip
 * before scoring, as the fused kernel of the WSVD page (section 2.C) does,
 * so that a position-dependent rotation can act between the rebuild and the
 * score (the absorbed form q . B_K^T of lrattn_decode cannot carry one).
 * For every b, h with g = h / (Hq / Hkv), n = seq_lens[b], t < n:
 *   K[t] = rot(L_K[b,g,t,:] . B_K[g], t)      V[t] = L_V[b,g,t,:] . B_V[g]
 *   q'   = rot(q[b,h,:], n - 1)               (the query is the last token)
 *   out[b,h,:] = sum_t softmax_t(softmax_scale * <q', K[t]>) V[t]
 * where rot(x, p) turns each pair (x[j], x[j + d/2]), j < d/2, by the angle
 * whose cosine is rope[p, j] and sine rope[p, d/2 + j]:
 *   (a, b) -> (a cos - b sin, a sin + b cos).
 *   rope  [T, d] fp32, T = max_seq_len, 16-byte aligned; NULL: no rotation
 *         (the result then equals lrattn_decode's up to rounding).
 * Values are not rotated.  q, latents and factors must be bf16 (LRATTN_BF16),
 * head_dim in {64, 128}, rank in {32, 64}, group in {1, 2, 4, 8}, and
 * T * d * 4 < 2^31 when rope is given; anything else returns
 * LRATTN_ERR_UNSUPPORTED.  The keys are rebuilt with exact bf16 products and
 * fp32 sums; rotation, scores, softmax and accumulation run in fp32.
 * Plan and workspace are this call's own: one wave streams one sequence's
 * partition (four sequences per workgroup share the rotation table's rows),
 * so by default T is split into more partitions than lrattn_decode uses;
 * lrattn_rebuild_plan reports them (num_splits > 0 is used as given) and the
 * workspace must hold lrattn_rebuild_workspace_size bytes.  Ownership,
 * seq_lens handling, errors and determinism are those of lrattn_decode.
 */
int lrattn_rebuild_plan(const lrattn_params* p, int32_t* num_splits, int32_t* split_tokens);
int lrattn_rebuild_workspace_size(const lrattn_params* p, size_t* bytes);
int lrattn_rebuild_decode(const lrattn_params* p,
                          const void* q,
                          const void* L_K,
                          const void* L_V,
                          const void* B_K,
                          const void* B_V,
                          const float* rope,
                          const int32_t* seq_lens,
                          void* out,
                          void* workspace,
                          size_t workspace_bytes,
                          lrattn_stream stream);

/*
 * Attention-aware rank (AttentionPack page, section 2.B: a moving average of
 * each token's accumulated attention marks the important tokens, which are
 * rebuilt at the full rank; the others are rebuilt at a reduced rank).  The
 * latent coordinates are taken as ordered by importance (leading singular
 * directions first), so rank k keeps coordinates [0, k).  For every b, g and
 * t < n = seq_lens[b], with k_t = r if importance[b, g, t] >= threshold and
 * low_rank otherwise:
 *   K[t] = Lk[t, :k_t] . B_K[g, :k_t, :]     V[t] = Lv[t, :k_t] . B_V[g, :k_t, :]
 *   out[b,h,:] = sum_t p[b,h,t] V[t],  p = softmax_t(softmax_scale * <q[b,h,:], K[t]>)
 * and afterwards, in place, for t < n (other entries untouched):
 *   importance[b, g, t] = decay * importance[b, g, t]
 *                         + (1 - decay) * mean over the query heads h of g of p[b,h,t]
 *   importance [B, Hkv, T] fp32, 16-byte aligned, read and written
 *   low_rank in [1, r]; decay in [0, 1]; threshold not NaN
 * Three launches: the partitions (which also write each token's logits),
 * the combine (which also writes each row's final max and denominator), the
 * update.  The workspace (lrattn_adaptive_workspace_size bytes) holds the
 * records, the logits and the row statistics.  Supported: bf16
 * latents with r in {32, 48, 64, 128} and group in {1, 2, 4, 8}; int8 latents
 * with r = 32 and group 1 or 4; fp32 latents with r = 16 and group 1; and
 * group * T * 4 < 2^31 bytes; else LRATTN_ERR_UNSUPPORTED.  Other tensors,
 * dtypes, seq_lens handling,
 * ownership, errors and determinism as in lrattn_decode.
 */
typedef struct lrattn_adaptive {
  int32_t low_rank;   /* rank of the tokens below the threshold */
  float threshold;    /* importance at or above it: full rank */
  float decay;        /* weight of the old score in the moving average */
} lrattn_adaptive;
int lrattn_adaptive_workspace_size(const lrattn_params* p, const lrattn_adaptive* ad,
                                   size_t* bytes);
/* Host-only.  Name of the partition kernel lrattn_adaptive_decode launches
 * for `p` and `ad`, as profilers list it: "partition_mfma_kernel" (bf16
 * latents, r a multiple of 32, 4 or 8 query heads per kv-head) or
 * "partition_kernel"; static text.  NULL when the call would be rejected. */
const char* lrattn_adaptive_kernel(const lrattn_params* p, const lrattn_adaptive* ad);
int lrattn_adaptive_decode(const lrattn_params* p,
                           const lrattn_adaptive* ad,
                           const void* q,
                           const void* L_K,
                           const void* L_V,
                           const void* B_K,
                           const void* B_V,
                           const float* scales,
                           const int32_t* seq_lens,
                           float* importance,
                           void* out,
                           void* workspace,
                           size_t workspace_bytes,
                           lrattn_stream stream);

/*
 * Separate factors for the image block and the text (AttentionPack page,
 * section 2.A: visual and textual tokens are compressed apart, as their
 * statistics differ).  Every sequence starts with an image block of
 * image_tokens tokens; token t uses factor set 0 when t < image_tokens and
 * set 1 otherwise.  For every b, h with g = h / (Hq / Hkv), n = seq_lens[b]:
 *   K[t] = Lk[t] . B_K[m(t), g]     V[t] = Lv[t] . B_V[m(t), g]     t < n
 *   out[b,h,:] = sum_t softmax_t(softmax_scale * <q[b,h,:], K[t]>) V[t]
 * with m(t) = 0 for t < image_tokens, else 1; Lk, Lv as in lrattn_decode.
 *   B_K, B_V [2, Hkv, r, d]   set 0 (image) then set 1 (text)
 *   image_tokens >= 0 (0: every token uses set 1; >= T: every token set 0)
 * The image tokens and the text are split into partitions apart, so no
 * partition mixes the sets; the combine keeps one latent-space sum per set
 * under the common log-sum-exp and projects each with its own B_V.  Other
 * tensors, dtypes, alignment, seq_lens handling, ownership, errors and
 * determinism as in lrattn_decode; head_dim in {64, 128} and rank <= 64,
 * else LRATTN_ERR_UNSUPPORTED.  The workspace must hold
 * lrattn_modal_workspace_size bytes.
 */
int lrattn_modal_workspace_size(const lrattn_params* p, int32_t image_tokens, size_t* bytes);
int lrattn_modal_decode(const lrattn_params* p,
                        int32_t image_tokens,
                        const void* q,
                        const void* L_K,
                        const void* L_V,
                        const void* B_K,
                        const void* B_V,
                        const float* scales,
                        const int32_t* seq_lens,
                        void* out,
                        void* workspace,
                        size_t workspace_bytes,
                        lrattn_stream stream);

/*
 * Shared latent streams with per-query-head factors (AttentionPack page,
 * section 2.A: the heads' keys and values are factored together, so the
 * cache keeps one compressed row per token shared by the heads, and head h
 * rebuilds with its own block of the decompression matrix).  For every b, h,
 * with stream s = h / (Hq / S) (S = params.num_kv_heads streams; S = 1 is a
 * single cache shared by all heads) and n = seq_lens[b]:
 *   K[t] = Lk[t] . B_K[h]     V[t] = Lv[t] . B_V[h]      t < n
 *   out[b,h,:] = sum_t softmax_t(softmax_scale * <q[b,h,:], K[t]>) V[t]
 * with Lk[t] = L_K[b,s,t,:] (times scales[0,b,s,t] for int8), likewise Lv.
 *   L_K, L_V [B, S, T, r]; scales [2, B, S, T] iff int8
 *   B_K, B_V [Hq, r, d]   one block per query head
 * Other tensors, dtypes, alignment, seq_lens handling, ownership, errors and
 * determinism as in lrattn_decode; supported shapes as there, with the group
 * Hq / S any multiple of 1, 2, 4 or 8.  Three launches: q~ for every head,
 * the partitions, the combine.  With bf16 latents, rank 32, 64 or 128 and
 * Hq / S >= 32, each partition workgroup reads its tile of the stream once
 * for up to 64 heads (scores and value sums on the matrix cores, the
 * weights split into two bf16 terms); otherwise heads run in groups of up to
 * 8 that read the same stream.  The plan (and so the workspace size) depends
 * on which applies; the workspace holds the partial records and q~.
 */
int lrattn_shared_workspace_size(const lrattn_params* p, size_t* bytes);
int lrattn_shared_decode(const lrattn_params* p,
                         const void* q,
                         const void* L_K,
                         const void* L_V,
                         const void* B_K,
                         const void* B_V,
                         const float* scales,
                         const int32_t* seq_lens,
                         void* out,
                         void* workspace,
                         size_t workspace_bytes,
                         lrattn_stream stream);

/*
 * The append step: the new token's latent rows, written into the cache.
 * WSVD page, section 2.A: each head's key (value) projection is factored per
 * head, W_Kh = A_Kh . B_Kh with rank r, so a token with hidden state x enters
 * the cache as its latent x . A_Kh; section 2.C keeps such latents in low
 * precision.  For every sequence b < B and kv-head g, with p = positions[b]:
 *   L_K[b,g,p,j] = sum_i x[b,i] A_K[g,j,i]     (likewise L_V with A_V)
 *   x        [B, D]          x_dtype (BF16 or F16)
 *   A_K, A_V [Hkv, r, D]     factor_dtype == x_dtype; row j holds the D
 *                            weights of latent coordinate j (A_Kh transposed)
 *   positions [B] int32      device; rows with p outside [0, T) are not written
 *   L_K, L_V [B, Hkv, T, r]  latent_dtype (F32, BF16, F16 or I8): rounded to
 *                            nearest even; I8: symmetric, per (b, g, p) and
 *                            K / V: s = max_j |l_j| / 127, code = rint(l_j / s)
 *                            (ties to even; s = 0 gives codes 0), s stored in
 *   scales   [2, B, Hkv, T]  fp32 (index 0: K, 1: V); required iff I8
 * The products are exact and summed in fp32 in a fixed order (bitwise
 * reproducible); the int8 decision is taken in fp32 on those sums.
 * Supported: r in {16, 32, 48, 64, 128}, 1 <= B <= 64, D a multiple of 128;
 * else LRATTN_ERR_UNSUPPORTED.  All pointers 16-byte aligned.  Only the
 * addressed rows (and scales) are written.  On `stream`: float latents with
 * Hkv * 2 * r / 16 >= 192 take one launch (each workgroup sums all of D for
 * 16 latent coordinates; the workspace is not touched); otherwise, and for
 * I8 latents, two launches (partial sums over chunks of D into the caller's
 * workspace, then the rows and scales).  No allocation, no host
 * synchronization; workspace contents on entry do not matter.
 */
typedef struct lrattn_append_params {
  int32_t batch;        /* B: sequences, one new token each */
  int32_t num_kv_heads; /* Hkv */
  int32_t model_dim;    /* D: width of x */
  int32_t rank;         /* r */
  int32_t max_seq_len;  /* T: token capacity (stride) of the cache */
  int32_t x_dtype;      /* lrattn_dtype of x (and of A_K, A_V) */
  int32_t factor_dtype; /* lrattn_dtype of A_K, A_V: equal to x_dtype */
  int32_t latent_dtype; /* lrattn_dtype of the cache */
} lrattn_append_params;

/* Host-only.  Bytes of workspace lrattn_append needs for `p` (partial rows,
 * fp32, a few MB at most). */
int lrattn_append_workspace_size(const lrattn_append_params* p, size_t* bytes);

int lrattn_append(const lrattn_append_params* p,
                  const void* x,
                  const void* A_K,
                  const void* A_V,
                  const int32_t* positions,
                  void* L_K,
                  void* L_V,
                  float* scales,
                  void* workspace,
                  size_t workspace_bytes,
                  lrattn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* LRATTN_H */
