/*
 * dsa.h - C ABI of the DeepSeek-Sparse-Attention (DSA) step on AMD gfx950.
 *
 * One DSA step of one MLA layer has three stages, each an entry point here:
 *
 *   dsa_indexer_logits  lightning-indexer scores over a paged fp8 index-K cache
 *   dsa_topk            per-row top-k of those scores with causal/length masking
 *   dsa_indexer_topk    both in one call, without the scores in memory
 *   sparse_mla_decode   sparse MLA attention over the selected latent rows
 *   sparse_mla_prefill  (decode: one query row per request; prefill: many)
 *
 * and two for the indexer's inputs, the step before the scores:
 *
 *   dsa_quant_index_q   fp8 index queries, per-head scale folded into the gates
 *   dsa_store_index_k   fp8 quantization of new index keys + their paged store
 *
 * and the attention over an fp8 latent cache:
 *
 *   sparse_mla_decode_fp8, sparse_mla_prefill_fp8
 *
 * Sources: the SGLang "dsa_indexer.py" page (Indexer._get_topk_paged calls the
 * paged fp8 MQA-logits kernel with q_fp8 [T,H,128], the 132-byte-per-token
 * index cache, weights [T,H], seqlens and block tables, then topk_transform),
 * the Ascend "sfa_v1.py" page (npu_lightning_indexer / npu_sparse_flash_attention
 * take TND queries, a paged PA_BSND cache, block_table, cumulative query
 * lengths and key lengths, sparse_count=2048, sparse_mode=3 i.e. causal), and
 * the vLLM "mla/common.py" page (decode returns (out, lse); LSE merge of
 * partial results with merge_attn_states).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the comment says "host". The dsa_batch_t
 *   struct itself is read on the host during the call and may be freed after it.
 * - Every call is asynchronous on `stream` (a hipStream_t; 0 = the null
 *   stream), never synchronizes the host, allocates no memory, keeps no state
 *   between calls and is safe to call from several threads (except
 *   sparse_mla_decode_noalloc, which keeps its partials in a static per-GPU
 *   array: see there). Calls contain no host-device synchronization and no
 *   memset nodes, so they can be captured into a HIP graph.
 * - The caller owns every buffer. Inputs are read-only; outputs must not alias
 *   inputs.
 * - Arguments are validated on the host before anything is launched. On error
 *   nothing is launched and a dsa_status_t other than DSA_OK is returned;
 *   dsa_last_error() then gives a thread-local description.
 * - Device-side contents (block-table entries, lengths, top-k indices) are
 *   not validated on the host, but the kernels never read outside the buffers
 *   the shapes describe: a page id outside [0, num_pages) or a position outside
 *   the request's length is treated as absent (logit -inf, attention entry
 *   skipped).
 *
 * Batch and causality
 * -------------------
 * Request b owns `seq_lens_k[b]` keys at logical positions [0, seq_lens_k[b]);
 * position p lives in physical page block_table[b * max_pages_per_seq + p / P],
 * slot p % P (both caches share page ids). Query rows are laid out "TND":
 * with cu_seqlens_q == NULL there is one row per request (decode, row t =
 * request t); otherwise request b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.
 * Causality is bottom-right aligned (sparse_mode=3): the j-th of q_len_b rows
 * of request b sees visible = seq_lens_k[b] - q_len_b + j + 1 keys, positions
 * [0, visible). In decode every row sees its whole request.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *dsa_stream_t; /* identical to hipStream_t */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride or count */
  DSA_ERR_UNSUPPORTED = 2,      /* valid, but a shape/dtype this build has no kernel for */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4               /* the HIP runtime reported an error at launch */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2 /* OCP E4M3 ("fn": no infinities, 0x7F/0xFF NaN, max 448) */
} dsa_dtype_t;

typedef enum {
  DSA_OP_TOPK = 0,
  DSA_OP_MLA_DECODE = 1,
  DSA_OP_MLA_PREFILL = 2,
  DSA_OP_INDEXER_TOPK = 3
} dsa_op_t;

typedef struct {
  int32_t num_seqs;          /* B >= 0 */
  int32_t num_rows;          /* T: query rows; must equal B when cu_seqlens_q == NULL */
  int32_t page_size;         /* P: tokens per page, a positive multiple of 16 */
  int32_t max_pages_per_seq; /* row stride of block_table, >= 1 */
  int32_t num_pages;         /* pages in each cache pool; page ids outside [0, num_pages) are absent */
  int32_t max_seq_len_k;     /* host: >= every seq_lens_k[b], at most 2^24; sizes grids, never read back */
  int32_t max_seq_len_q;     /* host: >= every q_len_b (1 for decode) */
  const int32_t *block_table;  /* [B, max_pages_per_seq] physical page ids */
  const int32_t *seq_lens_k;   /* [B] keys in the cache, this step's tokens included */
  const int32_t *cu_seqlens_q; /* [B+1] row prefix sums (cu[0] = 0, cu[B] = T), or NULL */
} dsa_batch_t;

/*
 * dsa_indexer_logits - lightning-indexer scores (SGLang page,
 * Indexer._get_topk_paged / forward_indexer):
 *
 *   logits[t, s] = sum_h w[t,h] * relu(sigma_s * (q[t,h,:] . k_s[:]))   for s < visible(t)
 *
 * q:        [T, H, D], q_dtype FP8_E4M3 with H = 64, D = 128, or F32 with
 *           H <= 64, D <= 128 (any H, D in that range).
 * w:        [T, H] fp32 head gates with the query's quantization scale (and any
 *           head or softmax scale) already folded in.
 * index_cache: paged keys. Page i starts at byte i * (P*D*esize + 4*P): P*D key
 *           elements of k_dtype (token-major, D per token), then P fp32 scales
 *           sigma. With P = 64, D = 128 and fp8 keys this is the 132 bytes per
 *           token of the pages. k_dtype must equal q_dtype. sigma must be >= 0
 *           (absmax-derived scales are); the kernel applies it after the head sum,
 *           which equals the formula for sigma >= 0.
 * logits:   [T, logits_row_stride] fp32, logits_row_stride >= max visible.
 *           Columns >= visible(t) are left unwritten (the pages call their kernels
 *           with clean_logits=False); a position whose page is absent gets -inf.
 * num_init_tokens, num_local_tokens >= 0: init/local-token forcing (SGLang page,
 *           Indexer._mask_init_and_local_tokens): the positions s < num_init_tokens
 *           and s >= visible(t) - num_local_tokens of each row (s < visible(t))
 *           get +inf, so that dsa_topk always selects them (ties at +inf go to
 *           the lower positions). 0 and 0 turn it off.
 * With FP8_E4M3, q, w and index_cache must be 16-byte aligned
 * (DSA_ERR_INVALID_ARGUMENT otherwise).
 */
dsa_status_t dsa_indexer_logits(const dsa_batch_t *batch,
                                const void *q, dsa_dtype_t q_dtype,
                                const float *w,
                                const void *index_cache, dsa_dtype_t k_dtype,
                                int32_t num_heads, int32_t head_dim,
                                float *logits, int64_t logits_row_stride,
                                int32_t num_init_tokens, int32_t num_local_tokens,
                                dsa_stream_t stream);

/*
 * dsa_quant_index_q - fp8 index queries and their head gates, the input side
 * of dsa_indexer_logits (SGLang page, Indexer.forward_cuda: act_quant of the
 * bf16 query into (q_fp8, q_scale); _get_logits_head_gate: gates times q_scale).
 * For each row t and head h, over the head's D = 128 elements:
 *
 *   s[t,h]     = max(max_d |q[t,h,d]|, 1e-30) / 448                 (fp32)
 *   q8[t,h,d]  = E4M3FN(q[t,h,d] / s[t,h])   fp32 quotient, nearest, ties to even
 *   w_eff[t,h] = w[t,h] * s[t,h]                                    (fp32)
 *
 * (act_quant is not on the pages; this is the reading with one fp32 scale per
 * 128-wide block.) A magnitude that rounds past 448 becomes NaN (E4M3FN has no
 * infinity); with these scales finite inputs never do. A block holding NaN
 * gets a NaN scale and NaN codes (their sign bit unspecified).
 *
 * q:     [T, H, 128] bf16, 16-byte aligned.   w: [T, H] fp32 (the n_heads^-0.5
 *        and softmax factors already applied).
 * q8:    [T, H, 128] E4M3FN codes, 8-byte aligned.   w_eff: [T, H] fp32; may be w.
 * num_rows = T >= 0, 1 <= num_heads, head_dim must be 128.
 */
dsa_status_t dsa_quant_index_q(const void *q, const float *w, int32_t num_rows, int32_t num_heads,
                               int32_t head_dim, void *q8, float *w_eff, dsa_stream_t stream);

/*
 * dsa_store_index_k - fp8 quantization of a step's new index keys and their
 * paged store (SGLang page, Indexer._store_index_k_cache: act_quant(key) and
 * set_index_k_scale_buffer at out_cache_loc). Key i gets the block scale and
 * codes of dsa_quant_index_q (sigma_i and k8[i, :]) and is written at slot
 * s = slot_mapping[i], i.e. page s / P, position s % P of index_cache: its 128
 * codes at byte 128 * (s % P) of the page, sigma_i at byte 128 * P + 4 * (s % P)
 * (the fp8 layout dsa_indexer_logits reads). Negative slots and slots
 * >= num_pages * P are skipped (padding tokens). Slots must be distinct.
 *
 * key: [N, 128] bf16, 16-byte aligned.   slot_mapping: [N] int64.
 * index_cache: [num_pages, 132 * P] bytes, 16-byte aligned; P a positive
 *              multiple of 16.   num_tokens = N >= 0, head_dim must be 128.
 */
dsa_status_t dsa_store_index_k(const void *key, int32_t num_tokens, int32_t head_dim,
                               const int64_t *slot_mapping, int32_t page_size, int32_t num_pages,
                               void *index_cache, dsa_stream_t stream);

/*
 * dsa_topk - per-row top-k selection (SGLang page: topk_transform after the
 * logits; forward_indexer takes topk(min(topk, seq_len)) and pads with -1;
 * _forward_cuda_k_only relies on rows of length <= k giving [0 .. len-1, -1 ...]).
 *
 * For each row t, with n = min(visible(t), logits_row_stride):
 *   n <= k: topk_idx[t] = 0, 1, ..., n-1, then -1.
 *   n >  k: the k positions s < n with the largest logits[t, s], in ascending
 *           position order; among equal values at the k-th place the lower
 *           positions are taken. Values are compared as floats with -0 == +0;
 *           logits must not be NaN.
 * topk_idx: [T, k] int32 logical positions. 1 <= k <= 4096.
 * workspace: at least dsa_workspace_bytes(DSA_OP_TOPK, ...) bytes of device
 *           memory, else DSA_ERR_WORKSPACE_TOO_SMALL. It is non-zero for batches
 *           of few, long rows, which are selected in two phases (per chunk of
 *           the row, then among the chunks' candidates); NULL if it is 0.
 */
dsa_status_t dsa_topk(const dsa_batch_t *batch,
                      const float *logits, int64_t logits_row_stride, int32_t k,
                      int32_t *topk_idx,
                      void *workspace, size_t workspace_bytes,
                      dsa_stream_t stream);

/*
 * dsa_indexer_topk - the lightning-indexer scores and their per-row top-k in
 * one call, with no [rows x keys] score matrix in memory (SGLang page:
 * Indexer._get_topk_ragged materialises the scores of a batch, in row chunks
 * when _should_chunk_mqa_logits finds them too large, and hands them to
 * topk_transform; this call gives the same top-k lists without them).
 *
 * topk_idx[t] is what dsa_topk(k) writes for the scores that
 * dsa_indexer_logits(FP8_E4M3, num_init_tokens, num_local_tokens) computes
 * for the same inputs: the fp8 contraction and its summation order are those
 * of the decode-row scores, so for decode and multi-token decode rows the two
 * paths give identical lists; init/local forcing and absent pages (-inf) as
 * there. Rows with visible(t) <= k get 0 .. visible(t) - 1, then -1, without
 * being scored.
 *
 * q, w, index_cache: as dsa_indexer_logits with FP8_E4M3 keys and queries
 *           (64 heads x 128 only, else DSA_ERR_UNSUPPORTED; 16-byte aligned).
 * topk_idx: [T, k] int32, 1 <= k <= 4096.
 * workspace: at least dsa_workspace_bytes(DSA_OP_INDEXER_TOPK, ...) bytes of
 *           device memory (each row's chunks hand their k best (key, position)
 *           pairs to a merge: 8 bytes x k per started chunk of up to 8192 keys).
 */
dsa_status_t dsa_indexer_topk(const dsa_batch_t *batch,
                              const void *q, const float *w, const void *index_cache,
                              int32_t num_heads, int32_t head_dim,
                              int32_t num_init_tokens, int32_t num_local_tokens,
                              int32_t k, int32_t *topk_idx,
                              void *workspace, size_t workspace_bytes,
                              dsa_stream_t stream);

/*
 * sparse_mla_decode / sparse_mla_prefill - sparse MLA attention over the
 * selected latent rows (Ascend SFA page, npu_sparse_flash_attention with
 * key = value = latent cache, the rope key passed separately, token-granular
 * sparse indices and sparse_mode=3; vLLM MLA page: the decode path returns
 * (attn_out, lse), and the cached row is the 512-d latent followed by the 64-d
 * rope key). For each row t and head h, over the valid entries i of topk_idx[t]
 * (entries < 0 or >= seq_lens_k[b] are skipped, so are absent pages):
 *
 *   C_i   = kv_cache row of position topk_idx[t, i]   (d_latent + d_rope values)
 *   z_i   = softmax_scale * (q[t,h,:] . C_i)
 *   out[t,h,:] = sum_i softmax(z)_i * C_i[:d_latent]
 *   lse[t,h]   = log(sum_i exp(z_i))                  (natural log)
 *
 * A row with no valid entry gets out = 0 and lse = -inf. Duplicate entries are
 * counted as many times as they appear. Entries should lie below the row's
 * visible length; the call does not enforce causality itself.
 *
 * q:        [T, Hm, d_latent + d_rope] (absorbed no-rope part, then rope part)
 * kv_cache: [num_pages, P, d_latent + d_rope]
 * dtype:    BF16 with (Hm, d_latent, d_rope) = (128, 512, 64) or any Hm that is
 *           a multiple of 64 with those dims; or F32 with Hm <= 128,
 *           d_latent + d_rope <= 1024, d_latent <= 512. (An fp8 cache goes
 *           through sparse_mla_*_fp8; FP8_E4M3 here is UNSUPPORTED.)
 * topk_idx: [T, k] int32, 1 <= k <= 4096.
 * softmax_scale: any finite value whose product with log2(e) is finite
 *           (DSA_ERR_INVALID_ARGUMENT otherwise); zero gives uniform weights.
 * out:      [T, Hm, d_latent] in dtype.   lse: [T, Hm] fp32, may be NULL.
 * workspace: at least dsa_workspace_bytes(DSA_OP_MLA_DECODE or _PREFILL, ...)
 *           bytes of device memory (split-KV partial results); NULL if that is 0.
 * With BF16, q, kv_cache, out and a non-empty workspace must be 16-byte
 * aligned (DSA_ERR_INVALID_ARGUMENT otherwise).
 *
 * sparse_mla_decode requires cu_seqlens_q == NULL (one row per request);
 * sparse_mla_prefill requires cu_seqlens_q != NULL.
 */
dsa_status_t sparse_mla_decode(const dsa_batch_t *batch,
                               const void *q, const void *kv_cache, dsa_dtype_t dtype,
                               const int32_t *topk_idx, int32_t k,
                               int32_t num_heads, int32_t d_latent, int32_t d_rope,
                               float softmax_scale,
                               void *out, float *lse,
                               void *workspace, size_t workspace_bytes,
                               dsa_stream_t stream);

dsa_status_t sparse_mla_prefill(const dsa_batch_t *batch,
                                const void *q, const void *kv_cache, dsa_dtype_t dtype,
                                const int32_t *topk_idx, int32_t k,
                                int32_t num_heads, int32_t d_latent, int32_t d_rope,
                                float softmax_scale,
                                void *out, float *lse,
                                void *workspace, size_t workspace_bytes,
                                dsa_stream_t stream);

/*
 * sparse_mla_decode_fp8 / sparse_mla_prefill_fp8 - the same attention over an
 * fp8 latent cache (vLLM MLA page, the decode path under fp8_attention: the
 * absorbed query and its rope part quantized with the layer's q scale by
 * scaled_fp8_quant, the cache written in fp8 with the layer's k scale). q and
 * kv_cache hold OCP E4M3 codes, one scale per tensor:
 *
 *   z_i        = softmax_scale * q_scale * kv_scale * (q8[t,h,:] . C8_i)
 *   out[t,h,:] = kv_scale * sum_i softmax(z)_i * C8_i[:512]
 *   lse[t,h]   = log(sum_i exp(z_i))                  (natural log)
 *
 * with the entry rules of sparse_mla_decode (invalid entries skipped, empty
 * selection -> out 0 and lse -inf).
 * q:        [T, Hm, 576] codes (512 latent, then 64 rope), 16-byte aligned rows.
 * kv_cache: [num_pages, P, 576] codes (576 bytes per cached row).
 * Hm a multiple of 64, d_latent 512, d_rope 64; q_scale, kv_scale finite, > 0;
 * softmax_scale * q_scale * kv_scale * log2(e) finite.
 * out:      [T, Hm, 512] bf16.   lse: [T, Hm] fp32, may be NULL.
 * workspace: at least dsa_workspace_bytes(DSA_OP_MLA_DECODE or _PREFILL, ...,
 *           DSA_FP8_E4M3) bytes (split partials; always at least two splits
 *           when k > 1024); NULL if that is 0.
 * q, kv_cache, out and the workspace must be 16-byte aligned
 * (DSA_ERR_INVALID_ARGUMENT otherwise).
 */
dsa_status_t sparse_mla_decode_fp8(const dsa_batch_t *batch,
                                   const void *q, float q_scale,
                                   const void *kv_cache, float kv_scale,
                                   const int32_t *topk_idx, int32_t k,
                                   int32_t num_heads, int32_t d_latent, int32_t d_rope,
                                   float softmax_scale,
                                   void *out, float *lse,
                                   void *workspace, size_t workspace_bytes,
                                   dsa_stream_t stream);

dsa_status_t sparse_mla_prefill_fp8(const dsa_batch_t *batch,
                                    const void *q, float q_scale,
                                    const void *kv_cache, float kv_scale,
                                    const int32_t *topk_idx, int32_t k,
                                    int32_t num_heads, int32_t d_latent, int32_t d_rope,
                                    float softmax_scale,
                                    void *out, float *lse,
                                    void *workspace, size_t workspace_bytes,
                                    dsa_stream_t stream);

/*
 * sparse_mla_decode_noalloc - sparse_mla_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same attention, arguments and entry
 * rules as sparse_mla_decode, without the workspace arguments. The split-KV
 * partials go to a static device array of the library, 32 MiB per GPU, which
 * each GPU the library runs on holds until the process ends. The call itself
 * allocates nothing.
 *
 * A batch whose partials need more than 32 MiB (dsa_workspace_bytes(
 * DSA_OP_MLA_DECODE, ...) > 33554432, e.g. k > 2048 over very many rows)
 * returns DSA_ERR_UNSUPPORTED before anything is launched; use
 * sparse_mla_decode with a workspace then. Every call on one GPU shares that
 * GPU's array and leaves its partials in it: calls that may overlap on one GPU
 * (on different streams, or from several threads without ordering) race and
 * must be serialized by the caller. The array is looked up for the current
 * device (hipGetDevice), which must be the device of `stream`.
 */
dsa_status_t sparse_mla_decode_noalloc(const dsa_batch_t *batch,
                                       const void *q, const void *kv_cache, dsa_dtype_t dtype,
                                       const int32_t *topk_idx, int32_t k,
                                       int32_t num_heads, int32_t d_latent, int32_t d_rope,
                                       float softmax_scale,
                                       void *out, float *lse,
                                       dsa_stream_t stream);

/*
 * dsa_workspace_bytes - device workspace an op needs for this batch (host-only,
 * launches nothing). Returns 0 for an op that needs none, and (size_t)-1 when
 * the arguments are invalid (dsa_last_error() says why). `num_heads` and
 * `d_latent` are the MLA ones; they are ignored for DSA_OP_TOPK and
 * DSA_OP_INDEXER_TOPK. `dtype` is the
 * MLA dtype (DSA_FP8_E4M3 for the sparse_mla_*_fp8 calls).
 */
size_t dsa_workspace_bytes(dsa_op_t op, const dsa_batch_t *batch, int32_t k,
                           int32_t num_heads, int32_t d_latent, dsa_dtype_t dtype);

/* Static description of a status code. Never NULL. */
const char *dsa_status_string(dsa_status_t status);

/* Thread-local text of the last non-OK status returned on this thread ("" if none). */
const char *dsa_last_error(void);

/* Library version, "major.minor.patch". */
const char *dsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
