// C ABI of the DSA step: argument validation, dispatch to the kernel launchers,
// workspace sizing and error reporting. Validation runs entirely on the host
// before any HIP call, so invalid calls return without touching a device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "dsa.h"
#include "dsa_internal.h"

using namespace dsa;

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status_t ok() { return DSA_OK; }

dsa_status_t from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks shared by every entry point; fills `bv` on success.
bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

dsa_status_t check_batch(const dsa_batch_t* batch, BatchView* bv) {
  if (!batch) return fail(DSA_ERR_INVALID_ARGUMENT, "batch is NULL");
  const dsa_batch_t& b = *batch;
  if (b.num_seqs < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", b.num_seqs);
  if (b.num_rows < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows %d < 0", b.num_rows);
  if (b.page_size <= 0 || b.page_size % 16 != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "page_size %d is not a positive multiple of 16", b.page_size);
  if (b.max_pages_per_seq < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "max_pages_per_seq %d < 1", b.max_pages_per_seq);
  if (b.num_pages < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "num_pages %d < 1", b.num_pages);
  if ((int64_t)b.num_pages * b.page_size > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "num_pages * page_size exceeds 2^31 - 1 cache rows");
  if ((int64_t)b.max_pages_per_seq * b.page_size > INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "max_pages_per_seq * page_size exceeds 2^31 - 1 positions");
  if (b.max_seq_len_k < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "max_seq_len_k %d < 0", b.max_seq_len_k);
  // 2^24 keys per row keeps every key and group count of a launch (up to 1024
  // rows in one stream launch) and every grid dimension inside 32 bits
  if (b.max_seq_len_k > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED, "max_seq_len_k %d exceeds 2^24", b.max_seq_len_k);
  if (b.max_seq_len_q < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "max_seq_len_q %d < 0", b.max_seq_len_q);
  if (b.num_seqs > 0 && (!b.block_table || !b.seq_lens_k))
    return fail(DSA_ERR_INVALID_ARGUMENT, "block_table / seq_lens_k is NULL");
  if (b.cu_seqlens_q == nullptr) {
    if (b.num_rows != b.num_seqs)
      return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows %d != num_seqs %d with cu_seqlens_q == NULL",
                  b.num_rows, b.num_seqs);
    if (b.num_rows > 0 && b.max_seq_len_q > 1)
      return fail(DSA_ERR_INVALID_ARGUMENT, "max_seq_len_q %d > 1 with cu_seqlens_q == NULL", b.max_seq_len_q);
  } else {
    if (b.num_seqs < 1 && b.num_rows > 0)
      return fail(DSA_ERR_INVALID_ARGUMENT, "rows without requests");
    if (b.num_rows > 0 && b.max_seq_len_q < 1)
      return fail(DSA_ERR_INVALID_ARGUMENT, "max_seq_len_q %d < 1 with rows present", b.max_seq_len_q);
  }
  bv->num_seqs = b.num_seqs;
  bv->num_rows = b.num_rows;
  bv->page_size = b.page_size;
  bv->max_pages_per_seq = b.max_pages_per_seq;
  bv->num_pages = b.num_pages;
  bv->max_seq_len_k = b.max_seq_len_k;
  bv->max_seq_len_q = b.max_seq_len_q;
  bv->block_table = b.block_table;
  bv->seq_lens_k = b.seq_lens_k;
  bv->cu_seqlens_q = b.cu_seqlens_q;
  return ok();
}

struct MlaPlan {
  bool bf16;
  bool fp8;
  int splits;
  int entries_per_split;
  size_t workspace;
};

dsa_status_t plan_mla(const BatchView& bv, int32_t k, int32_t num_heads, int32_t d_latent,
                      int32_t d_rope, dsa_dtype_t dtype, MlaPlan* plan) {
  if (k < 1 || k > kTopkMaxK) return fail(DSA_ERR_INVALID_ARGUMENT, "k %d outside [1, %d]", k, kTopkMaxK);
  if (num_heads < 1 || d_latent < 1 || d_rope < 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "num_heads %d, d_latent %d, d_rope %d", num_heads, d_latent, d_rope);
  plan->fp8 = false;
  if (dtype == DSA_BF16 || dtype == DSA_FP8_E4M3) {
    if (d_latent != kMlaDl || d_rope != kMlaDr || num_heads % kMlaHeadsPerGroup != 0)
      return fail(DSA_ERR_UNSUPPORTED,
                  "%s sparse MLA needs d_latent 512, d_rope 64 and a multiple of 64 heads "
                  "(got %d, %d, %d)", dtype == DSA_BF16 ? "bf16" : "fp8", d_latent, d_rope, num_heads);
    plan->bf16 = dtype == DSA_BF16;
    plan->fp8 = dtype == DSA_FP8_E4M3;
    plan->splits = plan->fp8 ? mla_fp8_splits(bv.num_rows, k, num_heads)
                             : mla_bf16_splits(bv.num_rows, k, num_heads);
    plan->entries_per_split = mla_entries_per_split(k, plan->splits);
    plan->workspace = 0;
    if (plan->splits > 1) {
      const size_t parts = (size_t)bv.num_rows * plan->splits * num_heads;
      // partial outputs in bf16, then their fp32 log-sum-exps
      plan->workspace = parts * (size_t)d_latent * sizeof(uint16_t) + parts * sizeof(float);
    }
    return ok();
  }
  if (dtype == DSA_F32) {
    plan->fp8 = false;
    if (num_heads > 128 || d_latent > 512 || d_latent + d_rope > 1024)
      return fail(DSA_ERR_UNSUPPORTED, "f32 sparse MLA supports num_heads <= 128, d_latent <= 512, "
                  "d_latent + d_rope <= 1024 (got %d, %d, %d)", num_heads, d_latent, d_rope);
    plan->bf16 = false;
    plan->splits = 1;
    plan->entries_per_split = k;
    plan->workspace = 0;
    return ok();
  }
  return fail(DSA_ERR_UNSUPPORTED, "sparse MLA dtype %d (BF16 or F32 only)", (int)dtype);
}

dsa_status_t run_mla(const dsa_batch_t* batch, bool decode, const void* q, const void* kv_cache,
                     dsa_dtype_t dtype, const int32_t* topk_idx, int32_t k, int32_t num_heads,
                     int32_t d_latent, int32_t d_rope, float softmax_scale, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, dsa_stream_t stream,
                     float q_scale = 1.f, float kv_scale = 1.f) {
  BatchView bv;
  dsa_status_t st = check_batch(batch, &bv);
  if (st != DSA_OK) return st;
  if (decode && bv.cu_seqlens_q != nullptr)
    return fail(DSA_ERR_INVALID_ARGUMENT, "sparse_mla_decode needs cu_seqlens_q == NULL");
  if (!decode && bv.cu_seqlens_q == nullptr)
    return fail(DSA_ERR_INVALID_ARGUMENT, "sparse_mla_prefill needs cu_seqlens_q");
  MlaPlan plan;
  st = plan_mla(bv, k, num_heads, d_latent, d_rope, dtype, &plan);
  if (st != DSA_OK) return st;
  if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY || softmax_scale == -INFINITY)
    return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if (!(q_scale > 0.f && q_scale < INFINITY && kv_scale > 0.f && kv_scale < INFINITY))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q_scale / kv_scale must be finite and positive");
  {
    // the kernels work in base 2 with the scale times log2(e) (times the fp8
    // scales), multiplied in this order in fp32: it must stay finite
    const volatile float log2e = 1.4426950408889634f;
    const float s2 = plan.fp8 ? softmax_scale * q_scale * kv_scale * log2e : softmax_scale * log2e;
    if (!(s2 > -INFINITY && s2 < INFINITY))
      return fail(DSA_ERR_INVALID_ARGUMENT, "softmax_scale overflows in base 2 (times log2(e)%s)",
                  plan.fp8 ? " and the fp8 scales" : "");
  }
  if (bv.num_rows > 0 && (!q || !kv_cache || !topk_idx || !out))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q / kv_cache / topk_idx / out is NULL");
  if (workspace_bytes < plan.workspace)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, plan.workspace);
  if (plan.workspace > 0 && !workspace)
    return fail(DSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if ((plan.bf16 || plan.fp8) && bv.num_rows > 0 &&
      !(aligned16(q) && aligned16(kv_cache) && aligned16(out) && (plan.workspace == 0 || aligned16(workspace))))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q, kv_cache, out and workspace must be 16-byte aligned");
  if (bv.num_rows == 0) return ok();

  MlaParams p;
  p.batch = bv;
  p.q = q;
  p.kv = kv_cache;
  p.topk_idx = topk_idx;
  p.k = k;
  p.heads = num_heads;
  p.d_latent = d_latent;
  p.d_rope = d_rope;
  p.softmax_scale = softmax_scale;
  p.q_scale = q_scale;
  p.kv_scale = kv_scale;
  p.out = out;
  p.lse = lse;
  p.splits = plan.splits;
  p.entries_per_split = plan.entries_per_split;
  p.part_o = nullptr;
  p.part_lse = nullptr;
  if (plan.splits > 1) {
    const size_t parts = (size_t)bv.num_rows * plan.splits * num_heads;
    p.part_o = static_cast<uint16_t*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<uint16_t*>(workspace) + parts * (size_t)d_latent);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(plan.fp8 ? launch_mla_fp8(p, s) : plan.bf16 ? launch_mla_bf16(p, s) : launch_mla_f32(p, s),
                  "sparse MLA launch");
}

}  // namespace

dsa_status_t dsa::set_error(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

extern "C" {

dsa_status_t dsa_indexer_logits(const dsa_batch_t* batch, const void* q, dsa_dtype_t q_dtype,
                                const float* w, const void* index_cache, dsa_dtype_t k_dtype,
                                int32_t num_heads, int32_t head_dim, float* logits,
                                int64_t logits_row_stride, int32_t num_init_tokens, int32_t num_local_tokens,
                                dsa_stream_t stream) {
  BatchView bv;
  dsa_status_t st = check_batch(batch, &bv);
  if (st != DSA_OK) return st;
  if (q_dtype != k_dtype)
    return fail(DSA_ERR_UNSUPPORTED, "q_dtype %d != k_dtype %d", (int)q_dtype, (int)k_dtype);
  if (num_heads < 1 || head_dim < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "num_heads %d / head_dim %d < 1", num_heads, head_dim);
  if (q_dtype == DSA_FP8_E4M3) {
    if (num_heads != kIdxHeads || head_dim != kIdxDim)
      return fail(DSA_ERR_UNSUPPORTED, "fp8 indexer needs 64 heads x 128 (got %d x %d)", num_heads, head_dim);
  } else if (q_dtype == DSA_F32) {
    if (num_heads > kIdxHeads || head_dim > kIdxDim)
      return fail(DSA_ERR_UNSUPPORTED, "f32 indexer supports up to 64 heads x 128 (got %d x %d)",
                  num_heads, head_dim);
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype %d (FP8_E4M3 or F32 only)", (int)q_dtype);
  }
  if (logits_row_stride < (int64_t)bv.max_seq_len_k || logits_row_stride < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "logits_row_stride %lld < max_seq_len_k %d",
                (long long)logits_row_stride, bv.max_seq_len_k);
  if (bv.num_rows > 0 && (!q || !w || !index_cache || !logits))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q / w / index_cache / logits is NULL");
  if (num_init_tokens < 0 || num_local_tokens < 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "num_init_tokens %d / num_local_tokens %d < 0", num_init_tokens,
                num_local_tokens);
  if (q_dtype == DSA_FP8_E4M3 && bv.num_rows > 0 && !(aligned16(q) && aligned16(w) && aligned16(index_cache)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q, w and index_cache must be 16-byte aligned");
  if (bv.num_rows == 0 || bv.max_seq_len_k == 0) return ok();
  IndexerParams p;
  p.batch = bv;
  p.q = q;
  p.w = w;
  p.cache = static_cast<const uint8_t*>(index_cache);
  const int64_t esize = q_dtype == DSA_FP8_E4M3 ? 1 : 4;
  p.page_bytes = (int64_t)bv.page_size * head_dim * esize + 4LL * bv.page_size;
  p.heads = num_heads;
  p.dim = head_dim;
  p.logits = logits;
  p.stride = logits_row_stride;
  p.num_init = num_init_tokens;
  p.num_local = num_local_tokens;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = from_hip(q_dtype == DSA_FP8_E4M3 ? launch_indexer_fp8(p, s) : launch_indexer_f32(p, s), "indexer launch");
  if (st != DSA_OK) return st;
  return from_hip(launch_indexer_force(p, s), "indexer forcing launch");
}

dsa_status_t dsa_quant_index_q(const void* q, const float* w, int32_t num_rows, int32_t num_heads,
                               int32_t head_dim, void* q8, float* w_eff, dsa_stream_t stream) {
  if (num_rows < 0 || num_heads < 1)
    return fail(DSA_ERR_INVALID_ARGUMENT, "num_rows %d < 0 or num_heads %d < 1", num_rows, num_heads);
  if (head_dim != kIdxDim) return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (128 only)", head_dim);
  if (num_rows == 0) return ok();
  if (!q || !w || !q8 || !w_eff) return fail(DSA_ERR_INVALID_ARGUMENT, "q / w / q8 / w_eff is NULL");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0 || reinterpret_cast<uintptr_t>(q8) % 8 != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "q must be 16-byte and q8 8-byte aligned");
  QuantQParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.w = w;
  p.q8 = static_cast<uint8_t*>(q8);
  p.w_eff = w_eff;
  p.rows = (int64_t)num_rows * num_heads;
  return from_hip(launch_quant_index_q(p, reinterpret_cast<hipStream_t>(stream)), "q quantization launch");
}

dsa_status_t dsa_store_index_k(const void* key, int32_t num_tokens, int32_t head_dim,
                               const int64_t* slot_mapping, int32_t page_size, int32_t num_pages,
                               void* index_cache, dsa_stream_t stream) {
  if (num_tokens < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "num_tokens %d < 0", num_tokens);
  if (head_dim != kIdxDim) return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (128 only)", head_dim);
  if (page_size < 16 || page_size % 16 != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "page_size %d is not a positive multiple of 16", page_size);
  if (num_pages < 0) return fail(DSA_ERR_INVALID_ARGUMENT, "num_pages %d < 0", num_pages);
  if (num_tokens == 0) return ok();
  if (!key || !slot_mapping || !index_cache)
    return fail(DSA_ERR_INVALID_ARGUMENT, "key / slot_mapping / index_cache is NULL");
  if (reinterpret_cast<uintptr_t>(key) % 16 != 0 || reinterpret_cast<uintptr_t>(index_cache) % 16 != 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "key and index_cache must be 16-byte aligned");
  StoreKParams p;
  p.key = static_cast<const uint16_t*>(key);
  p.slot_mapping = slot_mapping;
  p.cache = static_cast<uint8_t*>(index_cache);
  p.num_tokens = num_tokens;
  p.page_bytes = (int64_t)page_size * (kIdxDim + 4);
  p.page_size = page_size;
  p.num_pages = num_pages;
  return from_hip(launch_store_index_k(p, reinterpret_cast<hipStream_t>(stream)), "index-K store launch");
}

dsa_status_t dsa_topk(const dsa_batch_t* batch, const float* logits, int64_t logits_row_stride,
                      int32_t k, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                      dsa_stream_t stream) {
  BatchView bv;
  dsa_status_t st = check_batch(batch, &bv);
  if (st != DSA_OK) return st;
  if (k < 1 || k > kTopkMaxK) return fail(DSA_ERR_INVALID_ARGUMENT, "k %d outside [1, %d]", k, kTopkMaxK);
  if (logits_row_stride < 1) return fail(DSA_ERR_INVALID_ARGUMENT, "logits_row_stride < 1");
  if (bv.num_rows > 0 && (!logits || !topk_idx))
    return fail(DSA_ERR_INVALID_ARGUMENT, "logits / topk_idx is NULL");
  const size_t need = topk_workspace_bytes(bv.num_rows, bv.max_seq_len_k, k);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (bv.num_rows == 0) return ok();
  TopkParams p;
  p.batch = bv;
  p.logits = logits;
  p.stride = logits_row_stride;
  p.k = k;
  p.topk_idx = topk_idx;
  p.chunk = need > 0 ? topk_chunk(bv.num_rows, bv.max_seq_len_k, k) : 0;
  p.chunks = p.chunk > 0 ? (bv.max_seq_len_k + p.chunk - 1) / p.chunk : 0;
  const size_t cands = (size_t)bv.num_rows * p.chunks * k;
  p.cand_key = p.chunk > 0 ? static_cast<uint32_t*>(workspace) : nullptr;
  p.cand_pos = p.chunk > 0 ? reinterpret_cast<int32_t*>(static_cast<uint32_t*>(workspace) + cands) : nullptr;
  p.q8 = nullptr;
  p.w = nullptr;
  p.cache = nullptr;
  p.page_bytes = 0;
  p.num_init = 0;
  p.num_local = 0;
  return from_hip(launch_topk(p, reinterpret_cast<hipStream_t>(stream)), "top-k launch");
}

dsa_status_t dsa_indexer_topk(const dsa_batch_t* batch, const void* q, const float* w, const void* index_cache,
                              int32_t num_heads, int32_t head_dim, int32_t num_init_tokens,
                              int32_t num_local_tokens, int32_t k, int32_t* topk_idx, void* workspace,
                              size_t workspace_bytes, dsa_stream_t stream) {
  BatchView bv;
  dsa_status_t st = check_batch(batch, &bv);
  if (st != DSA_OK) return st;
  if (num_heads != kIdxHeads || head_dim != kIdxDim)
    return fail(DSA_ERR_UNSUPPORTED, "dsa_indexer_topk needs 64 fp8 heads x 128 (got %d x %d)", num_heads, head_dim);
  if (k < 1 || k > kTopkMaxK) return fail(DSA_ERR_INVALID_ARGUMENT, "k %d outside [1, %d]", k, kTopkMaxK);
  if (num_init_tokens < 0 || num_local_tokens < 0)
    return fail(DSA_ERR_INVALID_ARGUMENT, "num_init_tokens %d / num_local_tokens %d < 0", num_init_tokens,
                num_local_tokens);
  if (bv.num_rows > 0 && (!q || !w || !index_cache || !topk_idx))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q / w / index_cache / topk_idx is NULL");
  if (bv.num_rows > 0 && !(aligned16(q) && aligned16(w) && aligned16(index_cache)))
    return fail(DSA_ERR_INVALID_ARGUMENT, "q, w and index_cache must be 16-byte aligned");
  const size_t need = indexer_topk_workspace_bytes(bv.num_rows, bv.max_seq_len_k, k);
  if (workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (need > 0 && !workspace) return fail(DSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (bv.num_rows == 0) return ok();
  TopkParams p;
  p.batch = bv;
  p.logits = nullptr;
  p.stride = bv.max_seq_len_k > 0 ? bv.max_seq_len_k : 1;   // rows end at their visible length
  p.k = k;
  p.topk_idx = topk_idx;
  p.chunk = indexer_topk_chunk(bv.num_rows, bv.max_seq_len_k, k);
  p.chunks = (bv.max_seq_len_k + p.chunk - 1) / p.chunk;
  const size_t cands = (size_t)bv.num_rows * p.chunks * k;
  p.cand_key = static_cast<uint32_t*>(workspace);
  p.cand_pos = reinterpret_cast<int32_t*>(static_cast<uint32_t*>(workspace) + cands);
  p.q8 = static_cast<const uint8_t*>(q);
  p.w = w;
  p.cache = static_cast<const uint8_t*>(index_cache);
  p.page_bytes = (int64_t)bv.page_size * (kIdxDim + 4);
  p.num_init = num_init_tokens;
  p.num_local = num_local_tokens;
  return from_hip(launch_indexer_topk(p, reinterpret_cast<hipStream_t>(stream)), "indexer top-k launch");
}

dsa_status_t sparse_mla_decode(const dsa_batch_t* batch, const void* q, const void* kv_cache,
                               dsa_dtype_t dtype, const int32_t* topk_idx, int32_t k,
                               int32_t num_heads, int32_t d_latent, int32_t d_rope, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               dsa_stream_t stream) {
  if (dtype == DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "an fp8 latent cache goes through sparse_mla_decode_fp8 (it needs the scales)");
  return run_mla(batch, true, q, kv_cache, dtype, topk_idx, k, num_heads, d_latent, d_rope,
                 softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

dsa_status_t sparse_mla_prefill(const dsa_batch_t* batch, const void* q, const void* kv_cache,
                                dsa_dtype_t dtype, const int32_t* topk_idx, int32_t k,
                                int32_t num_heads, int32_t d_latent, int32_t d_rope, float softmax_scale,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                dsa_stream_t stream) {
  if (dtype == DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "an fp8 latent cache goes through sparse_mla_prefill_fp8 (it needs the scales)");
  return run_mla(batch, false, q, kv_cache, dtype, topk_idx, k, num_heads, d_latent, d_rope,
                 softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

dsa_status_t sparse_mla_decode_fp8(const dsa_batch_t* batch, const void* q, float q_scale, const void* kv_cache,
                                   float kv_scale, const int32_t* topk_idx, int32_t k, int32_t num_heads,
                                   int32_t d_latent, int32_t d_rope, float softmax_scale, void* out, float* lse,
                                   void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  return run_mla(batch, true, q, kv_cache, DSA_FP8_E4M3, topk_idx, k, num_heads, d_latent, d_rope,
                 softmax_scale, out, lse, workspace, workspace_bytes, stream, q_scale, kv_scale);
}

dsa_status_t sparse_mla_prefill_fp8(const dsa_batch_t* batch, const void* q, float q_scale, const void* kv_cache,
                                    float kv_scale, const int32_t* topk_idx, int32_t k, int32_t num_heads,
                                    int32_t d_latent, int32_t d_rope, float softmax_scale, void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
  return run_mla(batch, false, q, kv_cache, DSA_FP8_E4M3, topk_idx, k, num_heads, d_latent, d_rope,
                 softmax_scale, out, lse, workspace, workspace_bytes, stream, q_scale, kv_scale);
}

size_t dsa_workspace_bytes(dsa_op_t op, const dsa_batch_t* batch, int32_t k, int32_t num_heads,
                           int32_t d_latent, dsa_dtype_t dtype) {
  BatchView bv;
  if (check_batch(batch, &bv) != DSA_OK) return (size_t)-1;
  if (op == DSA_OP_TOPK) {
    if (k < 1 || k > kTopkMaxK) {
      fail(DSA_ERR_INVALID_ARGUMENT, "k %d outside [1, %d]", k, kTopkMaxK);
      return (size_t)-1;
    }
    return topk_workspace_bytes(bv.num_rows, bv.max_seq_len_k, k);
  }
  if (op == DSA_OP_INDEXER_TOPK) {
    if (k < 1 || k > kTopkMaxK) {
      fail(DSA_ERR_INVALID_ARGUMENT, "k %d outside [1, %d]", k, kTopkMaxK);
      return (size_t)-1;
    }
    return indexer_topk_workspace_bytes(bv.num_rows, bv.max_seq_len_k, k);
  }
  if (op == DSA_OP_MLA_DECODE || op == DSA_OP_MLA_PREFILL) {
    MlaPlan plan;
    const int d_rope = (dtype == DSA_BF16 || dtype == DSA_FP8_E4M3) ? kMlaDr : 0;
    if (plan_mla(bv, k, num_heads, d_latent, d_rope, dtype, &plan) != DSA_OK) return (size_t)-1;
    return plan.workspace;
  }
  fail(DSA_ERR_INVALID_ARGUMENT, "unknown op %d", (int)op);
  return (size_t)-1;
}

const char* dsa_status_string(dsa_status_t status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "0.1.0"; }

}  // extern "C"
