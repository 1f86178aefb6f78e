// Launch parameters shared between the host API layer and the kernel files.
// The host layer validates every field before a launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

struct BatchView {
  int32_t num_seqs;
  int32_t num_rows;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t max_seq_len_k;
  int32_t max_seq_len_q;
  const int32_t* block_table;
  const int32_t* seq_lens_k;
  const int32_t* cu_seqlens_q;  // nullptr = decode
};

struct IndexerParams {
  BatchView batch;
  const void* q;          // [T, H, D]
  const float* w;         // [T, H]
  const uint8_t* cache;   // pages of page_bytes
  int64_t page_bytes;
  int32_t heads;
  int32_t dim;
  float* logits;
  int64_t stride;
  int32_t num_init;   // forced positions: the first num_init and the last num_local of a row get +inf
  int32_t num_local;
};

struct TopkParams {
  BatchView batch;
  const float* logits;
  int64_t stride;
  int32_t k;
  int32_t* topk_idx;      // [T, k]
  // two phases (chunk > 0): per (row, chunk) candidates [T, chunks, k]
  int32_t chunk;          // positions per chunk, 0 = one work-group per row
  int32_t chunks;         // chunks of the longest row
  uint32_t* cand_key;     // order-preserving keys
  int32_t* cand_pos;      // positions
  // fused with the scores (dsa_indexer_topk): the indexer's fp8 inputs; the
  // chunk selections then take their keys from the scores they compute
  const uint8_t* q8;      // [T, 64, 128] E4M3 codes
  const float* w;         // [T, 64] gates
  const uint8_t* cache;   // index-K pages
  int64_t page_bytes;
  int32_t num_init;       // forced positions (init / local), as in IndexerParams
  int32_t num_local;
};

struct MlaParams {
  BatchView batch;
  const void* q;          // [T, Hm, Dqk]
  const void* kv;         // [num_pages, P, Dqk]
  const int32_t* topk_idx;
  int32_t k;
  int32_t heads;
  int32_t d_latent;
  int32_t d_rope;
  float softmax_scale;
  float q_scale;          // fp8 path: q = codes * q_scale, rows = codes * kv_scale
  float kv_scale;
  void* out;              // [T, Hm, Dl]
  float* lse;             // [T, Hm] or nullptr
  // split-KV partials (splits > 1): O / l as [T, splits, Hm, Dl] bf16 bits and
  // the lse as [T, splits, Hm] fp32
  uint16_t* part_o;
  float* part_lse;
  int32_t splits;
  int32_t entries_per_split;  // multiple of the tile height
};

// Shape constants of the MFMA paths.
constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kMlaHeadsPerGroup = 64;
constexpr int kMlaDl = 512;
constexpr int kMlaDr = 64;
constexpr int kMlaDqk = kMlaDl + kMlaDr;
constexpr int kMlaTile = 32;
constexpr int kMlaMaxEntriesPerBlock = 2048;
constexpr int kMlaFp8MaxEntriesPerBlock = 1024;
constexpr int kTopkMaxK = 4096;

// Split-KV policy for the bf16 kernel: enough work-groups to cover the chip
// while keeping every split at least a few tiles long.
int mla_bf16_splits(int num_rows, int k, int heads);
int mla_entries_per_split(int k, int splits);

// Top-k plan: chunk length of the two-phase selection (0 = one phase) and the
// workspace it needs.
int topk_chunk(int num_rows, int max_len, int k);
size_t topk_workspace_bytes(int num_rows, int max_len, int k);

// fp8 quantization of the index query rows (T * H rows of 128) and gates
struct QuantQParams {
  const uint16_t* q;        // [rows, 128] bf16
  const float* w;           // [rows]
  uint8_t* q8;              // [rows, 128] E4M3FN codes
  float* w_eff;             // [rows]
  int64_t rows;
};

// fp8 quantization of new index keys and their paged store
struct StoreKParams {
  const uint16_t* key;            // [num_tokens, 128] bf16
  const int64_t* slot_mapping;    // [num_tokens]
  uint8_t* cache;                 // [num_pages, page_bytes]
  int64_t num_tokens;
  int64_t page_bytes;             // page_size * 128 + 4 * page_size
  int32_t page_size;
  int32_t num_pages;
};

hipError_t launch_quant_index_q(const QuantQParams& p, hipStream_t s);
hipError_t launch_store_index_k(const StoreKParams& p, hipStream_t s);
hipError_t launch_indexer_fp8(const IndexerParams& p, hipStream_t s);
hipError_t launch_indexer_f32(const IndexerParams& p, hipStream_t s);
hipError_t launch_indexer_force(const IndexerParams& p, hipStream_t s);
hipError_t launch_topk(const TopkParams& p, hipStream_t s);
// Scores and top-k in one pass over the index cache, no logits in memory:
// per (row, chunk of `chunk` keys) the scores go straight into the
// selection's LDS key cache and the chunk's top k become candidates; a merge
// over the candidates gives each row's top k.
int indexer_topk_chunk(int num_rows, int max_len, int k);
size_t indexer_topk_workspace_bytes(int num_rows, int max_len, int k);
hipError_t launch_indexer_topk(const TopkParams& p, hipStream_t s);
hipError_t launch_mla_bf16(const MlaParams& p, hipStream_t s);
hipError_t launch_mla_f32(const MlaParams& p, hipStream_t s);
hipError_t launch_mla_fp8(const MlaParams& p, hipStream_t s);
hipError_t launch_mla_combine_bf16(const MlaParams& p, hipStream_t s);
int mla_fp8_splits(int num_rows, int k, int heads);

// Records a printf-style message as this thread's dsa_last_error() text and
// returns `st`.
dsa_status_t set_error(dsa_status_t st, const char* fmt, ...);

}  // namespace dsa
