// Lightning-indexer scores over a paged fp8 index-K cache.
//
//   logits[t, s] = sum_h w[t, h] * relu(sigma_s * (q[t, h] . k_s))
//
// (SGLang "dsa_indexer.py" page: Indexer._get_topk_paged feeds q_fp8 [T, 64, 128],
// the 132-byte-per-token paged cache, weights [T, 64] and the block table to the
// paged MQA-logits kernel; forward_indexer gives the same score per request.)
//
// fp8 path (H = 64, D = 128): the q . k contraction runs on the gfx950 fp8 MFMA
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales. Heads are the M
// dimension and keys the N dimension, so one 16x16 accumulator holds 16 heads x
// 16 keys and each lane ends up with 16 heads of a single key: relu, head weight
// and the head sum are lane-local, followed by two cross-lane adds. sigma >= 0
// commutes with relu, so it multiplies the head sum once per key.
//
// Work split: one work-group per (row, chunk of 512 keys); the hardware
// dispatcher balances the ragged rows. The row's q is staged once in LDS. Each
// wave owns 128 consecutive keys (8 groups of 16; a 64-token page holds 4
// groups), issues all of their loads straight from HBM into MFMA operand
// registers before computing anything (16 KB in flight per wave), and writes
// one fp32 logit per key. The kernel is bound by HBM: 132 bytes of cache per
// key against 16384 fp8 MACs.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIdxWaves = 4;
constexpr int kIdxGroupsPerWave = 8;                               // 16 keys each
constexpr int kIdxChunk = 16 * kIdxGroupsPerWave * kIdxWaves;      // 512 keys per work-group

__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c) {
  // format 0 = fp8 e4m3 for both operands; E8M0 scale 127 = 2^0 for both.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__global__ __launch_bounds__(64 * kIdxWaves) void indexer_fp8_kernel(IndexerParams p) {
  __shared__ i32x8 q_lds[kIdxHeads * kIdxDim / 32];   // the row's q, 8 KB
  const BatchView& bv = p.batch;
  const int t = blockIdx.x;
  int b, j, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &j, &q_len);
  int cap = bv.max_pages_per_seq * bv.page_size;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int visible = visible_keys(bv.seq_lens_k[b], q_len, j, cap);
  const int k0 = blockIdx.y * kIdxChunk;
  if (k0 >= visible) return;
  const int k_end = min(k0 + kIdxChunk, visible);

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());   // uniform: scalar page lookups
  const int g = lane >> 4;   // lane group: which 32-byte slice of the 128-wide dot product
  const int c = lane & 15;   // head (A rows) / key (B columns) inside a 16-wide tile

  // q (64 x 128 fp8) is staged in LDS once for the four waves; its load is
  // issued first and stored to LDS after the key loads are in flight
  const i32x8* qrow = reinterpret_cast<const i32x8*>(static_cast<const uint8_t*>(p.q) +
                                                     (int64_t)t * (kIdxHeads * kIdxDim));
  const i32x8 qv = qrow[tid];

  const int P = bv.page_size;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;
  const int64_t scale_off = (int64_t)P * kIdxDim;
  const int wbase = k0 + 16 * kIdxGroupsPerWave * wave;   // this wave's first key

  // page of every group first (wave-uniform scalar loads, one wait), then every
  // key load of this wave before any compute: lane (c, g) of group u holds key
  // wbase + 16u + c, bytes [32g, 32g + 32)
  int page[kIdxGroupsPerWave];
#pragma unroll
  for (int u = 0; u < kIdxGroupsPerWave; ++u) {
    const int s0 = wbase + 16 * u;
    page[u] = (s0 < k_end) ? bt[s0 / P] : -1;
  }
  i32x8 kb[kIdxGroupsPerWave];
  float sig[kIdxGroupsPerWave];
  bool ok[kIdxGroupsPerWave];
#pragma unroll
  for (int u = 0; u < kIdxGroupsPerWave; ++u) {
    const int s0 = wbase + 16 * u;
    ok[u] = page[u] >= 0 && page[u] < bv.num_pages;
    const uint8_t* pg = p.cache + (int64_t)(ok[u] ? page[u] : 0) * p.page_bytes;
    const int slot = (s0 % P) + c;   // < P: s0 is a multiple of 16 and P of 16
    kb[u] = *reinterpret_cast<const i32x8*>(pg + (int64_t)slot * kIdxDim + 32 * g);
    sig[u] = *reinterpret_cast<const float*>(pg + scale_off + 4 * slot);
  }

  // head weights in accumulator order: lane (c, g) holds rows 4g + i of each tile
  float wv[16];
  const float* wrow = p.w + (int64_t)t * kIdxHeads;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 16 * m + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[4 * m + i] = w4[i];
  }

  q_lds[tid] = qv;
  __syncthreads();
  // q as four 16-head A operands: lane (c, g) holds head 16m + c, bytes [32g, 32g + 32)
  i32x8 qa[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) qa[m] = q_lds[(16 * m + c) * (kIdxDim / 32) + g];

  float* out = p.logits + (int64_t)t * p.stride;
#pragma unroll
  for (int u = 0; u < kIdxGroupsPerWave; ++u) {
    const int s0 = wbase + 16 * u;
    if (s0 >= k_end) break;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 acc = mfma_fp8_16x16x128(qa[m], kb[u], zero);
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(wv[4 * m + i], fmaxf(acc[i], 0.f), part);
    }
    part += shfl_xor_f(part, 16);
    part += shfl_xor_f(part, 32);
    const int s = s0 + c;
    if (g == 0 && s < k_end) out[s] = ok[u] ? part * sig[u] : -INFINITY;
  }
}

// fp32 keys (H <= 64, D <= 128): one thread per key, q of the row staged in LDS.
constexpr int kF32Block = 256;

__global__ __launch_bounds__(kF32Block) void indexer_f32_kernel(IndexerParams p) {
  __shared__ float qs[kIdxHeads * kIdxDim];
  __shared__ float ws[kIdxHeads];
  const BatchView& bv = p.batch;
  const int t = blockIdx.x;
  int b, j, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &j, &q_len);
  int cap = bv.max_pages_per_seq * bv.page_size;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int visible = visible_keys(bv.seq_lens_k[b], q_len, j, cap);
  const int s = blockIdx.y * kF32Block + threadIdx.x;
  if (blockIdx.y * kF32Block >= visible) return;
  const int H = p.heads, D = p.dim;
  const float* qrow = static_cast<const float*>(p.q) + (int64_t)t * H * D;
  for (int i = threadIdx.x; i < H * D; i += kF32Block) qs[i] = qrow[i];
  for (int i = threadIdx.x; i < H; i += kF32Block) ws[i] = p.w[(int64_t)t * H + i];
  __syncthreads();
  if (s >= visible) return;
  const int P = bv.page_size;
  const int page = bv.block_table[(int64_t)b * bv.max_pages_per_seq + s / P];
  float* out = p.logits + (int64_t)t * p.stride;
  if (page < 0 || page >= bv.num_pages) { out[s] = -INFINITY; return; }
  const uint8_t* pg = p.cache + (int64_t)page * p.page_bytes;
  const float* key = reinterpret_cast<const float*>(pg) + (int64_t)(s % P) * D;
  const float sigma = reinterpret_cast<const float*>(pg + (int64_t)P * D * 4)[s % P];
  float acc = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qs[h * D + d], key[d], dot);
    acc = fmaf(ws[h], fmaxf(dot, 0.f), acc);
  }
  out[s] = acc * sigma;
}

}  // namespace

hipError_t launch_indexer_fp8(const IndexerParams& p, hipStream_t s) {
  const int chunks = (p.batch.max_seq_len_k + kIdxChunk - 1) / kIdxChunk;
  if (p.batch.num_rows == 0 || chunks == 0) return hipSuccess;
  dim3 grid(p.batch.num_rows, chunks);
  hipLaunchKernelGGL(indexer_fp8_kernel, grid, dim3(64 * kIdxWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_indexer_f32(const IndexerParams& p, hipStream_t s) {
  const int chunks = (p.batch.max_seq_len_k + kF32Block - 1) / kF32Block;
  if (p.batch.num_rows == 0 || chunks == 0) return hipSuccess;
  dim3 grid(p.batch.num_rows, chunks);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(kF32Block), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
