// Per-row top-k of the indexer logits with causal/length masking.
//
// (SGLang "dsa_indexer.py" page: topk_transform over the [rows, keys] logits;
// forward_indexer takes topk(min(topk, seq_len)) and pads with -1;
// _forward_cuda_k_only relies on rows of length <= k giving [0 .. len-1, -1 ...].)
//
// One work-group of 1024 threads per row. Scores become order-preserving 32-bit
// keys. A radix select on the key bits (12 + 12 + 8 bits, three LDS histograms)
// finds the exact k-th largest key `thr` and how many of the k winners are equal
// to it. A last ordered pass writes the winners in ascending position order:
// everything above `thr`, plus the first `need` positions equal to `thr`, so ties
// go to the lower positions. Rows of up to 32768 scores are kept in LDS after the
// first read from HBM; longer rows are re-read from global memory (L2) by each
// pass.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkCache = 32768;
constexpr int kTkBins = 4096;

struct TopkShared {
  uint32_t hist[kTkBins];
  uint32_t keys[kTkCache];
  uint32_t wave_sum[kTkWaves];
  uint32_t wave_cnt[2][2][kTkWaves];
  uint32_t sel_bin;
  uint32_t sel_above;
};

__device__ __forceinline__ uint32_t load_key(const float* __restrict__ row, const TopkShared& sh,
                                             bool cached, int i) {
  return cached ? sh.keys[i] : ordered_key(row[i]);
}

// Find the largest bin b (of nbins, counted in `hist`) whose suffix count
// sum_{b' >= b} hist[b'] reaches `need`; return b and the count strictly above it.
__device__ void select_bin(TopkShared& sh, int nbins, uint32_t need, uint32_t* bin, uint32_t* above) {
  const int tid = threadIdx.x;
  const int per = nbins / kTkThreads > 0 ? nbins / kTkThreads : 1;
  const int active = nbins / per;       // threads that own bins
  // thread tid owns bins [nbins - per*(tid+1), nbins - per*tid), counted from the top
  uint32_t local = 0;
  if (tid < active) {
    for (int q = 0; q < per; ++q) local += sh.hist[nbins - 1 - per * tid - q];
  }
  // block-wide exclusive scan of `local` in thread order
  const int lane = lane_id(), wave = wave_id();
  uint32_t incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t v = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += v;
  }
  if (lane == kWave - 1) sh.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t before = incl - local;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  if (tid < active && before < need && before + local >= need) {
    uint32_t cum = before;
    for (int q = 0; q < per; ++q) {
      const int bb = nbins - 1 - per * tid - q;
      const uint32_t h = sh.hist[bb];
      if (cum + h >= need) {
        sh.sel_bin = (uint32_t)bb;
        sh.sel_above = cum;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
  *bin = sh.sel_bin;
  *above = sh.sel_above;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const BatchView& bv = p.batch;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  int b, j, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &j, &q_len);
  int cap = bv.max_pages_per_seq * bv.page_size;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int n = visible_keys(bv.seq_lens_k[b], q_len, j, cap);
  const int k = p.k;
  int32_t* out = p.topk_idx + (int64_t)t * k;

  if (n <= k) {  // short row: every visible position, in order, then -1
    for (int i = tid; i < k; i += kTkThreads) out[i] = i < n ? i : -1;
    return;
  }

  const float* row = p.logits + (int64_t)t * p.stride;
  const bool cached = n <= kTkCache;

  // level 0: bits 31..20, loading the row (and caching its keys)
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kTkThreads) {
    const uint32_t u = ordered_key(row[i]);
    if (cached) sh.keys[i] = u;
    atomicAdd(&sh.hist[u >> 20], 1u);
  }
  __syncthreads();
  uint32_t need = (uint32_t)k;
  uint32_t bin, above;
  select_bin(sh, kTkBins, need, &bin, &above);
  uint32_t prefix = bin;
  need -= above;

  // level 1: bits 19..8 among keys whose top 12 bits equal the prefix
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kTkThreads) {
    const uint32_t u = load_key(row, sh, cached, i);
    if ((u >> 20) == prefix) atomicAdd(&sh.hist[(u >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  select_bin(sh, kTkBins, need, &bin, &above);
  prefix = (prefix << 12) | bin;
  need -= above;

  // level 2: bits 7..0 among keys whose top 24 bits equal the prefix
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kTkThreads) {
    const uint32_t u = load_key(row, sh, cached, i);
    if ((u >> 8) == prefix) atomicAdd(&sh.hist[u & 0xffu], 1u);
  }
  __syncthreads();
  select_bin(sh, 256, need, &bin, &above);
  const uint32_t thr = (prefix << 8) | bin;
  need -= above;  // how many keys equal to thr are among the winners (>= 1)

  // ordered output pass: position of a winner = winners before it
  //   = (#keys > thr before it) + min(#keys == thr before it, need)
  const int lane = lane_id(), wave = wave_id();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t base_gt = 0, base_eq = 0;
  int it = 0;
  for (int i0 = 0; i0 < n; i0 += kTkThreads, ++it) {
    const int i = i0 + tid;
    const uint32_t u = i < n ? load_key(row, sh, cached, i) : 0u;
    const bool gt = i < n && u > thr;
    const bool eq = i < n && u == thr;
    const uint64_t mgt = __ballot(gt);
    const uint64_t meq = __ballot(eq);
    const int buf = it & 1;
    if (lane == 0) {
      sh.wave_cnt[buf][0][wave] = (uint32_t)__popcll(mgt);
      sh.wave_cnt[buf][1][wave] = (uint32_t)__popcll(meq);
    }
    __syncthreads();
    uint32_t off_gt = 0, off_eq = 0, tot_gt = 0, tot_eq = 0;
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t a = sh.wave_cnt[buf][0][w], e = sh.wave_cnt[buf][1][w];
      if (w < wave) { off_gt += a; off_eq += e; }
      tot_gt += a;
      tot_eq += e;
    }
    const uint32_t gt_before = base_gt + off_gt + (uint32_t)__popcll(mgt & lt_mask);
    const uint32_t eq_before = base_eq + off_eq + (uint32_t)__popcll(meq & lt_mask);
    if (gt || (eq && eq_before < need)) {
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      if (pos < (uint32_t)k) out[pos] = i;
    }
    base_gt += tot_gt;
    base_eq += tot_eq;
    if (base_gt + (base_eq < need ? base_eq : need) >= (uint32_t)k) break;
  }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(p.batch.num_rows), dim3(kTkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
