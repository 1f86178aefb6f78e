// Per-row top-k of the indexer logits with causal/length masking.
//
// (SGLang "dsa_indexer.py" page: topk_transform over the [rows, keys] logits;
// forward_indexer takes topk(min(topk, seq_len)) and pads with -1;
// _forward_cuda_k_only relies on rows of length <= k giving [0 .. len-1, -1 ...].)
//
// One work-group of 1024 threads per selection (four waves per SIMD, so that
// the latency of one wave's LDS and memory operations is covered by the
// others). A selection is a whole row when there are enough rows to fill the
// chip. Otherwise (few rows, long rows) the row is cut into chunks: phase one
// selects, per (row, chunk), the chunk's own top k (key, position) pairs into
// the workspace, in position order; phase two selects the row's top k among
// the concatenated candidates. This is exact: an element of the row's top k
// has fewer than k elements before it in (key descending, position ascending)
// order within its own chunk, so its chunk keeps it. Scores become order-preserving 32-bit
// keys. A radix select on the key bits (12 + 12 + 8 bits, three LDS histograms)
// finds the exact k-th largest key `thr` and how many of the k winners are equal
// to it. A last ordered pass writes the winners in ascending position order:
// everything above `thr`, plus the first `need` positions equal to `thr`, so ties
// go to the lower positions.
//
// Rows of up to 32768 scores are read from HBM once: each thread keeps eight
// 16-byte loads in flight (the whole row is requested at once), converts them to
// keys into LDS and counts the first digit on the way. Longer rows are re-read
// from global memory (L2) by each pass. The histogram passes handle 8
// consecutive positions per thread per step; keys sharing the first digit with
// the k-th largest are appended (wave-aggregated) to a candidate list for the
// last digit. The ordered output gives each thread one contiguous run of
// positions: count winners in the run, one block-wide scan, place the run's
// winners in order in LDS, then write the row out with coalesced stores.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkCache = 32768;
constexpr int kTkBins = 4096;
constexpr int kTkLoadUnroll = 8;           // float4 loads in flight per thread
constexpr int kTkPer = 8;                  // consecutive positions per thread per pass step
constexpr int kTkCand = 4032;              // keys sharing the top 12 bits kept for the last level
constexpr int kTkRun = kTkCache / kTkThreads;   // 32 positions per thread in the output pass (cached rows)
constexpr int kTkCandPerWave = kTkCand / kTkWaves; // 252 candidate slots per wave
static_assert(kTkRun == 32, "the output pass handles one 32-position mask per cached run");
static_assert(kTkCache / (kTkPer * kTkThreads) * kTkPer == 32, "a cached selection gives each thread at most 32 positions");

struct TopkShared {
  uint32_t hist[kTkBins];
  alignas(16) uint32_t keys[kTkCache];
  uint32_t cand[kTkCand];
  uint32_t n_cand;
  uint32_t wave_cand[kTkWaves];
  uint32_t wave_sum[2][kTkWaves];
  uint32_t sel_bin;
  uint32_t sel_above;
};

// LDS word of position p. Each run of 32 positions (one thread's run in the
// output pass) keeps its eight 16-byte blocks, block j of run r stored at
// j ^ ((r >> 1) % 8), so that consecutive threads reading their runs block by
// block, and consecutive threads reading consecutive blocks, spread over the
// banks.
__device__ __forceinline__ int kslot(int p) {
  return (p & ~31) | ((((p >> 2) & 7) ^ ((p >> 6) & 7)) << 2) | (p & 3);
}

// Key of element q of a selection's source: a logit (converted) or a candidate key.
template <bool kKeys>
__device__ __forceinline__ uint32_t src_key(const void* __restrict__ src, int q) {
  if (kKeys) return static_cast<const uint32_t*>(src)[q];
  return ordered_key(static_cast<const float*>(src)[q]);
}

// Keys of elements [i, i + 8) (i a multiple of 8); elements >= n give 0.
template <bool kKeys>
__device__ __forceinline__ void load8(const void* __restrict__ src, const TopkShared& sh, bool cached,
                                      int n, int i, uint32_t (&u)[kTkPer]) {
  if (cached) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(sh.keys + kslot(i));
    const i32x4 b = *reinterpret_cast<const i32x4*>(sh.keys + kslot(i + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) { u[e] = (uint32_t)a[e]; u[4 + e] = (uint32_t)b[e]; }
  } else {
#pragma unroll
    for (int e = 0; e < kTkPer; ++e) {
      const int q = i + e < n ? i + e : n - 1;   // clamped: always in bounds
      u[e] = src_key<kKeys>(src, q);
    }
  }
#pragma unroll
  for (int e = 0; e < kTkPer; ++e) u[e] = (i + e < n) ? u[e] : 0u;
}

// Inclusive scan of v over the work-group in thread order; returns the
// inclusive prefix and stores the total in *total. One barrier; `buf` selects
// the double-buffered wave totals so consecutive calls need no extra barrier.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t block_scan(TopkShared& sh, uint32_t v, int buf, uint32_t* total) {
  const int lane = lane_id(), wave = wave_id();
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) sh.wave_sum[buf][wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t s = sh.wave_sum[buf][w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return before + incl;
}

// Largest bin b whose suffix count sum_{b' >= b} hist[b'] reaches `need`; also
// the count strictly above it.
__device__ void select_bin(TopkShared& sh, int nbins, uint32_t need, int buf, uint32_t* bin,
                           uint32_t* above) {
  const int tid = threadIdx.x;
  const int per = nbins >= kTkThreads ? nbins / kTkThreads : 1;
  const int active = nbins / per;
  // thread tid owns bins nbins-1-per*tid down to nbins-per*(tid+1), counted from the top
  uint32_t local = 0;
  if (tid < active)
    for (int q = 0; q < per; ++q) local += sh.hist[nbins - 1 - per * tid - q];
  uint32_t total;
  const uint32_t incl = block_scan(sh, local, buf, &total);
  const uint32_t before = incl - local;
  if (tid < active && before < need && incl >= need) {
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

enum TopkMode { kWholeRow = 0, kChunk = 1, kMerge = 2 };

template <int kMode>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkParams p) {
  constexpr bool kKeys = kMode == kMerge;             // the source holds keys, not logits
  __shared__ TopkShared sh;
  const BatchView& bv = p.batch;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  int b, j, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &j, &q_len);
  int cap = bv.max_pages_per_seq * bv.page_size;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int n_row = visible_keys(bv.seq_lens_k[b], q_len, j, cap);
  const int k = p.k;
  int32_t* out = p.topk_idx + (int64_t)t * k;
  const int64_t cand0 = ((int64_t)t * p.chunks + (kMode == kChunk ? blockIdx.y : 0)) * k;

  // this selection: elements [0, n) of `src`
  int n = n_row;
  int base = 0;                                       // chunk: position of element 0
  const void* src = p.logits + (int64_t)t * p.stride;
  if (kMode == kChunk) {
    if (n_row <= k) return;                           // short rows are the merge's
    base = (int)blockIdx.y * p.chunk;
    if (base >= n_row) return;
    n = min(p.chunk, n_row - base);
    src = p.logits + (int64_t)t * p.stride + base;
    if (n <= k) {                                     // the whole chunk is a candidate
      for (int i = tid; i < n; i += kTkThreads) {
        p.cand_key[cand0 + i] = src_key<false>(src, i);
        p.cand_pos[cand0 + i] = base + i;
      }
      return;
    }
  } else if (kMode == kMerge) {
    if (n_row > k) {                                  // every chunk but the last gave k candidates
      const int nch = (n_row + p.chunk - 1) / p.chunk;
      n = (nch - 1) * k + min(k, n_row - (nch - 1) * p.chunk);
    }
    src = p.cand_key + cand0;
  }
  if (n <= k) {  // short row (or as many candidates as winners): every element, in order, then -1
    for (int i = tid; i < k; i += kTkThreads)
      out[i] = i < n ? (kMode == kMerge && n_row > k ? p.cand_pos[cand0 + i] : i) : -1;
    return;
  }

  const bool cached = n <= kTkCache;
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();

  // ---- level 0 (bits 31..20) while reading the row once ----
  const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
  const int n4 = vec ? n / 4 : 0;
  for (int i0 = 0; i0 < n4; i0 += kTkThreads * kTkLoadUnroll) {
    i32x4 v[kTkLoadUnroll];
#pragma unroll
    for (int u = 0; u < kTkLoadUnroll; ++u) {
      int i4 = i0 + u * kTkThreads + tid;
      i4 = i4 < n4 ? i4 : n4 - 1;               // clamped: always in bounds
      v[u] = static_cast<const i32x4*>(src)[i4];
    }
#pragma unroll
    for (int u = 0; u < kTkLoadUnroll; ++u) {
      const int i4 = i0 + u * kTkThreads + tid;
      if (i4 < n4) {
        uint32_t kk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kk[e] = kKeys ? (uint32_t)v[u][e] : ordered_key(__int_as_float(v[u][e]));
          atomicAdd(&sh.hist[kk[e] >> 20], 1u);
        }
        if (cached)
          *reinterpret_cast<i32x4*>(sh.keys + kslot(4 * i4)) = i32x4{(int)kk[0], (int)kk[1], (int)kk[2], (int)kk[3]};
      }
    }
  }
  for (int i = 4 * n4 + tid; i < n; i += kTkThreads) {
    const uint32_t kk = src_key<kKeys>(src, i);
    if (cached) sh.keys[kslot(i)] = kk;
    atomicAdd(&sh.hist[kk >> 20], 1u);
  }
  __syncthreads();
  uint32_t need = (uint32_t)k;
  uint32_t bin, above;
  select_bin(sh, kTkBins, need, 0, &bin, &above);
  uint32_t prefix = bin;
  need -= above;

  // ---- level 1 (bits 19..8) among keys whose top 12 bits equal the prefix;
  //      those keys are also collected (unordered) for the last level ----
  const bool keep = sh.hist[prefix] <= (uint32_t)kTkCand;   // read before the histogram is cleared
  __syncthreads();
  for (int i = tid; i < kTkBins; i += kTkThreads) sh.hist[i] = 0;
  if (tid == 0) sh.n_cand = 0;
  __syncthreads();
  // Each wave appends its matches to its own 252 slots of the list (ballot and
  // lane rank: no returning atomics in the loop); a wave that runs out of
  // slots makes the last digit take the full pass instead.
  const int wave = wave_id();
  uint32_t wcnt = 0;                                   // this wave's matches so far (wave-uniform)
  // one matching key of the lane per round: histogram count and list append
  auto take_match = [&](bool m, uint32_t x) {
    if (m) atomicAdd(&sh.hist[(x >> 8) & 0xfffu], 1u);
    const uint64_t mask = __ballot(m);
    const uint32_t slot = wcnt + lanes_below(mask);
    if (keep && m && slot < (uint32_t)kTkCandPerWave) sh.cand[wave * kTkCandPerWave + slot] = x;
    wcnt += (uint32_t)__builtin_popcountll(mask);
  };
  if (cached) {
    // The thread's (at most 32) positions i = 8 tid + 8192 j + e first give
    // one match mask; the matches are then handled in rounds of one per lane,
    // so the rounds of the whole pass number the most matches of one lane.
    uint32_t mm = 0;
#pragma unroll
    for (int j = 0; j < kTkCache / (kTkPer * kTkThreads); ++j) {
      const int i = kTkPer * tid + kTkPer * kTkThreads * j;
      if (i < n) {
        uint32_t u[kTkPer];
        load8<kKeys>(src, sh, true, n, i, u);
#pragma unroll
        for (int e = 0; e < kTkPer; ++e) mm |= ((i + e < n && (u[e] >> 20) == prefix) ? 1u : 0u) << (kTkPer * j + e);
      }
    }
    while (__ballot(mm != 0u)) {
      const bool m = mm != 0u;
      uint32_t x = 0;
      if (m) {
        const int b = __builtin_ctz(mm);
        mm &= mm - 1u;
        x = sh.keys[kslot(kTkPer * tid + kTkPer * kTkThreads * (b / kTkPer) + b % kTkPer)];
      }
      take_match(m, x);
    }
  }
  for (int i = kTkPer * tid; !cached && i < n; i += kTkPer * kTkThreads) {
    uint32_t u[kTkPer];
    load8<kKeys>(src, sh, cached, n, i, u);
    // matches are rare: each round handles one match per lane, so a wave issues
    // as many LDS atomics as its busiest lane has matches (not one per element)
    uint32_t mm = 0;
#pragma unroll
    for (int e = 0; e < kTkPer; ++e) mm |= ((i + e < n && (u[e] >> 20) == prefix) ? 1u : 0u) << e;
    while (__ballot(mm != 0u)) {
      const bool m = mm != 0u;
      uint32_t x = 0;
      if (m) {
        const int e = __builtin_ctz(mm);
        mm &= mm - 1u;
        x = u[0];
#pragma unroll
        for (int q = 1; q < kTkPer; ++q) x = (e == q) ? u[q] : x;
      }
      take_match(m, x);
    }
  }
  if (lane_id() == 0) sh.wave_cand[wave] = wcnt;
  __syncthreads();
  select_bin(sh, kTkBins, need, 1, &bin, &above);
  prefix = (prefix << 12) | bin;
  need -= above;

  // ---- level 2 (bits 7..0) among keys whose top 24 bits equal the prefix ----
  for (int i = tid; i < 256; i += kTkThreads) sh.hist[i] = 0;
  __syncthreads();
  bool kept = keep;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) kept = kept && sh.wave_cand[w] <= (uint32_t)kTkCandPerWave;
  if (kept) {
    const uint32_t nc = sh.wave_cand[wave];            // wave w scans wave w's slots
    for (uint32_t i = lane_id(); i < nc; i += kWave) {
      const uint32_t u = sh.cand[wave * kTkCandPerWave + i];
      if ((u >> 8) == prefix) atomicAdd(&sh.hist[u & 0xffu], 1u);
    }
  } else {
    for (int i = kTkPer * tid; i < n; i += kTkPer * kTkThreads) {
      uint32_t u[kTkPer];
      load8<kKeys>(src, sh, cached, n, i, u);
#pragma unroll
      for (int e = 0; e < kTkPer; ++e)
        if (i + e < n && (u[e] >> 8) == prefix) atomicAdd(&sh.hist[u[e] & 0xffu], 1u);
    }
  }
  __syncthreads();
  select_bin(sh, 256, need, 0, &bin, &above);
  const uint32_t thr = (prefix << 8) | bin;
  need -= above;  // how many keys equal to thr are among the winners (>= 1)

  // ---- ordered output ----
  // A winner at position p goes to slot #winners before p = (#keys > thr before
  // p) + min(#keys == thr before p, need). Thread tid owns a run of
  // consecutive positions, handled 32 at a time as bit masks: count its winners,
  // one block-wide scan, then place them in order.
  const int run_len = cached ? kTkRun : ((n + kTkThreads - 1) / kTkThreads + 31) & ~31;
  const int run0 = run_len * tid;
  // masks of the keys > thr and == thr among positions [p0, p0 + 32)
  auto masks32 = [&](int p0, uint32_t* gtm, uint32_t* eqm) {
    uint32_t key[32];
    if (cached) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const i32x4 a = *reinterpret_cast<const i32x4*>(sh.keys + kslot(p0 + 4 * j));
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * j + e] = (uint32_t)a[e];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t u[kTkPer];
        load8<kKeys>(src, sh, false, n, p0 + 8 * j, u);
#pragma unroll
        for (int e = 0; e < kTkPer; ++e) key[8 * j + e] = u[e];
      }
    }
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      g |= (key[e] > thr ? 1u : 0u) << e;
      q |= (key[e] == thr ? 1u : 0u) << e;
    }
    const int nv = n - p0;                                  // valid positions in the block
    const uint32_t vmask = nv >= 32 ? ~0u : (nv <= 0 ? 0u : ((1u << nv) - 1u));
    *gtm = g & vmask;
    *eqm = q & vmask;
  };
  uint32_t cgt = 0, ceq = 0;
  uint32_t gtm0 = 0, eqm0 = 0;                          // cached rows: the run's only block, kept for the write
  for (int p0 = run0; p0 < run0 + run_len && p0 < n; p0 += 32) {
    uint32_t gtm, eqm;
    masks32(p0, &gtm, &eqm);
    gtm0 = gtm;
    eqm0 = eqm;
    cgt += (uint32_t)__builtin_popcount(gtm);
    ceq += (uint32_t)__builtin_popcount(eqm);
  }
  // winners and ties before this thread's run: for selections below 65536
  // elements one scan of both counts, (> thr) in the high half and (== thr)
  // in the low half (neither reaches 2^16, so no carry crosses); else two
  uint32_t gt_before, eq_before, total;
  if (n < 65536) {
    const uint32_t both = (cgt << 16) | ceq;
    const uint32_t before = block_scan(sh, both, 0, &total) - both;
    gt_before = before >> 16;
    eq_before = before & 0xffffu;
  } else {
    gt_before = block_scan(sh, cgt, 1, &total) - cgt;
    eq_before = block_scan(sh, ceq, 0, &total) - ceq;
  }
  uint32_t slot = gt_before + (eq_before < need ? eq_before : need);
  if (cgt + ceq) {
    for (int p0 = run0; p0 < run0 + run_len && p0 < n; p0 += 32) {
      uint32_t gtm = gtm0, eqm = eqm0;
      if (!cached) masks32(p0, &gtm, &eqm);
      // the first (need - eq_before) ties of the block are winners
      uint32_t win = gtm;
      for (uint32_t r = eq_before; r < need && eqm; ++r) {
        const uint32_t low = eqm & (0u - eqm);
        win |= low;
        eqm ^= low;
      }
      eq_before += (uint32_t)__builtin_popcount(eqm) + (uint32_t)__builtin_popcount(win & ~gtm);
      while (win) {
        const int e = __builtin_ctz(win);
        if (slot < (uint32_t)k) sh.hist[slot] = (uint32_t)(p0 + e);
        ++slot;
        win &= win - 1u;
      }
    }
  }
  // The winners (element indices, ascending) were staged in LDS in the
  // histogram area, free since the last bin selection; they leave in
  // consecutive, coalesced stores instead of each thread's scattered ones.
  __syncthreads();
  for (int i = tid; i < k; i += kTkThreads) {
    const int e = (int)sh.hist[i];
    if (kMode == kWholeRow) {
      out[i] = e;
    } else if (kMode == kChunk) {
      p.cand_key[cand0 + i] = cached ? sh.keys[kslot(e)] : src_key<false>(src, e);
      p.cand_pos[cand0 + i] = base + e;
    } else {
      out[i] = p.cand_pos[cand0 + e];
    }
  }
}

}  // namespace

int topk_chunk(int num_rows, int max_len, int k) {
  // Two phases pay off when whole-row work-groups cannot fill the chip and
  // the rows are longer than the LDS key cache (a whole-row work-group would
  // re-read them from L2 in every pass; for cached rows one phase is faster,
  // measured). The candidates of a row (chunks x k) must fit the merge's LDS
  // key cache, and a chunk its own. Chunks start at 16384 positions: both
  // phases are dominated by the fixed cost of a selection, and 16384 beats
  // 8192 (more, shorter phase-one selections and twice the candidates) and
  // 32768 on the 8 x 128k decode (34.6 against 38.7 and 35.5 us, measured).
  if (num_rows > 256 || k > kTkCache / 2 || max_len <= kTkCache) return 0;
  int chunk = 16384;
  if (chunk < 2 * k) chunk = 2 * k;
  const int64_t need = ((int64_t)max_len * k + kTkCache - 1) / kTkCache;   // chunks * k <= kTkCache
  while (chunk < need) chunk *= 2;
  if (chunk > kTkCache || max_len < 2 * chunk - chunk / 2) return 0;
  return chunk;
}

size_t topk_workspace_bytes(int num_rows, int max_len, int k) {
  const int chunk = topk_chunk(num_rows, max_len, k);
  if (chunk == 0) return 0;
  const int chunks = (max_len + chunk - 1) / chunk;
  return (size_t)num_rows * chunks * k * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  if (p.chunk == 0) {
    hipLaunchKernelGGL(topk_kernel<kWholeRow>, dim3(p.batch.num_rows), dim3(kTkThreads), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_kernel<kChunk>, dim3(p.batch.num_rows, p.chunks), dim3(kTkThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel<kMerge>, dim3(p.batch.num_rows), dim3(kTkThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
