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
// winners in order in LDS, then write the row out with coalesced stores. For
// selections held in LDS the middle pass reads each thread's output run and
// keeps two masks of it (first digit above the prefix, equal to it), so the
// output pass compares only the run's positions in the prefix bin with the
// exact k-th key.
//
// Fused with the scores (dsa_indexer_topk): phase one runs in work-groups of
// 256 threads, one per (row, chunk of up to 8192 keys), three per CU. Each
// computes its chunk's lightning-indexer scores itself (the fp8 MFMA
// contraction of the decode indexer, same operand layout and summation order,
// so the scores are the same floats), converts them to keys straight into its
// LDS key cache while counting the first digit, and selects the chunk's
// candidates from there; the merge phase is the one above. No score reaches
// memory.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTkThreads = 1024;           // whole-row, chunk and merge selections
constexpr int kFuThreads = 256;            // fused scores + chunk selection
constexpr int kFuAhead = 1;                // fused scores: batches of 64 keys in flight per wave
constexpr int kTkBins = 4096;
constexpr int kTkLoadUnroll = 8;           // float4 loads in flight per thread
constexpr int kTkPer = 8;                  // consecutive positions per thread per pass step
constexpr int kTkRun = 32;                 // positions per thread in the output pass (cached selections)
constexpr int kTkCandPerWave = 252;        // candidate slots per wave for the last level

// LDS of a selection by kThreads threads: the key cache holds 32 positions per
// thread (one output run each), the candidate list 252 keys per wave.
template <int kThreads>
struct TopkShared {
  static constexpr int kWaves = kThreads / kWave;
  static constexpr int kCache = kTkRun * kThreads;
  static constexpr int kCand = kWaves * kTkCandPerWave;
  uint32_t hist[kTkBins];
  alignas(16) uint32_t keys[kCache];
  uint32_t cand[kCand];
  uint32_t n_cand;
  uint32_t wave_cand[kWaves];
  uint32_t wave_sum[2][kWaves];
  uint32_t sel_bin;
  uint32_t sel_above;
  uint32_t sel_count;
};

constexpr int kTkCache = TopkShared<kTkThreads>::kCache;   // 32768 keys
constexpr int kFuCache = TopkShared<kFuThreads>::kCache;   // 8192 keys
// three fused work-groups fit one CU's 160 KiB of LDS
static_assert(3 * sizeof(TopkShared<kFuThreads>) <= 160 * 1024, "fused selection LDS");
// the fused scores keep the page of each 16-key group in the (then unused) candidate list
static_assert(kFuCache / 16 * sizeof(int) <= sizeof(TopkShared<kFuThreads>::cand), "page list");

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
template <bool kKeys, int kThreads>
__device__ __forceinline__ void load8(const void* __restrict__ src, const TopkShared<kThreads>& sh, bool cached,
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

template <int kThreads>
__device__ __forceinline__ uint32_t block_scan(TopkShared<kThreads>& sh, uint32_t v, int buf, uint32_t* total) {
  constexpr int kWaves = TopkShared<kThreads>::kWaves;
  const int lane = lane_id(), wave = wave_id();
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == kWave - 1) sh.wave_sum[buf][wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = sh.wave_sum[buf][w];
    before += (w < wave) ? s : 0u;
    tot += s;
  }
  *total = tot;
  return before + incl;
}

// Largest bin b whose suffix count sum_{b' >= b} hist[b'] reaches `need`; also
// the count strictly above it and the count in it. Ends with a barrier after
// which the histogram is no longer read.
template <int kThreads>
__device__ void select_bin(TopkShared<kThreads>& sh, int nbins, uint32_t need, int buf, uint32_t* bin,
                           uint32_t* above, uint32_t* count) {
  const int tid = threadIdx.x;
  const int per = nbins >= kThreads ? nbins / kThreads : 1;
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
        sh.sel_count = h;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
  *bin = sh.sel_bin;
  *above = sh.sel_above;
  *count = sh.sel_count;
}

enum TopkMode { kWholeRow = 0, kChunk = 1, kMerge = 2, kFused = 3 };

// Fused phase one: the lightning-indexer scores of positions [base, base + n)
// of row t (request b, visible keys `vis`) into the LDS key cache, with the
// first-digit histogram. The contraction is the decode indexer's: lane (c, g)
// of a 16-key group holds bytes [32g, 32g + 32) of head 16m + c of q (A) and
// of key c (B); the 16 relu'd, gated head values of a lane are summed in
// order, then over the four lane groups, then scaled by the key's sigma. A
// wave takes batches of four groups (64 keys), batch j + waves while batch j
// is computed, and after a batch lane (c, g) owns key c of group g. Positions
// on absent pages get -inf, forced (init / local) positions +inf.
template <int kThreads>
__device__ __forceinline__ void fused_scores(const TopkParams& p, TopkShared<kThreads>& sh, int t, int b,
                                             int base, int n, int vis) {
  constexpr int kWaves = TopkShared<kThreads>::kWaves;
  const BatchView& bv = p.batch;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = lane >> 4, c = lane & 15;
  const int P = bv.page_size;
  const int ngroups = (n + 15) >> 4;
  int* gpage = reinterpret_cast<int*>(sh.cand);     // the candidate list is free until the selection
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;
  for (int i = tid; i < kTkBins; i += kThreads) sh.hist[i] = 0;
  for (int i = tid; i < ngroups; i += kThreads) gpage[i] = bt[(base + 16 * i) / P];   // < visible <= pages * P

  // q as four 16-head A operands and the head gates in accumulator order
  // (lane (c, g) holds rows 4g + i of each 16-head tile)
  const uint8_t* qr = p.q8 + (int64_t)t * (kIdxHeads * kIdxDim);
  i32x8 qa[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) qa[m] = *reinterpret_cast<const i32x8*>(qr + (16 * m + c) * kIdxDim + 32 * g);
  float wv[16];
  const float* wrow = p.w + (int64_t)t * kIdxHeads;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 16 * m + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[4 * m + i] = w4[i];
  }
  const int n_init = min(p.num_init, vis);
  const int local0 = max(vis - p.num_local, n_init);  // forced: [0, n_init) and [local0, vis)
  __syncthreads();                                    // page list and cleared histogram

  const int64_t scale_off = (int64_t)P * kIdxDim;
  const int nb = (ngroups + 3) >> 2;                  // batches of four groups
  // Batch j: the key operands of its four groups (groups past the chunk
  // re-read its last group) and, for lane (c, g), the scale and page
  // validity of key c of group g, the key this lane scores.
  auto load = [&](int j, i32x8 (&kb)[4], float& sgl, int& okl) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gi = min(4 * j + u, ngroups - 1);
      const int pid = __builtin_amdgcn_readfirstlane(gpage[gi]);
      const bool okp = pid >= 0 && pid < bv.num_pages;
      const uint8_t* pg = p.cache + (int64_t)(okp ? pid : 0) * p.page_bytes;
      const int slot = (base + 16 * gi) % P + c;     // < P: base and P are multiples of 16
      kb[u] = *reinterpret_cast<const i32x8*>(pg + (int64_t)slot * kIdxDim + 32 * g);
    }
    const int gl = min(4 * j + g, ngroups - 1);
    const int pl = gpage[gl];
    okl = pl >= 0 && pl < bv.num_pages;
    const uint8_t* pg = p.cache + (int64_t)(okl ? pl : 0) * p.page_bytes;
    sgl = *reinterpret_cast<const float*>(pg + scale_off + 4 * ((base + 16 * gl) % P + c));
  };
  // Ring of kFuAhead + 1 slots: batch j0 + r * waves sits in slot r. The
  // slots rotate by name (the inner loop is unrolled), never by register
  // copies: a copy of a register that a load in flight writes would wait for
  // that load. Every prefetch is issued, past the end as a re-read of the
  // last batch: after a conditional load the compiler can no longer count the
  // loads in flight and waits for all of them. Either way the prefetch would
  // stop overlapping the contraction.
  i32x8 kb[kFuAhead + 1][4];
  float sg[kFuAhead + 1];
  int ok[kFuAhead + 1];
#pragma unroll
  for (int d = 0; d < kFuAhead; ++d) load(min(wave + d * kWaves, nb - 1), kb[d], sg[d], ok[d]);
  auto score = [&](int j, const i32x8 (&kbj)[4], float sgj, int okj) {
    float part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      part[u] = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 acc = mfma_fp8_16x16x128(qa[m], kbj[u], zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) part[u] = fmaf(wv[4 * m + i], relu_bits(acc[i]), part[u]);
      }
    }
    // lane (c, g): key c of group g of the batch
    const float v = sum_scatter_over_groups(part[0], part[1], part[2], part[3]);
    const int pos = 16 * (4 * j + g) + c;              // chunk position
    if (pos < n) {
      const int s = base + pos;
      float val = okj ? v * sgj : -INFINITY;
      if (s < n_init || s >= local0) val = INFINITY;
      const uint32_t key = ordered_key(val);
      sh.keys[kslot(pos)] = key;
      atomicAdd(&sh.hist[key >> 20], 1u);
    }
  };
  // The slots of an outer step past the last batch compute on re-read data
  // and store nothing (their positions are past the chunk); skipping them
  // would make the waits above conservative again.
  for (int j0 = wave; j0 < nb; j0 += (kFuAhead + 1) * kWaves) {
#pragma unroll
    for (int r = 0; r <= kFuAhead; ++r) {
      const int j = j0 + r * kWaves;
      const int jl = j + kFuAhead * kWaves;           // into the slot batch j - waves left
      constexpr int kSlots = kFuAhead + 1;
      const int sl = (r + kFuAhead) % kSlots;
      load(min(jl, nb - 1), kb[sl], sg[sl], ok[sl]);
      score(j, kb[r], sg[r], ok[r]);
    }
  }
  __syncthreads();
}

template <int kMode, int kThreads>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkParams p) {
  constexpr bool kKeys = kMode == kMerge;             // the source holds keys, not logits
  constexpr int kWaves = TopkShared<kThreads>::kWaves;
  constexpr int kCache = TopkShared<kThreads>::kCache;
  constexpr int kCand = TopkShared<kThreads>::kCand;
  __shared__ TopkShared<kThreads> sh;
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
  const int64_t cand0 = ((int64_t)t * p.chunks + ((kMode == kChunk || kMode == kFused) ? blockIdx.y : 0)) * k;

  // this selection: elements [0, n) of `src`
  int n = n_row;
  int base = 0;                                       // chunk: position of element 0
  const void* src = p.logits ? p.logits + (int64_t)t * p.stride : nullptr;   // fused: no logits
  if (kMode == kChunk) {
    if (n_row <= k) return;                           // short rows are the merge's
    base = (int)blockIdx.y * p.chunk;
    if (base >= n_row) return;
    n = min(p.chunk, n_row - base);
    src = p.logits + (int64_t)t * p.stride + base;
    if (n <= k) {                                     // the whole chunk is a candidate
      for (int i = tid; i < n; i += kThreads) {
        p.cand_key[cand0 + i] = src_key<false>(src, i);
        p.cand_pos[cand0 + i] = base + i;
      }
      return;
    }
  } else if (kMode == kFused) {
    if (n_row <= k) return;                           // short rows are the merge's
    base = (int)blockIdx.y * p.chunk;
    if (base >= n_row) return;
    n = min(p.chunk, n_row - base);
    fused_scores<kThreads>(p, sh, t, b, base, n, n_row);
    if (n <= k) {                                     // the whole chunk is a candidate
      for (int i = tid; i < n; i += kThreads) {
        p.cand_key[cand0 + i] = sh.keys[kslot(i)];
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
  if (kMode != kFused && n <= k) {  // short row (or as many candidates as winners): every element, in order, then -1
    for (int i = tid; i < k; i += kThreads)
      out[i] = i < n ? (kMode == kMerge && n_row > k ? p.cand_pos[cand0 + i] : i) : -1;
    return;
  }

  const bool cached = kMode == kFused || n <= kCache;
  // ---- level 0 (bits 31..20) while reading the row once (fused: done with the scores) ----
  if (kMode != kFused) {
    for (int i = tid; i < kTkBins; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    const bool vec = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
    const int n4 = vec ? n / 4 : 0;
    for (int i0 = 0; i0 < n4; i0 += kThreads * kTkLoadUnroll) {
      i32x4 v[kTkLoadUnroll];
#pragma unroll
      for (int u = 0; u < kTkLoadUnroll; ++u) {
        int i4 = i0 + u * kThreads + tid;
        i4 = i4 < n4 ? i4 : n4 - 1;               // clamped: always in bounds
        v[u] = static_cast<const i32x4*>(src)[i4];
      }
#pragma unroll
      for (int u = 0; u < kTkLoadUnroll; ++u) {
        const int i4 = i0 + u * kThreads + tid;
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
    for (int i = 4 * n4 + tid; i < n; i += kThreads) {
      const uint32_t kk = src_key<kKeys>(src, i);
      if (cached) sh.keys[kslot(i)] = kk;
      atomicAdd(&sh.hist[kk >> 20], 1u);
    }
    __syncthreads();
  }
  uint32_t need = (uint32_t)k;
  uint32_t bin, above, count;
  select_bin(sh, kTkBins, need, 0, &bin, &above, &count);
  uint32_t prefix = bin;
  need -= above;

  // ---- level 1 (bits 19..8) among keys whose top 12 bits equal the prefix;
  //      those keys are also collected (unordered) for the last level ----
  const bool keep = count <= (uint32_t)kCand;
  for (int i = tid; i < kTkBins; i += kThreads) sh.hist[i] = 0;
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
  // cached selections: masks of the thread's output run [32 tid, 32 tid + 32)
  // with a first digit above the prefix and equal to it, kept for the output
  uint32_t above_run = 0, inbin_run = 0;
  if (cached) {
    // The run's positions first give the two masks; the matches are then
    // handled in rounds of one per lane, so the rounds of the whole pass
    // number the most matches of one lane.
    const int r0 = kTkRun * tid;
    uint32_t mm = 0;
    if (r0 < n) {
#pragma unroll
      for (int q = 0; q < kTkRun / 4; ++q) {
        const i32x4 a = *reinterpret_cast<const i32x4*>(sh.keys + kslot(r0 + 4 * q));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool valid = r0 + 4 * q + e < n;
          const uint32_t d = (uint32_t)a[e] >> 20;
          mm |= (valid && d == prefix ? 1u : 0u) << (4 * q + e);
          above_run |= (valid && d > prefix ? 1u : 0u) << (4 * q + e);
        }
      }
    }
    inbin_run = mm;
    while (__ballot(mm != 0u)) {
      const bool m = mm != 0u;
      uint32_t x = 0;
      if (m) {
        const int e = __builtin_ctz(mm);
        mm &= mm - 1u;
        x = sh.keys[kslot(r0 + e)];
      }
      take_match(m, x);
    }
  }
  for (int i = kTkPer * tid; !cached && i < n; i += kTkPer * kThreads) {
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
  select_bin(sh, kTkBins, need, 1, &bin, &above, &count);
  prefix = (prefix << 12) | bin;
  need -= above;
  const uint32_t count24 = count;                      // keys sharing the top 24 bits with the k-th

  // ---- level 2 (bits 7..0) among keys whose top 24 bits equal the prefix ----
  bool kept = keep;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) kept = kept && sh.wave_cand[w] <= (uint32_t)kTkCandPerWave;
  uint32_t thr;
  if (kept && count24 <= (uint32_t)kWave) {
    // Few keys share the top 24 bits (the usual case): gather them from the
    // candidate lists into the histogram area (free since the last selection),
    // then every wave finds the need-th largest by ranking them, one lane per
    // key, with no further barrier.
    uint32_t* few = sh.hist;
    const uint32_t nc = sh.wave_cand[wave];            // wave w scans wave w's slots
    for (uint32_t i = lane_id(); i < nc; i += kWave) {
      const uint32_t u = sh.cand[wave * kTkCandPerWave + i];
      if ((u >> 8) == prefix) few[atomicAdd(&sh.n_cand, 1u)] = u;
    }
    __syncthreads();
    const uint32_t lane = (uint32_t)lane_id();
    const uint32_t mine = lane < count24 ? few[lane] : 0u;
    uint32_t gt = 0, ge = 0;                           // keys of the bin above / not below mine
    for (uint32_t j = 0; j < count24; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mine, (int)j);
      gt += kj > mine ? 1u : 0u;
      ge += kj >= mine ? 1u : 0u;
    }
    const uint64_t hit = __ballot(lane < count24 && gt < need && need <= ge);   // lanes holding the k-th key
    const int src_lane = (int)__builtin_ctzll(hit);
    thr = (uint32_t)__builtin_amdgcn_readlane((int)mine, src_lane);
    need -= (uint32_t)__builtin_amdgcn_readlane((int)gt, src_lane);
  } else {
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0;
    __syncthreads();
    if (kept) {
      const uint32_t nc = sh.wave_cand[wave];          // wave w scans wave w's slots
      for (uint32_t i = lane_id(); i < nc; i += kWave) {
        const uint32_t u = sh.cand[wave * kTkCandPerWave + i];
        if ((u >> 8) == prefix) atomicAdd(&sh.hist[u & 0xffu], 1u);
      }
    } else {
      for (int i = kTkPer * tid; i < n; i += kTkPer * kThreads) {
        uint32_t u[kTkPer];
        load8<kKeys>(src, sh, cached, n, i, u);
#pragma unroll
        for (int e = 0; e < kTkPer; ++e)
          if (i + e < n && (u[e] >> 8) == prefix) atomicAdd(&sh.hist[u[e] & 0xffu], 1u);
      }
    }
    __syncthreads();
    select_bin(sh, 256, need, 0, &bin, &above, &count);
    thr = (prefix << 8) | bin;
    need -= above;
  }
  // need: how many keys equal to thr are among the winners (>= 1)

  // ---- ordered output ----
  // A winner at position p goes to slot #winners before p = (#keys > thr before
  // p) + min(#keys == thr before p, need). Thread tid owns a run of
  // consecutive positions, handled 32 at a time as bit masks: count its winners,
  // one block-wide scan, then place them in order.
  const int run_len = cached ? kTkRun : ((n + kThreads - 1) / kThreads + 31) & ~31;
  const int run0 = run_len * tid;
  // masks of the keys > thr and == thr among positions [p0, p0 + 32)
  auto masks32 = [&](int p0, uint32_t* gtm, uint32_t* eqm) {   // selections read from memory
    uint32_t key[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t u[kTkPer];
      load8<kKeys>(src, sh, false, n, p0 + 8 * j, u);
#pragma unroll
      for (int e = 0; e < kTkPer; ++e) key[8 * j + e] = u[e];
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
  if (cached) {
    // positions with a first digit above the prefix are above thr; only the
    // run's positions in the prefix bin are compared with thr
    gtm0 = above_run;
    uint32_t rest = inbin_run;
    while (rest) {
      const int e = __builtin_ctz(rest);
      rest &= rest - 1u;
      const uint32_t key = sh.keys[kslot(run0 + e)];
      gtm0 |= (key > thr ? 1u : 0u) << e;
      eqm0 |= (key == thr ? 1u : 0u) << e;
    }
    cgt = (uint32_t)__builtin_popcount(gtm0);
    ceq = (uint32_t)__builtin_popcount(eqm0);
  } else {
    for (int p0 = run0; p0 < run0 + run_len && p0 < n; p0 += 32) {
      uint32_t gtm, eqm;
      masks32(p0, &gtm, &eqm);
      cgt += (uint32_t)__builtin_popcount(gtm);
      ceq += (uint32_t)__builtin_popcount(eqm);
    }
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
  for (int i = tid; i < k; i += kThreads) {
    const int e = (int)sh.hist[i];
    if (kMode == kWholeRow) {
      out[i] = e;
    } else if (kMode == kChunk || kMode == kFused) {
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
    hipLaunchKernelGGL(HIP_KERNEL_NAME(topk_kernel<kWholeRow, kTkThreads>), dim3(p.batch.num_rows), dim3(kTkThreads),
                       0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(HIP_KERNEL_NAME(topk_kernel<kChunk, kTkThreads>), dim3(p.batch.num_rows, p.chunks),
                     dim3(kTkThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(HIP_KERNEL_NAME(topk_kernel<kMerge, kTkThreads>), dim3(p.batch.num_rows), dim3(kTkThreads),
                     0, s, p);
  return hipGetLastError();
}

int indexer_topk_chunk(int num_rows, int max_len, int k) {
  // Chunks fill the fused work-group's key cache (8192 keys). With k at most a
  // quarter of that, chunks of 4096 when 8192 would leave fewer than two
  // work-groups per CU: phase one then spreads over more CUs, for twice the
  // candidates per chunk's keys, as long as a row's candidates still fit the
  // merge's LDS key cache. A chunk is never shorter than k, so every chunk but
  // a row's last gives exactly k candidates.
  const int64_t wgs = (int64_t)num_rows * ((max_len + kFuCache - 1) / kFuCache);
  const int64_t cands_half = (int64_t)((max_len + kFuCache / 2 - 1) / (kFuCache / 2)) * k;
  if (4 * k <= kFuCache && wgs < 512 && cands_half <= kTkCache) return kFuCache / 2;
  return kFuCache;
}

size_t indexer_topk_workspace_bytes(int num_rows, int max_len, int k) {
  const int chunk = indexer_topk_chunk(num_rows, max_len, k);
  const int chunks = (max_len + chunk - 1) / chunk;
  return (size_t)num_rows * chunks * k * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_indexer_topk(const TopkParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  if (p.chunks > 0) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(topk_kernel<kFused, kFuThreads>), dim3(p.batch.num_rows, p.chunks),
                       dim3(kFuThreads), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(HIP_KERNEL_NAME(topk_kernel<kMerge, kTkThreads>), dim3(p.batch.num_rows), dim3(kTkThreads),
                     0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
