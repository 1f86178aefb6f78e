// Lightning-indexer scores over a paged fp8 index-K cache.
//
//   logits[t, s] = sum_h w[t, h] * relu(sigma_s * (q[t, h] . k_s))
//
// (SGLang "dsa_indexer.py" page: Indexer._get_topk_paged feeds q_fp8 [T, 64, 128],
// the 132-byte-per-token paged cache, weights [T, 64] and the block table to the
// paged MQA-logits kernel; forward_indexer gives the same score per request.)
//
// fp8 path (H = 64, D = 128): the q . k contraction runs on the gfx950 fp8 MFMA
// v_mfma_f32_16x16x128_f8f6f4 (no block scales). Heads are the M
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
  // format 0 = fp8 e4m3 for both operands, no block scales: all-zero scale
  // operands select the unscaled v_mfma_f32_16x16x128_f8f6f4, which computes
  // the plain fp8 product (the same values as unit E8M0 scales) and lets the
  // wave issue independent VALU work under it far better than the scaled form.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// relu as an integer max with 0 on the float's bits (negative floats are
// negative integers): one VALU op, no NaN quieting as fmaxf needs
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// sum of v over lanes l, l ^ 16, l ^ 32, l ^ 48, with the gfx950 lane swaps (VALU, no LDS)
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
      for (int i = 0; i < 4; ++i) part = fmaf(wv[4 * m + i], relu_bits(acc[i]), part);
    }
    part += shfl_xor_f(part, 16);
    part += shfl_xor_f(part, 32);
    const int s = s0 + c;
    if (g == 0 && s < k_end) out[s] = ok[u] ? part * sig[u] : -INFINITY;
  }
}

// Decode rows (one query row per request): a streaming variant. The keys of
// all rows are cut into groups of 16 (row t has ceil(visible_t / 16) groups);
// every wave of a fixed grid takes an equal contiguous share of the flattened
// group list, whatever the row lengths, and walks it in batches of up to four
// groups inside one page. The batch list of a wave is built once (lane j holds
// batch j's row, first group, count, page and row length; all page lookups in
// one vector load), then the wave streams: the loads of batch j + 1 are issued
// before the MFMAs of batch j. q and the head weights are reloaded when the
// row changes (once or twice per wave). Every wave is independent: no barrier
// after the row prefix sums.
constexpr int kStreamThreads = 256;
constexpr int kStreamWaves = kStreamThreads / kWave;
constexpr int kStreamMaxRows = 1024;
constexpr int kStreamBatch = 4;                                  // groups per batch

struct StreamBatch {
  int t, gi, cnt;
};

__global__ __launch_bounds__(kStreamThreads) void indexer_fp8_stream_kernel(IndexerParams p) {
  __shared__ int pre[kStreamMaxRows + 1];                        // group prefix over rows
  __shared__ int wsum[kStreamWaves];
  const BatchView& bv = p.batch;
  const int T = bv.num_rows;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = lane >> 4, c = lane & 15;
  const int P = bv.page_size;
  const int gpp = P / 16;                                        // groups per page
  int cap = bv.max_pages_per_seq * P;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;

  // ---- groups per row and their prefix sums ----
  int carry = 0;
  for (int base = 0; base < T; base += kStreamThreads) {
    const int t = base + tid;
    const int vis = t < T ? visible_keys(bv.seq_lens_k[t], 1, 0, cap) : 0;
    const int cnt = (vis + 15) >> 4;
    const int incl = (int)wave_inclusive_scan((uint32_t)cnt);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) {
      const int v = wsum[w];
      before += (w < wave) ? v : 0;
      tot += v;
    }
    if (t < T) pre[t + 1] = carry + before + incl;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) pre[0] = 0;
  __syncthreads();

  const int N = pre[T];
  const int W = gridDim.x * kStreamWaves;
  const int wg = blockIdx.x * kStreamWaves + wave;
  int a = (int)((int64_t)N * wg / W);
  const int a_end = (int)((int64_t)N * (wg + 1) / W);
  if (a >= a_end) return;
  // row of group a: the largest t with pre[t] <= a (rows without groups are passed over)
  int t = 0;
  {
    int lo = 0, hi = T - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= a) lo = mid; else hi = mid - 1;
    }
    t = lo;
  }
  t = __builtin_amdgcn_readfirstlane(t);
  int gi = a - pre[t];
  gi = __builtin_amdgcn_readfirstlane(gi);

  const int64_t scale_off = (int64_t)P * kIdxDim;
  const uint8_t* cache = p.cache;
  while (a < a_end) {
    // ---- batch list (up to 64 batches): lane j holds batch j ----
    int bt_t = 0, bt_gi = 0, bt_cnt = 0, nb = 0;
    while (a < a_end && nb < kWave) {
      int n_t = pre[t + 1] - pre[t];
      while (gi >= n_t) {                                        // next row with groups
        ++t;
        gi = 0;
        n_t = pre[t + 1] - pre[t];
      }
      int gend = (gi / gpp + 1) * gpp;
      gend = min(gend, gi + kStreamBatch);
      gend = min(gend, n_t);
      gend = min(gend, gi + (a_end - a));
      if (lane == nb) { bt_t = t; bt_gi = gi; bt_cnt = gend - gi; }
      a += gend - gi;
      gi = gend;
      ++nb;
    }
    // pages and row lengths of every batch in one go
    int bt_page = -1, bt_vis = 0;
    if (lane < nb) {
      const int pi = bt_gi / gpp;
      bt_page = bv.block_table[(int64_t)bt_t * bv.max_pages_per_seq + pi];
      bt_vis = visible_keys(bv.seq_lens_k[bt_t], 1, 0, cap);
    }

    auto batch_of = [&](int j, int* bt, int* bg, int* bc, int* bp, int* bvv) {
      *bt = __builtin_amdgcn_readlane(bt_t, j);
      *bg = __builtin_amdgcn_readlane(bt_gi, j);
      *bc = __builtin_amdgcn_readlane(bt_cnt, j);
      *bp = __builtin_amdgcn_readlane(bt_page, j);
      *bvv = __builtin_amdgcn_readlane(bt_vis, j);
    };
    // key operands (lane (c, g): key 16u + c of the batch, bytes [32g, 32g + 32)) and scales
    auto load_batch = [&](int bg, int bc, int bp, i32x8 (&kb)[kStreamBatch], float (&sg)[kStreamBatch]) {
      const bool okp = bp >= 0 && bp < bv.num_pages;
      const uint8_t* pg = cache + (int64_t)(okp ? bp : 0) * p.page_bytes;
#pragma unroll
      for (int u = 0; u < kStreamBatch; ++u) {
        const int uu = u < bc ? u : 0;                           // past the batch: re-read group 0
        const int slot = (16 * (bg + uu)) % P + c;
        kb[u] = *reinterpret_cast<const i32x8*>(pg + (int64_t)slot * kIdxDim + 32 * g);
        sg[u] = *reinterpret_cast<const float*>(pg + scale_off + 4 * slot);
      }
    };

    i32x8 qa[4];
    float wv[16];
    int q_row = -1;
    auto load_row = [&](int rt) {
      const uint8_t* qr = static_cast<const uint8_t*>(p.q) + (int64_t)rt * (kIdxHeads * kIdxDim);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        qa[m] = *reinterpret_cast<const i32x8*>(qr + (16 * m + c) * kIdxDim + 32 * g);
      const float* wrow = p.w + (int64_t)rt * kIdxHeads;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 16 * m + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[4 * m + i] = w4[i];
      }
      q_row = rt;
    };

    // one batch in flight ahead of the one being computed
    int ct, cg, cc, cp, cv;
    batch_of(0, &ct, &cg, &cc, &cp, &cv);
    i32x8 k0[kStreamBatch];
    float s0[kStreamBatch];
    load_batch(cg, cc, cp, k0, s0);
    load_row(ct);
    for (int j = 0; j < nb; ++j) {
      int nt_ = 0, ng = 0, nc = 0, np = -1, nv = 0;
      i32x8 k1[kStreamBatch];
      float s1[kStreamBatch];
      const bool more = j + 1 < nb;
      if (more) {
        batch_of(j + 1, &nt_, &ng, &nc, &np, &nv);
        load_batch(ng, nc, np, k1, s1);
      }
      if (ct != q_row) load_row(ct);
      // ---- logits of batch j ----
      const bool okp = cp >= 0 && cp < bv.num_pages;
      float* out = p.logits + (int64_t)ct * p.stride;
#pragma unroll
      for (int u = 0; u < kStreamBatch; ++u) {
        if (u >= cc) break;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 acc = mfma_fp8_16x16x128(qa[m], k0[u], zero);
#pragma unroll
          for (int i = 0; i < 4; ++i) part = fmaf(wv[4 * m + i], relu_bits(acc[i]), part);
        }
        part += shfl_xor_f(part, 16);
        part += shfl_xor_f(part, 32);
        const int s = 16 * (cg + u) + c;
        if (g == 0 && s < cv) out[s] = okp ? part * s0[u] : -INFINITY;
      }
      if (!more) break;
      ct = nt_; cg = ng; cc = nc; cp = np; cv = nv;
#pragma unroll
      for (int u = 0; u < kStreamBatch; ++u) { k0[u] = k1[u]; s0[u] = s1[u]; }
    }
  }
}

// Prefill rows (cu_seqlens given, up to 1024 requests): MFMA-bound, so the
// work-group is a tile of 8 query rows of one request x 2048 keys. Keys stream
// through a two-slot LDS ring in stages of 256 (16 groups of 16, copied with
// global_load_lds; every wave copies four groups and their 64 scales); each
// wave holds the q of two rows in registers and runs every key group against
// both, so one LDS operand read feeds eight MFMAs. Inside a group the 16-byte
// chunk x of key c sits at chunk 16x + c: the sixteen keys' chunk x are one
// contiguous 256 B run, which the operand reads take at the linear LDS rate.
// The MFMA contraction order inside a lane group is free as long as both
// operands use the same one: lane (c, g) holds bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of its head (A) and of its key (B).
//
// Per 16-key group and row the epilogue (relu, head weight, head sum) costs
// about as many VALU cycles as the four MFMAs, so the group loop is software
// pipelined: the MFMAs of group i+1 are interleaved with the epilogue of
// group i, whose results they do not touch. relu is an integer max with 0 on
// the float's bits (negative floats are negative integers), which needs no NaN
// quieting. The two rows' head sums share one pair of lane swaps: after them
// lane group g holds row g & 1's total.
constexpr int kPfThreads = 256;
constexpr int kPfWaves = kPfThreads / kWave;                     // 4
constexpr int kPfRowsW = 2;                                      // query rows per wave
constexpr int kPfRows = kPfWaves * kPfRowsW;                     // 8 rows per work-group
constexpr int kPfStageGroups = 16;                               // 16-key groups per stage
constexpr int kPfStageKeys = 16 * kPfStageGroups;                // 256
constexpr int kPfChunk = 2048;                                   // keys per work-group
constexpr int kPfStages = kPfChunk / kPfStageKeys;               // 8
constexpr int kPfChunkGroups = kPfChunk / 16;                    // 128
constexpr int kPfMaxSeqs = 1024;
constexpr int64_t kPfMaxStride = 1 << 26;                        // two rows' bytes stay below 2^31

struct PfShared {
  alignas(16) uint8_t keys[2][kPfStageGroups][16 * kIdxDim];   // 2 x 32 KB
  alignas(16) float scale[2][kPfStageKeys];                      // 2 x 1 KB
  alignas(16) int gpage[kPfChunkGroups];                         // page of each group, -1 = masked
  int blk[kPfMaxSeqs + 1];                                       // row-block prefix over requests
  int wsum[kPfWaves];
};

// 4 bytes per lane from global memory straight into LDS at M0 + 4 l.
__device__ __forceinline__ void lds_dma4(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gsrc), "s"(lds_addr) : "memory", "m0");
}

__global__ __launch_bounds__(kPfThreads) void indexer_fp8_prefill_kernel(IndexerParams p) {
  __shared__ PfShared sh;
  const BatchView& bv = p.batch;
  const int B = bv.num_seqs;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = lane >> 4, c = lane & 15;
  const int P = bv.page_size;

  // ---- row blocks of 8 per request, prefix over requests ----
  int carry = 0;
  for (int base = 0; base < B; base += kPfThreads) {
    const int b = base + tid;
    const int ql = b < B ? bv.cu_seqlens_q[b + 1] - bv.cu_seqlens_q[b] : 0;
    const int cnt = ql > 0 ? (ql + kPfRows - 1) / kPfRows : 0;
    const int incl = (int)wave_inclusive_scan((uint32_t)cnt);
    if (lane == kWave - 1) sh.wsum[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) {
      const int v = sh.wsum[w];
      before += (w < wave) ? v : 0;
      tot += v;
    }
    if (b < B) sh.blk[b + 1] = carry + before + incl;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) sh.blk[0] = 0;
  __syncthreads();
  const int x = blockIdx.x;
  if (x >= sh.blk[B]) return;
  int b = 0;
  {
    int lo = 0, hi = B - 1;                                      // largest b with blk[b] <= x
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.blk[mid] <= x) lo = mid; else hi = mid - 1;
    }
    b = lo;
  }
  const int q0 = bv.cu_seqlens_q[b];
  const int q_len = bv.cu_seqlens_q[b + 1] - q0;
  const int j0 = (x - sh.blk[b]) * kPfRows;                      // first row of the block inside the request
  int cap = bv.max_pages_per_seq * P;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int seq_len = bv.seq_lens_k[b];
  const int last = min(j0 + kPfRows, q_len) - 1;
  const int vis_max = visible_keys(seq_len, q_len, last, cap);  // the block's last row sees the most keys
  const int k0 = blockIdx.y * kPfChunk;
  if (k0 >= vis_max) return;
  const int n_stages = min(kPfStages, (vis_max - k0 + kPfStageKeys - 1) / kPfStageKeys);
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;
  const int64_t scale_off = (int64_t)P * kIdxDim;

  // page of every 16-key group of the chunk (P is a multiple of 16, so a
  // group never straddles pages); -1 past the last visible key or for a page
  // id outside the cache
  if (tid < kPfChunkGroups) {
    const int key0 = k0 + 16 * tid;
    int pg = bt[min(key0, cap - 1) / P];
    pg = (key0 < vis_max && pg >= 0 && pg < bv.num_pages) ? pg : -1;
    sh.gpage[tid] = pg;
  }

  // this wave's two rows: q operands, head weights, visible keys
  i32x8 qa[kPfRowsW][4];
  float wv[kPfRowsW][16];
  int vis[kPfRowsW];
#pragma unroll
  for (int r = 0; r < kPfRowsW; ++r) {
    const int j = min(j0 + kPfRowsW * wave + r, q_len - 1);     // rows past the request repeat its last row
    vis[r] = (j0 + kPfRowsW * wave + r < q_len) ? visible_keys(seq_len, q_len, j, cap) : 0;
    const int t = q0 + j;
    const uint8_t* qr = static_cast<const uint8_t*>(p.q) + (int64_t)t * (kIdxHeads * kIdxDim);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(qr + (16 * m + c) * kIdxDim + 16 * g);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(qr + (16 * m + c) * kIdxDim + 64 + 16 * g);
      qa[r][m] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    const float* wrow = p.w + (int64_t)t * kIdxHeads;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 16 * m + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[r][4 * m + i] = w4[i];
    }
  }
  // Output: lane group g < 2 stores row g of the wave through a buffer
  // resource over the wave's two rows; out-of-range offsets drop the store.
  constexpr uint32_t kDrop = 0x80000000u;
  const int64_t row_w = (int64_t)q0 + j0 + kPfRowsW * wave;      // may lie past the batch: then vis = 0
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      p.logits + row_w * p.stride, (short)0, (int)(2 * p.stride * 4), 0x00020000);
  const int vis_g = g == 0 ? vis[0] : (g == 1 ? vis[1] : 0);
  const uint32_t row_off = (uint32_t)(g & 1) * (uint32_t)p.stride * 4u;

  // copies of stage st into slot st & 1: wave w copies groups 4w .. 4w+3
  // (two 1 KB copies each; copy h: lane l fetches chunk (64h + l) >> 4 of key
  // (64h + l) & 15) and their scales (lane l: key l & 15 of group 4w + l / 16)
  const uint8_t* cache = p.cache;
  auto issue_stage = [&](int st) {
    const int gb = st * kPfStageGroups + 4 * wave;               // first group of this wave in the chunk
    const i32x4 pg4 = *reinterpret_cast<const i32x4*>(&sh.gpage[gb]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key0 = k0 + 16 * (gb + u);
      const int pg = max(pg4[u], 0);                             // masked groups copy page 0; not stored
      const uint8_t* src = cache + (int64_t)pg * p.page_bytes + (int64_t)(key0 % P) * kIdxDim;
      const uint32_t dst = lds_offset(sh.keys[st & 1][4 * wave + u]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int L = 64 * h + lane;
        lds_dma16(src + (L & 15) * kIdxDim + 16 * (L >> 4), dst + 1024 * h);
      }
    }
    const int my = max(sh.gpage[gb + g], 0);
    const int key0 = k0 + 16 * (gb + g);
    lds_dma4(cache + (int64_t)my * p.page_bytes + scale_off + 4 * (key0 % P + c),
             lds_offset(&sh.scale[st & 1][64 * wave]));
  };

  const int kof0 = (16 * g + c) * 16;                           // chunk g of key c
  const int kof1 = (16 * (g + 4) + c) * 16;                     // chunk g + 4 of key c
  __syncthreads();                                               // page table visible
  issue_stage(0);
  if (n_stages > 1) issue_stage(1);
  // Consume q and the weights only now: their loads overlap the page lookups
  // and the first copies, and no compiler-placed vector-memory wait inside the
  // loop drains the (to the compiler invisible) copies.
#pragma unroll
  for (int r = 0; r < kPfRowsW; ++r) {
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" :: "v"(qa[r][m]));
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" :: "v"(wv[r][i]));
  }
  wait_vmcnt<0>();
  __syncthreads();

  // One software pipeline over all groups of the chunk: iteration i issues
  // the MFMAs of group i + 1 and runs the epilogue of group i. The stage
  // boundary sits in the last iteration of a stage, before the MFMAs of the
  // next stage's first group: wait for the next stage's copies, barrier (every
  // wave has read this stage's operands and scales), then start the copies of
  // the stage after into the slot just released. Vector-memory operations
  // complete in issue order, so the copies issued at the previous boundary are
  // done once at most the stores issued since (one per iteration, at least 15)
  // are outstanding.
  auto read_kb = [&](int slot, int grp) -> i32x8 {
    const uint8_t* kg = sh.keys[slot][grp];
    const i32x4 lo = *reinterpret_cast<const i32x4*>(kg + kof0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(kg + kof1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  f32x4 acc[2][kPfRowsW][4];
  auto mfmas = [&](f32x4 (&a)[kPfRowsW][4], const i32x8& kb) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kPfRowsW; ++r)
#pragma unroll
      for (int m = 0; m < 4; ++m) a[r][m] = mfma_fp8_16x16x128(qa[r][m], kb, zero);
  };
  i32x8 kb_next = read_kb(0, 1);
  mfmas(acc[0], read_kb(0, 0));
  __builtin_amdgcn_sched_barrier(0);
  for (int st = 0; st < n_stages; ++st) {
    const int slot = st & 1;
    const int kst = k0 + st * kPfStageKeys;
    const uint64_t valid = __ballot(lane < kPfStageGroups && sh.gpage[st * kPfStageGroups + c] >= 0);
    const int lim = vis_g - kst - c;                             // store key 16 i + c of the stage iff 16 i < lim
    const uint32_t off0 = row_off + 4u * (uint32_t)(kst + c);
#pragma unroll
    for (int grp = 0; grp < kPfStageGroups; ++grp) {
      const float sg = sh.scale[slot][16 * grp + c];
      i32x8 kb_after;
      if (grp + 2 < kPfStageGroups) {
        kb_after = read_kb(slot, grp + 2);
        mfmas(acc[(grp + 1) & 1], kb_next);
      } else if (grp + 2 == kPfStageGroups) {
        mfmas(acc[(grp + 1) & 1], kb_next);
      } else {
        // stage boundary (on the last stage the next-group MFMAs run on a
        // stale slot and are never used)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");      // own reads of this slot done
        wait_vmcnt<15>();
        __syncthreads();
        if (st + 2 < n_stages) issue_stage(st + 2);
        kb_next = read_kb(slot ^ 1, 1);
        mfmas(acc[0], read_kb(slot ^ 1, 0));
      }
      const f32x4 (&a)[kPfRowsW][4] = acc[grp & 1];
      float part[kPfRowsW];
#pragma unroll
      for (int r = 0; r < kPfRowsW; ++r) {
        float sum = wv[r][0] * relu_bits(a[r][0][0]);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = (m == 0 ? 1 : 0); i < 4; ++i) sum = fmaf(wv[r][4 * m + i], relu_bits(a[r][m][i]), sum);
        part[r] = sum;
      }
      // lane swaps: rows 0/1 of groups (0,1) and (2,3), then the halves
      const auto sw16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                         false, false);
      const float h = __uint_as_float(sw16[0]) + __uint_as_float(sw16[1]);
      const auto sw32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(h), __float_as_uint(h), false, false);
      const float tot = (__uint_as_float(sw32[0]) + __uint_as_float(sw32[1])) * sg;
      const float val = ((valid >> grp) & 1) ? tot : -INFINITY;
      const uint32_t off = (16 * grp < lim) ? off0 : kDrop;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val), out_rsrc, (int)(off + 64u * grp), 0, 0);
      if (grp + 2 < kPfStageGroups) kb_next = kb_after;
      // issue order: operand reads, then each MFMA followed by a slice of the epilogue
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < 2 * 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 9, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();
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
  if (p.batch.cu_seqlens_q == nullptr && p.batch.num_rows <= kStreamMaxRows) {
    // about 32 groups per wave, at most three work-groups per CU (one round)
    const int64_t groups = (int64_t)p.batch.num_rows * ((p.batch.max_seq_len_k + 15) / 16);
    int64_t wgs = (groups / 32 + kStreamWaves - 1) / kStreamWaves;
    if (wgs > 768) wgs = 768;
    if (wgs < 1) wgs = 1;
    hipLaunchKernelGGL(indexer_fp8_stream_kernel, dim3((unsigned)wgs), dim3(kStreamThreads), 0, s, p);
    return hipGetLastError();
  }
  if (p.batch.cu_seqlens_q != nullptr && p.batch.num_seqs <= kPfMaxSeqs && p.stride <= kPfMaxStride) {
    // row blocks: sum over requests of ceil(q_len / 8) <= num_rows / 8 + num_seqs
    const int blocks = (p.batch.num_rows + kPfRows - 1) / kPfRows + p.batch.num_seqs;
    dim3 grid(blocks, (p.batch.max_seq_len_k + kPfChunk - 1) / kPfChunk);
    hipLaunchKernelGGL(indexer_fp8_prefill_kernel, grid, dim3(kPfThreads), 0, s, p);
    return hipGetLastError();
  }
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
