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
#include <atomic>

#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kIdxWaves = 4;
constexpr int kIdxGroupsPerWave = 8;                               // 16 keys each
constexpr int kIdxChunk = 16 * kIdxGroupsPerWave * kIdxWaves;      // 512 keys per work-group

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
    part = sum_over_groups(part);
    const int s = s0 + c;
    if (g == 0 && s < k_end) out[s] = ok[u] ? part * sig[u] : -INFINITY;
  }
}

// Decode rows: a streaming variant. A unit is what shares one key stream: a
// request's single row (plain decode), or up to two consecutive rows of one
// request (multi-token decode, where a request carries next_n <= 4 rows and
// row i sees one key more than row i - 1; the SGLang indexer page scores the
// next_n rows of a request against the same paged keys). The keys of every
// unit are cut into groups of 16 (ceil(visible / 16) for its last row), and
// the groups into chunks: up to four groups inside one page. Every work-group
// (one per CU) takes an equal contiguous share of the flattened chunk list,
// whatever the lengths, writes a record per chunk into LDS (unit, first group,
// count, page, rows and their lengths; all page lookups at once), and its
// waves then take chunks one at a time from an LDS counter, so that the waves
// a CU issues first (which run ahead) take more of them and the CU's waves
// finish together. A wave issues the loads of its next chunk before the MFMAs
// of the current one, and each key group meets the q of every row of its
// unit; q and the head weights are reloaded when the unit changes. After the
// MFMAs of a chunk the four groups' head sums are reduce-scattered over the
// lane groups, so each row gets one 64-lane store per chunk.
constexpr int kStreamMaxUnits = 1024;
constexpr int kStreamBatch = 4;                                  // groups per chunk
constexpr int kStreamMaxQLen = 4;                                // rows per request, multi-row units
constexpr int kStreamMaxChunks = 1024;                           // chunk records per round
constexpr int kDecodeAhead = 1;                                  // chunks in flight per wave (decode)
constexpr int64_t kStreamMaxStride = 1LL << 29;                  // logits row bytes stay below 2^31

// Waves per work-group: as many as the registers let one CU hold
template <int kR, int kAhead> constexpr int stream_waves() { return kR == 1 && kAhead == 1 ? 12 : 8; }

// Unit u of a stream launch with kR rows per unit. kR = 1: unit u is decode
// row u. kR = 2: unit u is rows 2 (u & 1) and 2 (u & 1) + 1 of request u >> 1
// (those that exist). Returns the rows' request, first row, count and the
// visible keys of its first and last row.
template <int kR>
__device__ __forceinline__ void stream_unit(const BatchView& bv, int u, int cap, int* b, int* r0, int* nr,
                                            int* vis_first, int* vis_last) {
  if (kR == 1) {
    *b = u;
    *r0 = u;
    *nr = 1;
    *vis_first = *vis_last = visible_keys(bv.seq_lens_k[u], 1, 0, cap);
    return;
  }
  const int req = u >> 1, half = u & 1;
  const int c0 = bv.cu_seqlens_q[req];
  const int q_len = bv.cu_seqlens_q[req + 1] - c0;
  int n = q_len - 2 * half;
  n = n < 0 ? 0 : (n > 2 ? 2 : n);
  *b = req;
  *r0 = c0 + 2 * half;
  *nr = n;
  const int len = bv.seq_lens_k[req];
  *vis_first = n > 0 ? visible_keys(len, q_len, 2 * half, cap) : 0;
  *vis_last = n > 0 ? visible_keys(len, q_len, 2 * half + n - 1, cap) : 0;
}

// chunks of a unit with n groups, gpp groups per page and cpp chunks per full page
__device__ __forceinline__ int stream_chunks(int n, int gpp, int cpp) {
  return (n / gpp) * cpp + (n % gpp + kStreamBatch - 1) / kStreamBatch;
}

template <int kR, int kAhead>
__global__ __launch_bounds__((stream_waves<kR, kAhead>() * kWave)) void indexer_fp8_stream_kernel(IndexerParams p) {
  constexpr int kWaves = stream_waves<kR, kAhead>();
  constexpr int kThreads = kWaves * kWave;
  __shared__ int pre[kStreamMaxUnits + 1];                       // chunk prefix over units
  __shared__ int wsum[kWaves];
  __shared__ int4 rec_a[kStreamMaxChunks];                       // unit, first group, groups, page
  __shared__ int4 rec_b[kStreamMaxChunks];                       // first row, rows, visible keys of first / last row
  __shared__ int next_chunk;
  const BatchView& bv = p.batch;
  const int U = kR == 1 ? bv.num_rows : 2 * bv.num_seqs;         // units
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = lane >> 4, c = lane & 15;
  const int P = bv.page_size;
  const int gpp = P / 16;                                        // groups per page
  const int cpp = (gpp + kStreamBatch - 1) / kStreamBatch;       // chunks per full page
  int cap = bv.max_pages_per_seq * P;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;

  // ---- chunks per unit and their prefix sums ----
  int carry = 0;
  for (int base = 0; base < U; base += kThreads) {
    const int u = base + tid;
    int cnt = 0;
    if (u < U) {
      int b_, r0_, nr_, vf_, vl_;
      stream_unit<kR>(bv, u, cap, &b_, &r0_, &nr_, &vf_, &vl_);
      cnt = stream_chunks((vl_ + 15) >> 4, gpp, cpp);
    }
    const int incl = (int)wave_inclusive_scan((uint32_t)cnt);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int v = wsum[w];
      before += (w < wave) ? v : 0;
      tot += v;
    }
    if (u < U) pre[u + 1] = carry + before + incl;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) pre[0] = 0;
  __syncthreads();

  const int C = pre[U];
  const int c_begin = (int)((int64_t)C * blockIdx.x / gridDim.x);
  const int c_end = (int)((int64_t)C * (blockIdx.x + 1) / gridDim.x);

  const int64_t scale_off = (int64_t)P * kIdxDim;
  const uint8_t* cache = p.cache;

  struct Batch { int t, gi, cnt, page, r0, nr, vf, vl; };
  auto record = [&](int j) {                                     // chunk j of the round, wave-uniform
    const int4 a = rec_a[j];
    const int4 b = rec_b[j];
    Batch x;
    x.t = __builtin_amdgcn_readfirstlane(a.x);
    x.gi = __builtin_amdgcn_readfirstlane(a.y);
    x.cnt = __builtin_amdgcn_readfirstlane(a.z);
    x.page = __builtin_amdgcn_readfirstlane(a.w);
    x.r0 = __builtin_amdgcn_readfirstlane(b.x);
    x.nr = kR == 1 ? 1 : __builtin_amdgcn_readfirstlane(b.y);
    x.vf = __builtin_amdgcn_readfirstlane(b.z);
    x.vl = kR == 1 ? x.vf : __builtin_amdgcn_readfirstlane(b.w);
    return x;
  };
  auto take = [&]() {                                            // next chunk of the round, wave-uniform
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_chunk, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  // key operands (lane (c, g): key 16u + c of the chunk, bytes [32g, 32g + 32))
  // and, for lane (c, g), the scale of key 16g + c, the key this lane writes
  auto load_batch = [&](const Batch& x, i32x8 (&kb)[kStreamBatch], float& sgl) {
    const bool okp = x.page >= 0 && x.page < bv.num_pages;
    const uint8_t* pg = cache + (int64_t)(okp ? x.page : 0) * p.page_bytes;
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) {
      const int uu = u < x.cnt ? u : 0;                          // past the chunk: re-read group 0
      const int slot = (16 * (x.gi + uu)) % P + c;
      kb[u] = *reinterpret_cast<const i32x8*>(pg + (int64_t)slot * kIdxDim + 32 * g);
    }
    const int gl = g < x.cnt ? g : 0;
    sgl = *reinterpret_cast<const float*>(pg + scale_off + 4 * ((16 * (x.gi + gl)) % P + c));
  };

  // q of the unit's rows as 16-head A operands (lane (c, g): head 16m + c,
  // bytes [32g, 32g + 32)) and their head weights in accumulator order
  i32x8 qa[kR][4];
  float wv[kR][16];
  int q_unit = -1;
  auto load_unit = [&](const Batch& x) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      if (r < x.nr) {
        const int row = x.r0 + r;
        const uint8_t* qr = static_cast<const uint8_t*>(p.q) + (int64_t)row * (kIdxHeads * kIdxDim);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          qa[r][m] = *reinterpret_cast<const i32x8*>(qr + (16 * m + c) * kIdxDim + 32 * g);
        const float* wrow = p.w + (int64_t)row * kIdxHeads;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(wrow + 16 * m + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[r][4 * m + i] = w4[i];
        }
      }
    }
    q_unit = x.t;
  };

  for (int round = c_begin; round < c_end; round += kStreamMaxChunks) {
    const int n = min(kStreamMaxChunks, c_end - round);
    // ---- the round's chunk records ----
    for (int i = tid; i < n; i += kThreads) {
      const int ch = round + i;
      int lo = 0, hi = U - 1;                                    // unit: the largest t with pre[t] <= ch
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= ch) lo = mid; else hi = mid - 1;
      }
      int b_, r0_, nr_, vf_, vl_;
      stream_unit<kR>(bv, lo, cap, &b_, &r0_, &nr_, &vf_, &vl_);
      const int n_t = (vl_ + 15) >> 4;
      const int cu = ch - pre[lo];
      const int pgi = cu / cpp;                                  // page index inside the unit
      const int gi = pgi * gpp + kStreamBatch * (cu - pgi * cpp);
      const int gend = min(min(gi + kStreamBatch, (pgi + 1) * gpp), n_t);
      const int page = bv.block_table[(int64_t)b_ * bv.max_pages_per_seq + pgi];
      rec_a[i] = make_int4(lo, gi, gend - gi, page);
      rec_b[i] = make_int4(r0_, nr_, vf_, vl_);
    }
    if (tid == 0) next_chunk = 0;
    __syncthreads();

    // ---- the waves take chunks until the round is done. Two chunk slots,
    // A and B, alternate by name: while the MFMAs of one slot's chunk run,
    // the other slot's loads are in flight, and the index of the chunk after
    // that is taken. Every slot load is issued (once the round is out of
    // chunks, as a re-read of the chunk just computed), and no register of a
    // load in flight is copied: either would make the compiler wait for every
    // load in flight before the MFMAs. ----
    static_assert(kAhead == 1, "the stream loop holds two chunk slots");
    // logits of chunk x for every row of its unit: the four groups' head sums
    // are reduce-scattered so that lane (c, g) writes key 16g + c of the chunk
    auto compute = [&](const Batch& x, const i32x8 (&kb)[kStreamBatch], float sgl) {
      const bool okp = x.page >= 0 && x.page < bv.num_pages;
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (r >= x.nr) break;
        // rows of a unit see one key more each; the last one sees vl
        const int vis = (r == x.nr - 1) ? x.vl : x.vf;
        float part[kStreamBatch];
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          part[u] = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 acc = mfma_fp8_16x16x128(qa[r][m], kb[u], zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) part[u] = fmaf(wv[r][4 * m + i], relu_bits(acc[i]), part[u]);
          }
        }
        const float tot = sum_scatter_over_groups(part[0], part[1], part[2], part[3]);
        // one store per row for the whole wave, through a buffer resource over
        // the row: lanes past the chunk or the row get an offset out of range,
        // which drops their store (a branch around the store would make the
        // number of stores in flight unknown to the compiler's waits)
        const int s = 16 * (x.gi + g) + c;
        const __amdgpu_buffer_rsrc_t row = __builtin_amdgcn_make_buffer_rsrc(
            p.logits + (int64_t)(x.r0 + r) * p.stride, (short)0, (int)(p.stride * 4), 0x00020000);
        const uint32_t off = (g < x.cnt && s < vis) ? 4u * (uint32_t)s : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(okp ? tot * sgl : -INFINITY), row, (int)off, 0, 0);
      }
    };
    static_assert(kStreamBatch == 4, "one group per lane group");
    i32x8 kbA[kStreamBatch], kbB[kStreamBatch];
    float sgA, sgB;
    int ja = take();
    Batch ba = record(ja < n ? ja : 0), bb = ba;
    load_batch(ba, kbA, sgA);
    int jb = ja < n ? take() : n;
    while (ja < n) {
      // slot A computes chunk ja while slot B loads chunk jb
      int jt = n;                                                // read after the MFMAs
      if (lane == 0 && jb < n) jt = atomicAdd(&next_chunk, 1);
      if (ba.t != q_unit) load_unit(ba);
      bb = record(jb < n ? jb : ja);
      load_batch(bb, kbB, sgB);
      compute(ba, kbA, sgA);
      ja = jb < n ? __builtin_amdgcn_readfirstlane(jt) : n;
      if (jb >= n) break;
      // slot B computes chunk jb while slot A loads chunk ja
      jt = n;
      if (lane == 0 && ja < n) jt = atomicAdd(&next_chunk, 1);
      if (bb.t != q_unit) load_unit(bb);
      ba = record(ja < n ? ja : jb);
      load_batch(ba, kbA, sgA);
      compute(bb, kbB, sgB);
      jb = ja < n ? __builtin_amdgcn_readfirstlane(jt) : n;
    }
    __syncthreads();                                             // records free for the next round
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

// Work-groups of a stream kernel that the current device holds at once: CUs
// times the occupancy the kernel's registers and LDS allow (one per CU).
// Queried once per device and kernel (host calls only, nothing is enqueued).
template <int kR, int kAhead>
int resident_wgs() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0, per_cu = 0;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, indexer_fp8_stream_kernel<kR, kAhead>,
                                                   stream_waves<kR, kAhead>() * kWave, 0) != hipSuccess ||
      cus < 1 || per_cu < 1) {
    (void)hipGetLastError();
    return 256;                                                  // MI355X: 256 CUs
  }
  const int v = cus * per_cu;
  if (dev >= 0) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

// Init/local-token forcing (SGLang indexer page, Indexer._mask_init_and_local_tokens):
// +inf at the first num_init and the last num_local visible positions of every
// row, after the scores are written. One work-group per row.
__global__ __launch_bounds__(256) void indexer_force_kernel(IndexerParams p) {
  const BatchView& bv = p.batch;
  const int t = blockIdx.x;
  int b, j, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &j, &q_len);
  int cap = bv.max_pages_per_seq * bv.page_size;
  if (cap > bv.max_seq_len_k) cap = bv.max_seq_len_k;
  if ((int64_t)cap > p.stride) cap = (int)p.stride;
  const int vis = visible_keys(bv.seq_lens_k[b], q_len, j, cap);
  const int n_init = min(p.num_init, vis);
  const int local0 = max(vis - p.num_local, n_init);             // forced tail [local0, vis)
  float* out = p.logits + (int64_t)t * p.stride;
  for (int s = threadIdx.x; s < n_init; s += 256) out[s] = INFINITY;
  for (int s = local0 + threadIdx.x; s < vis; s += 256) out[s] = INFINITY;
}

hipError_t launch_indexer_force(const IndexerParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0 || (p.num_init <= 0 && p.num_local <= 0)) return hipSuccess;
  hipLaunchKernelGGL(indexer_force_kernel, dim3(p.batch.num_rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_indexer_fp8(const IndexerParams& p, hipStream_t s) {
  const int chunks = (p.batch.max_seq_len_k + kIdxChunk - 1) / kIdxChunk;
  if (p.batch.num_rows == 0 || chunks == 0) return hipSuccess;
  // the stream kernel stores each row through a buffer resource whose range
  // (stride * 4 bytes) must fit 32 bits
  const bool stream_stride = p.stride <= kStreamMaxStride;
  const bool decode = p.batch.cu_seqlens_q == nullptr && p.batch.num_rows <= kStreamMaxUnits && stream_stride;
  const bool multi = p.batch.cu_seqlens_q != nullptr && p.batch.max_seq_len_q <= kStreamMaxQLen &&
                     2 * p.batch.num_seqs <= kStreamMaxUnits && stream_stride;
  if (decode || multi) {
    // spread over as many CUs as there are chunks for one per wave (a bound
    // from the longest row), and no more work-groups than are resident at
    // once (one round: a second round would start late and finish last)
    const int64_t units = decode ? p.batch.num_rows : std::min<int64_t>(p.batch.num_rows, 2LL * p.batch.num_seqs);
    const int64_t chunks = units * ((p.batch.max_seq_len_k + 16 * kStreamBatch - 1) / (16 * kStreamBatch));
    const int waves = decode ? stream_waves<1, kDecodeAhead>() : stream_waves<2, 1>();
    int64_t wgs = (chunks + waves - 1) / waves;
    const int resident = decode ? resident_wgs<1, kDecodeAhead>() : resident_wgs<2, 1>();
    if (wgs > resident) wgs = resident;
    if (wgs < 1) wgs = 1;
    if (decode)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(indexer_fp8_stream_kernel<1, kDecodeAhead>), dim3((unsigned)wgs),
                         dim3(stream_waves<1, kDecodeAhead>() * kWave), 0, s, p);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(indexer_fp8_stream_kernel<2, 1>), dim3((unsigned)wgs),
                         dim3(stream_waves<2, 1>() * kWave), 0, s, p);
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
