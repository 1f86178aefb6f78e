// Sparse MLA attention over the top-k selected latent rows.
//
// (Ascend "sfa_v1.py" page: npu_sparse_flash_attention with key = value = the
// latent cache, the rope key passed separately, token-granular sparse indices
// and the block table; vLLM "mla/common.py" page: the cached row is the 512-d
// latent followed by the 64-d rope key, decode returns (out, lse), and partial
// results merge through their log-sum-exps with merge_attn_states.)
//
// For row t and head h over the valid entries i of topk_idx[t]:
//   z_i = scale * (q[t,h] . C_i),  out[t,h] = sum_i softmax(z)_i C_i[:512],
//   lse[t,h] = log sum_i exp(z_i).
//
// bf16 path (Dl = 512, Dr = 64, Hm a multiple of 64). One work-group of eight
// waves handles one (row, split of the top-k list, group of 64 heads).
// Gathered rows arrive 32 at a time (a tile) straight from HBM into a ring of
// four LDS slots (global_load_lds, 16 bytes per lane, no register staging),
// XOR-swizzled by 16-byte chunk. The waves have two roles, one wave of each
// per SIMD, so that the stalls of one (LDS latency, softmax) are covered by the
// MFMAs of the other:
//   * score waves 0..3: wave w computes S[32 rows x 16 heads] (heads 16 w ..)
//     of the next tile over the 576-wide contraction with
//     v_mfma_f32_16x16x32_bf16 (rows as M from LDS, heads as N from q held in
//     registers for the whole split), then the online softmax of its heads,
//     whose rows are all in the wave: fp32, base 2, lazy rescaling (the
//     running maximum of a head only moves when a tile exceeds it by more than
//     2^8). The probabilities go to a 4 KB LDS buffer as bf16;
//   * value waves 4..7: wave 4 + v owns value columns 128 v .. 128 v + 127 of
//     all 64 heads and computes O^T[128 columns x 64 heads] += V^T . P^T, so
//     every V element is read from LDS once per tile. V^T arrives as the A
//     operand through the gfx950 transposing LDS read (ds_read_b64_tr_b16),
//     P^T as the B operand from the probability buffer. The accumulator gives
//     each lane four consecutive columns of one head, so the output leaves in
//     8- or 16-byte stores.
// Every wave issues a share of the tile copies, spread over its MFMAs.
//
// Interval j (between two barriers B2): the score waves compute S and the
// softmax of tile j+1 while the value waves, having read P of tile j into
// registers, multiply tile j; all waves spread their copies of tile j+3 (into
// the slot of tile j-1, which no wave reads any more) over their MFMAs;
// barrier B1; the score waves write P of tile j+1; every wave waits for its
// copies of tile j+2; barrier B2.
//
// Single split: out = O / l in bf16 and lse; several splits: partials (O / l
// in bf16, lse in fp32) merged by mla_combine_kernel in fp32. Work-groups are ordered so that
// the head groups of one (row, split) unit, and neighbouring units, land on
// the same XCD (work-group i runs on XCD i % 8) and share the gathered rows
// through that XCD's L2.
#include <cfloat>

#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMlaThreads = 512;
constexpr int kMlaWaves = kMlaThreads / kWave;          // 8
constexpr int kRoleWaves = kMlaWaves / 2;               // 4 score waves, 4 value waves
constexpr int kRowBytes = kMlaDqk * 2;                  // 1152: one cached latent row
constexpr int kChunksPerRow = kRowBytes / 16;           // 72 chunks of 16 bytes
constexpr int kTileBytes = kMlaTile * kRowBytes;        // 36864
constexpr int kPiecesPerTile = kTileBytes / 1024;       // 36 wave-wide 1 KB copies
constexpr int kPiecesMax = (kPiecesPerTile + kMlaWaves - 1) / kMlaWaves;   // 5 (waves 0..3), else 4
constexpr int kRing = 4;                                // LDS tile slots
constexpr int kEntriesPerThread = kMlaMaxEntriesPerBlock / kMlaThreads;  // 4
constexpr int kKSteps = kMlaDqk / 32;                   // 18 K-steps of 32
constexpr int kKB = 2;                                  // K-steps per score operand batch
constexpr int kKBatches = kKSteps / kKB;                // 9
constexpr int kPvNT = kMlaDl / kRoleWaves / 16;         // 8 value-column tiles per value wave
constexpr int kPvHT = kMlaHeadsPerGroup / 16;           // 4 head tiles
constexpr int kSAhead = 3;                              // score operand batches read ahead of their MFMAs
constexpr int kVAhead = 4;                              // value-column tiles read ahead of their MFMAs
constexpr float kRescaleThreshold = 8.0f;               // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
static_assert(kPiecesPerTile > (kPiecesMax - 1) * kMlaWaves && kPiecesPerTile <= kPiecesMax * kRoleWaves + (kPiecesMax - 1) * kRoleWaves,
              "waves 0..3 copy kPiecesMax pieces of a tile, waves 4..7 one fewer");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

struct MlaShared {
  // Gathered rows, dense (1152 B per row). Inside row r the 16-byte chunk c is
  // stored at chunk position c ^ swz(r) (see swz).
  alignas(16) uint8_t kv[kRing][kTileBytes];
  // P of one tile, [head][contraction index] bf16: row 4g + i of the tile at
  // index 8g + i, row 16 + 4g + i at index 8g + 4 + i (the order in which the
  // value waves' transposing reads deliver V)
  alignas(16) uint16_t p[kMlaHeadsPerGroup * kMlaTile];
  alignas(16) float alpha[kMlaHeadsPerGroup];            // rescale factor of the tile; at the end 1 / l
  alignas(16) int flag[kRoleWaves];                      // some head of score wave w rescaled
  int32_t rowid[kMlaMaxEntriesPerBlock];
  int wave_sum[kMlaWaves];
};

// Chunk swizzle of row r: the low three bits of r. With it the score operand
// reads (sixteen rows, one logical chunk each) and the transposed value reads
// (rows 4g .. 4g+3, 32 bytes each, per 16-lane block g) run at the full LDS
// rate (measured on gfx950; rows are 1152 bytes apart).
__device__ __forceinline__ int swz(int row) { return row & 7; }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// transposing LDS read: lane 4k + m of each 16-lane block names 8 bytes (four
// bf16) of row k; lane i of the block receives element i % 4 of lane
// 4 * kk + i / 4's bytes in slot kk, i.e. one column of four rows
__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
}

// Wait until at most `tiles` tiles of this wave's copies are outstanding
// (vector-memory operations complete in issue order; a wave copies kPiecesMax
// or kPiecesMax - 1 pieces per tile).
__device__ __forceinline__ void wait_tiles(int tiles, bool five) {
  if (five) {
    if (tiles >= 2) wait_vmcnt<2 * kPiecesMax>();
    else if (tiles == 1) wait_vmcnt<kPiecesMax>();
    else wait_vmcnt<0>();
  } else {
    if (tiles >= 2) wait_vmcnt<2 * (kPiecesMax - 1)>();
    else if (tiles == 1) wait_vmcnt<kPiecesMax - 1>();
    else wait_vmcnt<0>();
  }
}

template <bool kPosScale>
__global__ __launch_bounds__(kMlaThreads) void mla_bf16_kernel(MlaParams p) {
  __shared__ MlaShared sh;
  const BatchView& bv = p.batch;
  const int T = bv.num_rows;
  const int HG = p.heads / kMlaHeadsPerGroup;
  const int S = p.splits;

  // work-group -> (row t, split s, head group hg), XCD-aware
  const int units = T * S;
  const int units_per_xcd = (units + 7) / 8;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int unit_local = slot / HG;
  const int hg = slot % HG;
  if (unit_local >= units_per_xcd) return;
  const int unit = xcd * units_per_xcd + unit_local;
  if (unit >= units) return;
  const int t = unit / S;
  const int s = unit % S;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int g = lane >> 4, c = lane & 15;
  const bool scorer = wave < kRoleWaves;     // uniform per wave
  const int rw = wave & (kRoleWaves - 1);    // index inside the role
  const bool five = wave + kMlaWaves * (kPiecesMax - 1) < kPiecesPerTile;   // copies kPiecesMax pieces

  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  const int addressable = bv.max_pages_per_seq * P;
  if (seq_len > addressable) seq_len = addressable;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;

  const int Hm = p.heads;
  const int hbase = hg * kMlaHeadsPerGroup;  // first head of the group
  const int hl_s = 16 * rw + c;              // score waves: this lane's head inside the group

  // ---- resolve this split's entries into cache-row ids (compacted, in order) ----
  const int e_begin = s * p.entries_per_split;
  int e_cnt = p.k - e_begin;
  if (e_cnt > p.entries_per_split) e_cnt = p.entries_per_split;
  if (e_cnt < 0) e_cnt = 0;
  const int32_t* idx = p.topk_idx + (int64_t)t * p.k + e_begin;
  int pos[kEntriesPerThread], page[kEntriesPerThread];
#pragma unroll
  for (int q = 0; q < kEntriesPerThread; ++q) {       // all index loads in flight
    const int e = kEntriesPerThread * tid + q;
    pos[q] = (e < e_cnt) ? idx[e] : -1;
  }
#pragma unroll
  for (int q = 0; q < kEntriesPerThread; ++q) {       // then all page lookups
    const bool in = pos[q] >= 0 && pos[q] < seq_len;
    page[q] = in ? bt[pos[q] / P] : -1;
  }
  int nmine = 0;
#pragma unroll
  for (int q = 0; q < kEntriesPerThread; ++q) nmine += (page[q] >= 0 && page[q] < bv.num_pages) ? 1 : 0;
  const int incl = (int)wave_inclusive_scan((uint32_t)nmine);
  if (lane == kWave - 1) sh.wave_sum[wave] = incl;
  __syncthreads();
  int nvalid = 0, w_off = 0;
#pragma unroll
  for (int w = 0; w < kMlaWaves; ++w) {
    const int v = sh.wave_sum[w];
    w_off += (w < wave) ? v : 0;
    nvalid += v;
  }
  {
    int o = w_off + incl - nmine;
#pragma unroll
    for (int q = 0; q < kEntriesPerThread; ++q)
      if (page[q] >= 0 && page[q] < bv.num_pages) sh.rowid[o++] = page[q] * P + pos[q] % P;
  }
  __syncthreads();

  const float scale_log2 = p.softmax_scale * kLog2e;
  const uint8_t* kvbase = static_cast<const uint8_t*>(p.kv);
  const int n_tiles = (nvalid + kMlaTile - 1) / kMlaTile;

  // ---- copies. A tile is 36 copies of 1 KB; copy i = wave + 8j covers LDS
  // chunks 64i .. 64i+63, lane l taking chunk 64i + l of the dense tile: row
  // r = chunk / 72, LDS chunk position col = chunk % 72, which holds the
  // logical chunk col ^ swz(r) of the row. Rows past the split's valid
  // entries re-read its first row (their scores are masked).
  auto fetch_rows = [&](int tile, int (&rid)[kPiecesMax]) {
    if ((tile + 1) * kMlaTile <= nvalid) {             // uniform: every row of the tile is valid
#pragma unroll
      for (int j = 0; j < kPiecesMax; ++j) {
        const int pc = min(wave + kMlaWaves * j, kPiecesPerTile - 1);
        rid[j] = sh.rowid[tile * kMlaTile + (64 * pc + lane) / kChunksPerRow];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPiecesMax; ++j) {
        const int pc = min(wave + kMlaWaves * j, kPiecesPerTile - 1);
        const int e = tile * kMlaTile + (64 * pc + lane) / kChunksPerRow;
        rid[j] = sh.rowid[e < nvalid ? e : 0];
      }
    }
  };
  auto issue_pieces = [&](int tile, const int (&rid)[kPiecesMax], int j0, int j1) {
    const uint32_t dst = lds_offset(sh.kv[tile % kRing]);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      if (j == kPiecesMax - 1 && !five) break;
      const int pc = wave + kMlaWaves * j;
      const int chunk = 64 * pc + lane;
      const int r = chunk / kChunksPerRow;
      const int col = ((chunk - r * kChunksPerRow) ^ swz(r)) * 16;
      lds_dma16(kvbase + (int64_t)rid[j] * kRowBytes + col, dst + 1024 * pc);
    }
  };


  // score operand (A): lane (c, g) reads rows c and 16 + c of the tile,
  // 16-byte chunk 4 ks + g of the row. With ks = 2a + u the swizzled position
  // is 8a + ((4u + g) ^ swz(row)): a per-lane base plus an immediate.
  const int a_off0 = c * kRowBytes + ((g ^ swz(c)) << 4);
  const int a_off1 = c * kRowBytes + (((4 + g) ^ swz(c)) << 4);
  // value operand (A of O^T += V^T P^T): two transposing reads give lane
  // (c, g) value column 128 v + 16 nt + c of rows 4g .. 4g+3 and 16+4g ..
  // 16+4g+3 (contraction index 8g + e, e = 0..7). Lane 4k + m of block g names
  // row 16h + 4g + k (h = which read), columns 16 nt + 4m .. + 3 of the wave's
  // 128: logical chunk 16 v + 2 nt + (m >> 1), byte 8 (m & 1). With
  // nt = 4a + u the chunk sits at 16 v + 8a + ((2u + (m >> 1)) ^ swz(row)).
  int v_off[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * h + 4 * g + (c >> 2);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v_off[h][u] = r * kRowBytes + ((16 * rw + ((2 * u + ((c & 3) >> 1)) ^ swz(r))) << 4) + ((c & 1) << 3);
  }
  // P^T operand (B): lane (c, g) reads P[head 16 hb + c][8g .. 8g+7]
  const int p_off = c * kMlaTile + 8 * g;

  constexpr int kAhead = kRing - 1;                    // tiles copied ahead of the one scored
  int rid_next[kPiecesMax];

  if (scorer) {
    // ================= score waves =================
    // The copies of tile 0, then q (the N operand: lane (c, g) holds head
    // hbase + hl_s, elements 32 ks + 8 g .. + 7), consumed at once: the
    // compiler then knows its loads have completed and places no
    // vector-memory waits inside the tile loop, where they would also drain the
    // (to it invisible) tile copies in flight. Its wait covers tile 0, which
    // the scores need first anyway; tiles 1 and 2 follow.
    if (n_tiles > 0) {
      fetch_rows(0, rid_next);
      issue_pieces(0, rid_next, 0, kPiecesMax);
    }
    bf16x8 qf[kKSteps];
    {
      const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)t * Hm + hbase + hl_s) * kMlaDqk;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
    }
    for (int tl = 1; tl < kAhead && tl < n_tiles; ++tl) {
      fetch_rows(tl, rid_next);
      issue_pieces(tl, rid_next, 0, kPiecesMax);
    }
    if (n_tiles > kAhead) fetch_rows(kAhead, rid_next);

    float m_ref = -INFINITY;   // running max (log2 units) of head hl_s
    float l_part = 0.f;        // this lane's share of that head's denominator

    // S[rows, head hl_s] of one tile (lane (c, g): rows 4g + i in s0,
    // 16 + 4g + i in s1), operands read one batch ahead of their MFMAs.
    auto scores = [&](const uint8_t* kvt, f32x4& s0, f32x4& s1, int copy_tile, int (&rid)[kPiecesMax]) {
      auto read_k = [&](int bk, bf16x8 (&dst)[kKB][2]) {
#pragma unroll
        for (int u = 0; u < kKB; ++u) {
          const int ks = kKB * bk + u;
          const int off = ((ks & 1) ? a_off1 : a_off0) + 128 * (ks >> 1);
          dst[u][0] = *reinterpret_cast<const bf16x8*>(kvt + off);
          dst[u][1] = *reinterpret_cast<const bf16x8*>(kvt + off + 16 * kRowBytes);
        }
      };
      constexpr int kDepth = kSAhead + 1;
      bf16x8 op[kDepth][kKB][2];                       // operands read kSAhead batches ahead
      s0 = f32x4{0.f, 0.f, 0.f, 0.f};
      s1 = s0;
#pragma unroll
      for (int bk = 0; bk < kSAhead; ++bk) read_k(bk, op[bk]);
#pragma unroll
      for (int bk = 0; bk < kKBatches; ++bk) {
        if (bk + kSAhead < kKBatches) read_k(bk + kSAhead, op[(bk + kSAhead) % kDepth]);
        // this wave's copies early in the interval, for the longest lead
        if (copy_tile >= 0 && bk < 3) issue_pieces(copy_tile, rid, 2 * bk, min(2 * bk + 2, kPiecesMax));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kKB; ++u) {
          s0 = mfma_bf16(op[bk % kDepth][u][0], qf[kKB * bk + u], s0);
          s1 = mfma_bf16(op[bk % kDepth][u][1], qf[kKB * bk + u], s1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // online softmax of one tile; returns the bf16 probabilities of the
    // lane's head at contraction indices 8g .. 8g+7 and its rescale factor
    auto softmax = [&](int tile, const f32x4& s0, const f32x4& s1, float* alpha) -> bf16x8 {
      const int rows_left = nvalid - tile * kMlaTile;   // padding rows (last tile only) -> -inf
      // With a positive scale the scores stay unscaled here: rounding is
      // monotone, so the maximum of the scaled scores is the scaled maximum,
      // and the scale enters each exponent through one fma.
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = kPosScale ? s0[i] : s0[i] * scale_log2;
        sv[4 + i] = kPosScale ? s1[i] : s1[i] * scale_log2;
      }
      if (rows_left < kMlaTile) {                        // uniform: the last, partial tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = (4 * g + i < rows_left) ? sv[i] : -INFINITY;
          sv[4 + i] = (16 + 4 * g + i < rows_left) ? sv[4 + i] : -INFINITY;
        }
      }
      float mx = fmaximum(fmaximum(fmaximum(sv[0], sv[1]), fmaximum(sv[2], sv[3])),
                          fmaximum(fmaximum(sv[4], sv[5]), fmaximum(sv[6], sv[7])));
      mx = max_over_groups(mx);                        // a NaN score makes the head's output NaN either way
      if (kPosScale) mx *= scale_log2;
      *alpha = 1.f;
      if (mx > m_ref + kRescaleThreshold) {
        *alpha = __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
        l_part *= *alpha;
      }
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(kPosScale ? fmaf(sv[i], scale_log2, -m_ref) : sv[i] - m_ref);
        l_part += pr[i];
      }
      bf16x8 pa;                                         // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 two = __builtin_convertvector(f32x2{pr[2 * i], pr[2 * i + 1]}, bf16x2);
        pa[2 * i] = two[0];
        pa[2 * i + 1] = two[1];
      }
      return pa;
    };
    auto publish = [&](const bf16x8& pa, float alpha) {  // between B1 and B2
      *reinterpret_cast<bf16x8*>(&sh.p[hl_s * kMlaTile + 8 * g]) = pa;
      if (g == 0) sh.alpha[hl_s] = alpha;
      const bool any = __ballot(alpha != 1.f) != 0ull;
      if (lane == 0) sh.flag[rw] = any ? 1 : 0;
    };

    if (n_tiles > 0) {                                 // prologue: tile 0
      wait_tiles(min(n_tiles, kAhead) - 1, five);      // tile 0 has landed
      __syncthreads();
      f32x4 s0, s1;
      scores(sh.kv[0], s0, s1, -1, rid_next);
      float alpha;
      const bf16x8 pa = softmax(0, s0, s1, &alpha);
      publish(pa, alpha);
      wait_tiles(min(n_tiles, kAhead) - 2, five);      // tile 1 has landed
      __syncthreads();
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      const bool more = tile + 1 < n_tiles;            // uniform
      bf16x8 pa;
      float alpha = 1.f;
      const int last = n_tiles - 1;
      const int copy_tile = tile + kAhead <= last ? tile + kAhead : -1;   // uniform
      if (more) {
        f32x4 s0, s1;
        scores(sh.kv[(tile + 1) % kRing], s0, s1, copy_tile, rid_next);
        pa = softmax(tile + 1, s0, s1, &alpha);
      } else if (copy_tile >= 0) {
        issue_pieces(copy_tile, rid_next, 0, kPiecesMax);
      }
      if (copy_tile >= 0 && copy_tile + 1 <= last) fetch_rows(copy_tile + 1, rid_next);
      __syncthreads();                                 // B1: every value wave holds P of tile
      if (more) publish(pa, alpha);
      wait_tiles(min(tile + kAhead, last) - (tile + 2), five);   // tile + 2 has landed
      __syncthreads();                                 // B2
    }
    // denominators, lse; 1 / l for the value waves
    const float l = sum_over_groups(l_part);
    if (g == 0) {
      const float lse_val = (l > 0.f) ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
      if (S == 1) {
        if (p.lse) p.lse[(int64_t)t * Hm + hbase + hl_s] = lse_val;
      } else {
        p.part_lse[((int64_t)t * S + s) * Hm + hbase + hl_s] = lse_val;
      }
      sh.alpha[hl_s] = l > 0.f ? 1.f / l : 0.f;
    }
    __syncthreads();
  } else {
    // ================= value waves =================
    for (int tl = 0; tl < kAhead && tl < n_tiles; ++tl) {
      fetch_rows(tl, rid_next);
      issue_pieces(tl, rid_next, 0, kPiecesMax);
    }
    if (n_tiles > kAhead) fetch_rows(kAhead, rid_next);
    f32x4 acc_o[kPvHT][kPvNT];   // O[head 16 hb + c][value column 128 v + 16 nt + 4g + i]
#pragma unroll
    for (int hb = 0; hb < kPvHT; ++hb)
#pragma unroll
      for (int nt = 0; nt < kPvNT; ++nt) acc_o[hb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (n_tiles > 0) {                                 // prologue (score waves: tile 0)
      wait_tiles(min(n_tiles, kAhead) - 1, five);      // tile 0 has landed
      __syncthreads();
      wait_tiles(min(n_tiles, kAhead) - 2, five);      // tile 1 has landed
      __syncthreads();
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      const uint8_t* kvt = sh.kv[tile % kRing];
      const int last = n_tiles - 1;
      const int copy_tile = tile + kAhead <= last ? tile + kAhead : -1;   // uniform
      // P of this tile; (rare) the heads whose running max moved with this
      // tile rescale their O first
      const i32x4 fl4 = *reinterpret_cast<const i32x4*>(sh.flag);
      bf16x8 pb[kPvHT];
#pragma unroll
      for (int hb = 0; hb < kPvHT; ++hb)
        pb[hb] = *reinterpret_cast<const bf16x8*>(&sh.p[16 * hb * kMlaTile + p_off]);
      if (__builtin_amdgcn_readfirstlane(fl4[0] | fl4[1] | fl4[2] | fl4[3])) {
#pragma unroll
        for (int hb = 0; hb < kPvHT; ++hb) {
          const float a = sh.alpha[16 * hb + c];
#pragma unroll
          for (int nt = 0; nt < kPvNT; ++nt) acc_o[hb][nt] *= a;
        }
      }
      // O += P . V(tile), value operands read kVAhead column tiles ahead of their MFMAs
      i16x4 vlo[kVAhead], vhi[kVAhead];
      auto read_v = [&](int nt) {
        const int imm = 128 * (nt >> 2);
        vlo[nt % kVAhead] = lds_read_tr16(kvt + v_off[0][nt & 3] + imm);
        vhi[nt % kVAhead] = lds_read_tr16(kvt + v_off[1][nt & 3] + imm);
      };
#pragma unroll
      for (int nt = 0; nt < kVAhead; ++nt) read_v(nt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < kPvNT; ++nt) {
        const bf16x8 v8 = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(vlo[nt % kVAhead], vhi[nt % kVAhead], 0, 1, 2, 3, 4, 5, 6, 7));
        if (nt + kVAhead < kPvNT) read_v(nt + kVAhead);
        if (copy_tile >= 0 && nt < 2) issue_pieces(copy_tile, rid_next, 2 * nt, 2 * nt + 2);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 0; hb < kPvHT; ++hb) acc_o[hb][nt] = mfma_bf16(v8, pb[hb], acc_o[hb][nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (copy_tile >= 0 && copy_tile + 1 <= last) fetch_rows(copy_tile + 1, rid_next);
      __syncthreads();                                 // B1: done with tile's slot
      wait_tiles(min(tile + kAhead, last) - (tile + 2), five);   // tile + 2 has landed
      __syncthreads();                                 // B2
    }
    __syncthreads();                                   // 1 / l of every head is in LDS
#pragma unroll
    for (int hb = 0; hb < kPvHT; ++hb) {
      const float inv = sh.alpha[16 * hb + c];
      const int h = hbase + 16 * hb + c;
      const int col0 = 128 * rw + 4 * g;
      if (S == 1) {
        uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * kMlaDl + col0;
#pragma unroll
        for (int nt = 0; nt < kPvNT; ++nt) {
          const f32x4 o = acc_o[hb][nt] * inv;
          *reinterpret_cast<bf16x4*>(orow + 16 * nt) = __builtin_convertvector(o, bf16x4);
        }
      } else {
        uint16_t* orow = p.part_o + (((int64_t)t * S + s) * Hm + h) * kMlaDl + col0;
#pragma unroll
        for (int nt = 0; nt < kPvNT; ++nt) {
          const f32x4 o = acc_o[hb][nt] * inv;
          *reinterpret_cast<bf16x4*>(orow + 16 * nt) = __builtin_convertvector(o, bf16x4);
        }
      }
    }
  }
}

// LSE merge of the split partials (merge_attn_states generalised to S parts).
// 256 threads cover four heads of one row; each thread owns eight value
// columns, so every partial arrives in one 16-byte load. With the split count
// known at compile time (kS > 0) all loads of a thread are issued together.
template <int kS>
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaParams p) {
  const int t = blockIdx.x;
  const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
  const int d8 = threadIdx.x & 63;                  // value columns 8*d8 .. 8*d8+7
  const int S = kS > 0 ? kS : p.splits, Hm = p.heads;
  if (h >= Hm) return;
  const float* pl = p.part_lse + (int64_t)t * S * Hm + h;
  const uint16_t* po = p.part_o + ((int64_t)t * S * Hm + h) * kMlaDl + 8 * d8;
  const int64_t o_stride = (int64_t)Hm * kMlaDl;    // next split's partial of the same head
  float mx = -INFINITY, tot = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  auto add = [&](float l, const bf16x8& ob) {       // wgt = exp(l - mx), mx final
    const float wgt = (l == -INFINITY) ? 0.f : __expf(l - mx);
    tot += wgt;
    acc0 += wgt * __builtin_convertvector(__builtin_shufflevector(ob, ob, 0, 1, 2, 3), f32x4);
    acc1 += wgt * __builtin_convertvector(__builtin_shufflevector(ob, ob, 4, 5, 6, 7), f32x4);
  };
  if (kS > 0) {
    float l[kS > 0 ? kS : 1];
    bf16x8 ob[kS > 0 ? kS : 1];
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      l[s] = pl[(int64_t)s * Hm];
      ob[s] = *reinterpret_cast<const bf16x8*>(po + s * o_stride);
    }
#pragma unroll
    for (int s = 0; s < kS; ++s) mx = fmaxf(mx, l[s]);
#pragma unroll
    for (int s = 0; s < kS; ++s) add(l[s], ob[s]);
  } else {
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[(int64_t)s * Hm]);
    for (int s = 0; s < S; ++s) add(pl[(int64_t)s * Hm], *reinterpret_cast<const bf16x8*>(po + s * o_stride));
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (d8 == 0 && p.lse) p.lse[(int64_t)t * Hm + h] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
  const bf16x4 lo = __builtin_convertvector(acc0 * inv, bf16x4);
  const bf16x4 hi = __builtin_convertvector(acc1 * inv, bf16x4);
  *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * kMlaDl + 8 * d8) =
      __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// fp32 path for small shapes: one work-group per (row, head), two-pass softmax.
constexpr int kF32Threads = 256;

__global__ __launch_bounds__(kF32Threads) void mla_f32_kernel(MlaParams p) {
  __shared__ float z[kTopkMaxK];
  __shared__ float qs[1024];
  __shared__ float red[kF32Threads / kWave];
  const BatchView& bv = p.batch;
  const int t = blockIdx.x, h = blockIdx.y;
  const int Hm = p.heads, Dl = p.d_latent, Dqk = p.d_latent + p.d_rope;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  if (seq_len > bv.max_pages_per_seq * P) seq_len = bv.max_pages_per_seq * P;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;
  const float* qrow = static_cast<const float*>(p.q) + ((int64_t)t * Hm + h) * Dqk;
  const float* kv = static_cast<const float*>(p.kv);
  const int32_t* idx = p.topk_idx + (int64_t)t * p.k;
  for (int d = tid; d < Dqk; d += kF32Threads) qs[d] = qrow[d];
  __syncthreads();

  auto row_of = [&](int e) -> int64_t {   // cache row of entry e, or -1
    const int pos = idx[e];
    if (pos < 0 || pos >= seq_len) return -1;
    const int page = bt[pos / P];
    if (page < 0 || page >= bv.num_pages) return -1;
    return (int64_t)page * P + pos % P;
  };

  float mx = -INFINITY;
  for (int e = tid; e < p.k; e += kF32Threads) {
    const int64_t r = row_of(e);
    float v = -INFINITY;
    if (r >= 0) {
      const float* crow = kv + r * Dqk;
      float dot = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(qs[d], crow[d], dot);
      v = dot * p.softmax_scale;
    }
    z[e] = v;
    mx = fmaxf(mx, v);
  }
  for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, d));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < kF32Threads / kWave; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int e = tid; e < p.k; e += kF32Threads) {
    const float v = z[e];
    const float pr = (v == -INFINITY) ? 0.f : expf(v - mx);
    z[e] = pr;
    sum += pr;
  }
  for (int d = 32; d >= 1; d >>= 1) sum += shfl_xor_f(sum, d);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  sum = 0.f;
  for (int w = 0; w < kF32Threads / kWave; ++w) sum += red[w];
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  float* orow = static_cast<float*>(p.out) + ((int64_t)t * Hm + h) * Dl;
  for (int d = tid; d < Dl; d += kF32Threads) {
    float acc = 0.f;
    for (int e = 0; e < p.k; ++e) {
      const float pr = z[e];
      if (pr == 0.f) continue;
      const int64_t r = row_of(e);
      acc = fmaf(pr, kv[r * Dqk + d], acc);
    }
    orow[d] = acc * inv;
  }
  if (tid == 0 && p.lse) p.lse[(int64_t)t * Hm + h] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

}  // namespace

int mla_bf16_splits(int num_rows, int k, int heads) {
  const int groups = num_rows * (heads / kMlaHeadsPerGroup);
  if (groups <= 0) return 1;
  const int min_splits = (k + kMlaMaxEntriesPerBlock - 1) / kMlaMaxEntriesPerBlock;
  int max_splits = (k + 2 * kMlaTile - 1) / (2 * kMlaTile);         // >= 2 tiles per split
  // at most 8: for few rows, longer splits cost less in prologues and merge
  // than the idle CUs they leave (measured on the batch-1 and batch-8 decodes:
  // 8 beats 4, 16 and 32)
  if (max_splits > 8) max_splits = 8;
  int sp = (256 + groups - 1) / groups;
  if (sp > max_splits) sp = max_splits;
  if (sp < min_splits) sp = min_splits;
  if (sp < 1) sp = 1;
  return sp;
}

int mla_entries_per_split(int k, int splits) {
  int e = (k + splits - 1) / splits;
  e = (e + kMlaTile - 1) / kMlaTile * kMlaTile;
  return e;
}

hipError_t launch_mla_bf16(const MlaParams& p, hipStream_t s) {
  const int T = p.batch.num_rows;
  if (T == 0) return hipSuccess;
  const int HG = p.heads / kMlaHeadsPerGroup;
  const int units = T * p.splits;
  const int units_per_xcd = (units + 7) / 8;
  const int64_t blocks = 8LL * units_per_xcd * HG;
  // the positive-scale path needs a normal scale: a padding row's -inf times
  // a zero (flushed) scale would give NaN in its exponent
  if (p.softmax_scale * kLog2e >= FLT_MIN)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mla_bf16_kernel<true>), dim3((unsigned)blocks), dim3(kMlaThreads), 0, s, p);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mla_bf16_kernel<false>), dim3((unsigned)blocks), dim3(kMlaThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_mla_combine_bf16(p, s);
}

hipError_t launch_mla_combine_bf16(const MlaParams& p, hipStream_t s) {
  const dim3 grid(p.batch.num_rows, (p.heads + 3) / 4);
  if (p.splits == 2)
    hipLaunchKernelGGL(mla_combine_kernel<2>, grid, dim3(256), 0, s, p);
  else if (p.splits == 4)
    hipLaunchKernelGGL(mla_combine_kernel<4>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(mla_combine_kernel<0>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// Splits of the fp8 kernel: as for bf16, with at most 1024 entries per split
// (its compacted row ids take 4 KB of LDS) and at least two 64-row tiles.
int mla_fp8_splits(int num_rows, int k, int heads) {
  const int groups = num_rows * (heads / kMlaHeadsPerGroup);
  const int min_splits = (k + kMlaFp8MaxEntriesPerBlock - 1) / kMlaFp8MaxEntriesPerBlock;
  if (groups <= 0) return min_splits < 1 ? 1 : min_splits;
  int max_splits = (k + 128 - 1) / 128;
  if (max_splits > 16) max_splits = 16;
  int sp = (256 + groups - 1) / groups;
  if (sp > max_splits) sp = max_splits;
  if (sp < min_splits) sp = min_splits;
  if (sp < 1) sp = 1;
  return sp;
}

hipError_t launch_mla_f32(const MlaParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_f32_kernel, dim3(p.batch.num_rows, p.heads), dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
