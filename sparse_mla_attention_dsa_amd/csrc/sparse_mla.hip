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
// waves handles one (row, split of the top-k list, group of 64 heads):
//   * the split's positions are resolved once through the block table into
//     cache-row ids in LDS, skipping -1 / out-of-range entries (so the -1 tail
//     of short rows costs nothing);
//   * gathered rows arrive 32 at a time straight from HBM into a ring of three
//     LDS tiles (global_load_lds, 16 bytes per lane): two tiles are in flight
//     while the third is computed on. Rows are stored dense with an XOR swizzle
//     of their 16-byte chunks so that both LDS read patterns below are free of
//     bank conflicts;
//   * scores: waves w and w + 4 compute S^T[32 rows x 16 heads] = C_tile . Q^T
//     over the two halves of the 576-wide contraction with
//     v_mfma_f32_16x16x32_bf16 (rows = M from LDS, heads = N from registers:
//     each wave keeps its 16 heads x 288 of q in VGPRs) and exchange the
//     halves through LDS;
//   * online softmax in fp32, base 2, with lazy rescaling: the running maximum
//     of a head only moves when a tile exceeds it by more than 2^8, so the
//     accumulator rescale is skipped on most tiles;
//   * probabilities (bf16) and the per-head rescale factors go through LDS so
//     that wave w can compute O[64 heads x 64 value columns] += P . V_tile,
//     again on 16x16x32 bf16 MFMA (heads = M, value columns = N). The small
//     per-wave register footprint (q 36, O 64) gives two waves per SIMD;
//   * single split: out = O / l in bf16 and lse; several splits: fp32 partials
//     (O / l, lse) merged by mla_combine_kernel.
// Work-groups are ordered so that the head groups of one (row, split) unit, and
// neighbouring units, land on the same XCD (work-group i runs on XCD i % 8) and
// share the gathered rows through that XCD's L2.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMlaThreads = 512;
constexpr int kMlaWaves = kMlaThreads / kWave;          // 8
constexpr int kRowBytes = kMlaDqk * 2;                  // 1152: one cached latent row
constexpr int kChunksPerRow = kRowBytes / 16;           // 72 chunks of 16 bytes
constexpr int kTileBytes = kMlaTile * kRowBytes;        // 36864
constexpr int kDmaPerTile = kTileBytes / 1024;          // 36 wave-wide 1 KB pieces
constexpr int kRing = 3;                                // LDS tile slots
constexpr int kCopies = 5;                              // 16-byte copies per thread per tile (36 per wave-slot)
constexpr int kEntriesPerThread = kMlaMaxEntriesPerBlock / kMlaThreads;  // 4
constexpr int kKSteps = kMlaDqk / 2 / 32;               // 9 K-steps of 32 in each half of 576
constexpr int kPRow = kMlaTile + 4;                     // P row stride (72 B): conflict-free rows
constexpr float kRescaleThreshold = 8.0f;               // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

struct MlaShared {
  // Gathered rows, dense (1152 B per row). Inside row r the 16-byte chunk c is
  // stored at chunk position c ^ swz(r) (see swz).
  alignas(16) uint8_t kv[kRing][kTileBytes];
  int32_t rowid[kMlaMaxEntriesPerBlock];
  alignas(16) uint16_t pbuf[2][kMlaHeadsPerGroup * kPRow];  // [parity][head][row] bf16, padded rows
  alignas(16) f32x4 sx[kMlaWaves / 2][2][kWave];            // second-half partial scores
  alignas(16) float alpha[2][kMlaHeadsPerGroup];
  alignas(16) float lsum[kMlaHeadsPerGroup];
  int flag[2];
  int wave_sum[kMlaWaves];
};

// Chunk swizzle of row r (bits 0-2 of r, bit 3 of r folded onto bits 0-1):
// sixteen consecutive rows reading the same logical chunk, and the rows
// {j, j+4, j+8, j+12} reading the same value column, hit distinct banks for
// both 8-lane (128 B) and 16-lane (256 B) LDS service groups. Rows r and r + 16
// share the swizzle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ (((row >> 3) & 1) * 3); }

// max of v over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups), with the
// gfx950 lane swaps (VALU, no LDS round trip)
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


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
  const int ht = wave & 3;     // score role: heads 16*ht .. 16*ht+15 of the group
  const int kh = wave >> 2;    //             half of the 576-wide contraction

  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  const int addressable = bv.max_pages_per_seq * P;
  if (seq_len > addressable) seq_len = addressable;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;

  const int head0 = hg * kMlaHeadsPerGroup;
  const int Hm = p.heads;
  // ---- q (loads overlap the index resolution below): this wave's 16 heads, its half of the contraction (N operand) ----
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                         ((int64_t)t * Hm + head0 + 16 * ht + c) * kMlaDqk + kh * (kMlaDqk / 2);
  bf16x8 qf[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);

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
  int incl = nmine;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) sh.wave_sum[wave] = incl;
  if (tid < 2) sh.flag[tid] = 0;
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

  // A tile is 36 pieces of 1 KB; piece i holds LDS chunks 64i .. 64i+63 and is
  // fetched by wave i % 8 (waves 0-3 fetch five pieces, waves 4-7 four), lane l
  // taking chunk 64i + l: the logical chunk col ^ swz(row) of its row goes to
  // LDS position col. The pieces of a tile travel global -> VGPR -> LDS.
  int cp_row[kCopies], cp_col[kCopies];
#pragma unroll
  for (int q = 0; q < kCopies; ++q) {
    const int i = min(wave + kMlaWaves * q, kDmaPerTile - 1);
    const int chunk = 64 * i + lane;
    const int r = chunk / kChunksPerRow;
    cp_row[q] = r;
    cp_col[q] = ((chunk % kChunksPerRow) ^ swz(r)) * 16;
  }
  const bool five = wave + kMlaWaves * (kCopies - 1) < kDmaPerTile;   // wave-uniform
  auto load_tile = [&](int tile, i32x4 (&st)[kCopies]) {
    if (tile >= n_tiles) return;
    int64_t rid[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
      const int e = tile * kMlaTile + cp_row[q];
      rid[q] = sh.rowid[e < nvalid ? e : 0];   // rows past the end re-read the split's first row (masked)
    }
#pragma unroll
    for (int q = 0; q < kCopies - 1; ++q)
      st[q] = *reinterpret_cast<const i32x4*>(kvbase + rid[q] * kRowBytes + cp_col[q]);
    if (five) st[kCopies - 1] = *reinterpret_cast<const i32x4*>(kvbase + rid[kCopies - 1] * kRowBytes + cp_col[kCopies - 1]);
  };
  auto store_tile = [&](int tile, const i32x4 (&st)[kCopies]) {
    if (tile >= n_tiles) return;
    uint8_t* dst = sh.kv[tile % kRing] + 16 * lane;
#pragma unroll
    for (int q = 0; q < kCopies - 1; ++q)
      *reinterpret_cast<i32x4*>(dst + 1024 * (wave + kMlaWaves * q)) = st[q];
    if (five) *reinterpret_cast<i32x4*>(dst + 1024 * (wave + kMlaWaves * (kCopies - 1))) = st[kCopies - 1];
  };

  // Consume q here: the compiler then knows its loads have completed, and it
  // places no vector-memory waits inside the tile loop, where they would also
  // drain the (to it invisible) tile copies in flight.
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" :: "v"(qf[ks]));


  f32x4 acc_o[4][4];   // O[heads 16mt + 4g + i][value column 64*wave + 16nt + c]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc_o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // running max (log2 units) of head 16*ht + c
  float l_part = 0.f;        // this lane's share of the softmax denominator

  // score operand: rows c and 16 + c share a swizzle; this wave's half of the row
  const int sw_c = swz(c);
  const int a_row = c * kRowBytes;
  const int kchunk0 = kh * (kMlaDqk / 2 / 8);        // first 16-byte chunk of the half (36)
  // value reads: slot jj < 4 -> row 4g + jj, slot jj >= 4 -> row 16 + 4g + jj - 4
  int v_row[8], v_sw[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = (jj < 4) ? 4 * g + jj : 16 + 4 * g + (jj - 4);
    v_row[jj] = r * kRowBytes + 2 * (c & 7);
    v_sw[jj] = swz(r);
  }

  // ---- helpers of the pipelined loop ----
  // partial scores of `tile` over this wave's half of the contraction
  auto scores = [&](int tile, f32x4& own0, f32x4& own1) {
    const uint8_t* kvt = sh.kv[tile % kRing];
    f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const int o = ((kchunk0 + 4 * ks + g) ^ sw_c) << 4;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kvt + a_row + o);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kvt + a_row + 16 * kRowBytes + o);
      if (ks & 1) {
        sb0 = mfma_bf16(a0, qf[ks], sb0);
        sb1 = mfma_bf16(a1, qf[ks], sb1);
      } else {
        sa0 = mfma_bf16(a0, qf[ks], sa0);
        sa1 = mfma_bf16(a1, qf[ks], sa1);
      }
    }
    own0 = sa0 + sb0;
    own1 = sa1 + sb1;
    if (kh == 1) {
      sh.sx[ht][0][lane] = own0;
      sh.sx[ht][1][lane] = own1;
    }
  };
  // O[64 heads x value columns 64w..64w+63] += P(tile) . V(tile), after the rescale
  auto pv = [&](int tile) {
    const int par = tile & 1;
    const uint8_t* kvt = sh.kv[tile % kRing];
    if (sh.flag[par]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(sh.alpha[par] + 16 * mt + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc_o[mt][nt] *= a4;
      }
    }
    bf16x8 pa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t* pr = sh.pbuf[par] + (16 * mt + c) * kPRow;
      const u16x4 lo = *reinterpret_cast<const u16x4*>(pr + 4 * g);
      const u16x4 hi = *reinterpret_cast<const u16x4*>(pr + 16 + 4 * g);
      const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      pa[mt] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = 8 * wave + 2 * nt + (c >> 3);    // 16-byte chunk of value column 64w + 16nt + c
      u16x8 v;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        v[jj] = *reinterpret_cast<const uint16_t*>(kvt + v_row[jj] + ((col ^ v_sw[jj]) << 4));
      const bf16x8 vb = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc_o[mt][nt] = mfma_bf16(pa[mt], vb, acc_o[mt][nt]);
    }
  };

  // Software pipeline, one tile deep: iteration j overlaps the softmax of tile j
  // (VALU, first-half waves) with P.V of tile j - 1 (MFMA, all waves), stores
  // tile j + 1 (fetched one iteration earlier) into the slot of tile j - 2 and
  // fetches tile j + 2; after barrier C it computes the scores of tile j + 1,
  // and barrier B makes the score halves visible. P, the rescale factors and
  // the rescale flag are double-buffered by tile parity.
  i32x4 st[kCopies];
  f32x4 own0 = {0.f, 0.f, 0.f, 0.f}, own1 = own0;
  if (n_tiles > 0) {
    load_tile(0, st);
    store_tile(0, st);
    load_tile(1, st);
    __syncthreads();                                     // tile 0 visible
    scores(0, own0, own1);
    __syncthreads();                                     // barrier B of tile 0
  }
  // st holds tile + 1 (in flight)
  auto step = [&](int tile, i32x4 (&X)[kCopies]) {
    const int par = tile & 1;
    if (kh == 0) {
      const f32x4 sc0 = own0 + sh.sx[ht][0][lane];
      const f32x4 sc1 = own1 + sh.sx[ht][1][lane];
      // lane (c, g) holds head c, rows 4g+i (sc0) and 16+4g+i (sc1)
      const int rowbase = tile * kMlaTile;
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = sc0[i] * scale_log2;
        sv[4 + i] = sc1[i] * scale_log2;
      }
      if (rowbase + kMlaTile > nvalid) {                 // only the last tile has padding rows
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = (rowbase + 4 * g + i < nvalid) ? sv[i] : -INFINITY;
          sv[4 + i] = (rowbase + 16 + 4 * g + i < nvalid) ? sv[4 + i] : -INFINITY;
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mx = max_over_groups(mx);
      float alpha = 1.f;
      if (mx > m_ref + kRescaleThreshold) {
        alpha = __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
        l_part *= alpha;
      }
      if (__ballot(alpha != 1.f) != 0ull && lane == 0) sh.flag[par] = 1;
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
        l_part += pr[i];
      }
      bf16x2 pb[4];                                      // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = __builtin_convertvector(f32x2{pr[2 * i], pr[2 * i + 1]}, bf16x2);
      uint16_t* prow = sh.pbuf[par] + (16 * ht + c) * kPRow;
      *reinterpret_cast<bf16x2*>(prow + 4 * g) = pb[0];
      *reinterpret_cast<bf16x2*>(prow + 4 * g + 2) = pb[1];
      *reinterpret_cast<bf16x2*>(prow + 16 + 4 * g) = pb[2];
      *reinterpret_cast<bf16x2*>(prow + 16 + 4 * g + 2) = pb[3];
      if (g == 0) sh.alpha[par][16 * ht + c] = alpha;
    }
    if (tile > 0) pv(tile - 1);
    store_tile(tile + 1, X);                             // slot of tile - 2: free since barrier C of tile - 1
    load_tile(tile + 2, X);
    __syncthreads();                                     // barrier C
    if (tid == 0) sh.flag[par ^ 1] = 0;                  // next used by the softmax of tile + 1
    if (tile + 1 < n_tiles) {
      scores(tile + 1, own0, own1);
      __syncthreads();                                   // barrier B of tile + 1
    }
  };
  for (int tile = 0; tile < n_tiles; ++tile) step(tile, st);
  if (n_tiles > 0) pv(n_tiles - 1);

  // ---- finish: denominators, lse, normalized output ----
  if (kh == 0) {
    const float l = sum_over_groups(l_part);
    const int hq = head0 + 16 * ht + c;     // head of this lane in the score layout
    const float lse_val = (l > 0.f) ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    if (g == 0) {
      sh.lsum[16 * ht + c] = l;
      if (S == 1) {
        if (p.lse) p.lse[(int64_t)t * Hm + hq] = lse_val;
      } else {
        p.part_lse[((int64_t)t * S + s) * Hm + hq] = lse_val;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sh.lsum + 16 * mt + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = head0 + 16 * mt + 4 * g + i;
      const float inv = l4[i] > 0.f ? 1.f / l4[i] : 0.f;
      if (S == 1) {
        uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * kMlaDl;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          orow[64 * wave + 16 * nt + c] = f32_to_bf16_bits(acc_o[mt][nt][i] * inv);
      } else {
        float* orow = p.part_o + (((int64_t)t * S + s) * Hm + h) * kMlaDl;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) orow[64 * wave + 16 * nt + c] = acc_o[mt][nt][i] * inv;
      }
    }
  }
}

// LSE merge of the split partials (merge_attn_states generalised to S parts).
// 256 threads cover two heads of one row; each thread owns four value columns.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaParams p) {
  const int t = blockIdx.x;
  const int h = 2 * blockIdx.y + (threadIdx.x >> 7);
  const int d4 = threadIdx.x & 127;                 // value columns 4*d4 .. 4*d4+3
  const int S = p.splits, Hm = p.heads, Dl = p.d_latent;
  if (h >= Hm || 4 * d4 >= Dl) return;
  const float* pl = p.part_lse + (int64_t)t * S * Hm + h;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[(int64_t)s * Hm]);
  float tot = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float l = pl[(int64_t)s * Hm];
    const float wgt = (l == -INFINITY) ? 0.f : __expf(l - mx);
    tot += wgt;
    const f32x4 o = *reinterpret_cast<const f32x4*>(p.part_o + (((int64_t)t * S + s) * Hm + h) * Dl + 4 * d4);
    acc += wgt * o;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  acc *= inv;
  if (d4 == 0 && p.lse) p.lse[(int64_t)t * Hm + h] = tot > 0.f ? mx + __logf(tot) : -INFINITY;
  if (kBf16Out) {
    const bf16x4 o = __builtin_convertvector(acc, bf16x4);
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * Dl + 4 * d4) = o;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + ((int64_t)t * Hm + h) * Dl + 4 * d4) = acc;
  }
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
  if (max_splits > 16) max_splits = 16;
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
  hipLaunchKernelGGL(mla_bf16_kernel, dim3((unsigned)blocks), dim3(kMlaThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel<true>, dim3(T, (p.heads + 1) / 2), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_f32_kernel, dim3(p.batch.num_rows, p.heads), dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
