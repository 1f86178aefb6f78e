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
// bf16 path (Dl = 512, Dr = 64, Hm a multiple of 64). One work-group of four
// waves (one per SIMD) handles one (row, split of the top-k list, group of 64
// heads); wave w owns heads 16w .. 16w+15 of the group outright, so scores,
// softmax and P.V of those heads never leave the wave:
//   * the split's positions are resolved once through the block table into
//     cache-row ids in LDS, skipping -1 / out-of-range entries (so the -1 tail
//     of short rows costs nothing);
//   * gathered rows arrive 32 at a time straight from HBM into a ring of four
//     LDS tiles (global_load_lds, 16 bytes per lane, no register staging); two
//     tiles are in flight while one is scored and the previous one multiplied
//     into the output. Rows are stored dense with an XOR swizzle of their
//     16-byte chunks, which keeps both LDS read patterns below free of bank
//     conflicts;
//   * scores: S^T[32 rows x 16 heads] = C_tile . Q^T over the 576-wide
//     contraction with v_mfma_f32_16x16x32_bf16 (rows = M from LDS, heads = N:
//     the wave keeps its 16 heads x 576 of q in registers);
//   * online softmax in fp32, base 2, with lazy rescaling: the running maximum
//     of a head only moves when a tile exceeds it by more than 2^8, so the
//     accumulator rescale is skipped on most tiles;
//   * the score accumulator of lane (c, g) holds head c at rows {4g+i, 16+4g+i},
//     which is exactly the A operand (head c, eight rows of the contraction)
//     of O[16 heads x 512] += P . V_tile, so P goes from registers to the MFMA
//     without an LDS round trip. V arrives as the B operand through the gfx950
//     transposing LDS read (ds_read_b64_tr_b16), two per 16 value columns;
//   * the scores of tile j + 1 are issued before the softmax and P.V of tile j,
//     so the wave has MFMA work while its softmax runs;
//   * single split: out = O / l in bf16 and lse; several splits: fp32 partials
//     (O / l, lse) merged by mla_combine_kernel.
// Work-groups are ordered so that the head groups of one (row, split) unit, and
// neighbouring units, land on the same XCD (work-group i runs on XCD i % 8) and
// share the gathered rows through that XCD's L2.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kMlaThreads = 256;
constexpr int kMlaWaves = kMlaThreads / kWave;          // 4
constexpr int kRowBytes = kMlaDqk * 2;                  // 1152: one cached latent row
constexpr int kChunksPerRow = kRowBytes / 16;           // 72 chunks of 16 bytes
constexpr int kTileBytes = kMlaTile * kRowBytes;        // 36864
constexpr int kPiecesPerTile = kTileBytes / 1024;       // 36 wave-wide 1 KB copies
constexpr int kPiecesPerWave = kPiecesPerTile / kMlaWaves;   // 9
constexpr int kRing = 4;                                // LDS tile slots
constexpr int kEntriesPerThread = kMlaMaxEntriesPerBlock / kMlaThreads;  // 8
constexpr int kKSteps = kMlaDqk / 32;                   // 18 K-steps of 32
constexpr int kVTiles = kMlaDl / 16;                    // 32 value-column tiles
constexpr float kRescaleThreshold = 8.0f;               // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

struct MlaShared {
  // Gathered rows, dense (1152 B per row). Inside row r the 16-byte chunk c is
  // stored at chunk position c ^ swz(r) (see swz).
  alignas(16) uint8_t kv[kRing][kTileBytes];
  int32_t rowid[kMlaMaxEntriesPerBlock];
  int wave_sum[kMlaWaves];
};

// Chunk swizzle of row r: the low three bits of r. With it the score operand
// reads (sixteen rows, one logical chunk each) and the transposed value reads
// (sixteen rows x 32 bytes) both run at the conflict-free LDS rate (measured on
// gfx950; rows are 1152 bytes apart). Rows r and r + 16 share the swizzle.
__device__ __forceinline__ int swz(int row) { return row & 7; }

// max / sum of v over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups),
// with the gfx950 lane swaps (VALU, no LDS round trip)
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

// transposing LDS read: lane 4k + m of each 16-lane block names 8 bytes (four
// bf16) of row k; lane i of the block receives element i % 4 of lane
// 4 * kk + i / 4's bytes in slot kk, i.e. one column of four rows
__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
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

  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  const int addressable = bv.max_pages_per_seq * P;
  if (seq_len > addressable) seq_len = addressable;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;

  const int head0 = hg * kMlaHeadsPerGroup + 16 * wave;   // this wave's first head
  const int Hm = p.heads;

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
  // q (head c of the wave, all 576: the N operand) is fetched after the page
  // lookups so that waiting for those (vector loads complete in order) does not
  // also wait for q
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)t * Hm + head0 + c) * kMlaDqk;
  bf16x8 qf[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);
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

  // A tile is 36 copies of 1 KB; copy i = wave + 4j covers LDS chunks
  // 64i .. 64i+63, lane l taking chunk 64i + l of the dense tile: row
  // r = chunk / 72, LDS chunk position col = chunk % 72, which holds the
  // logical chunk col ^ swz(r) of the row.
  // source row ids of this wave's copies of `tile`
  auto fetch_rows = [&](int tile, int (&rid)[kPiecesPerWave]) {
#pragma unroll
    for (int j = 0; j < kPiecesPerWave; ++j) {
      const int r = (64 * (wave + kMlaWaves * j) + lane) / kChunksPerRow;
      const int e = tile * kMlaTile + r;
      rid[j] = sh.rowid[e < nvalid ? e : 0];   // rows past the end re-read the split's first row (masked)
    }
  };
  // copies j0 .. j1-1 of this wave for `tile`
  auto issue_pieces = [&](int tile, const int (&rid)[kPiecesPerWave], int j0, int j1) {
    const uint32_t dst = lds_offset(sh.kv[tile % kRing]);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int chunk = 64 * (wave + kMlaWaves * j) + lane;
      const int r = chunk / kChunksPerRow;
      const int col = ((chunk - r * kChunksPerRow) ^ swz(r)) * 16;
      lds_dma16(kvbase + (int64_t)rid[j] * kRowBytes + col, dst + 1024 * (wave + kMlaWaves * j));
    }
  };
  auto issue_tile = [&](int tile) {
    int rid[kPiecesPerWave];
    fetch_rows(tile, rid);
    issue_pieces(tile, rid, 0, kPiecesPerWave);
  };

  // Consume q here: the compiler then knows its loads have completed, and it
  // places no vector-memory waits inside the tile loop, where they would also
  // drain the (to it invisible) tile copies in flight.
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" : "+a"(qf[ks]));

  // score operand (A): lane (c, g) reads row c (and 16 + c) of the tile, 16-byte
  // chunk 4 ks + g of the row. With ks = 2a + u the swizzled position is
  // 8a + ((4u + g) ^ swz(c)): a per-lane base plus an immediate.
  const int sw_c = swz(c);
  const int a_off0 = c * kRowBytes + (((g) ^ sw_c) << 4);
  const int a_off1 = c * kRowBytes + (((4 + g) ^ sw_c) << 4);
  // value operand (B): for rows 16h + 4g + (c >> 2) and value columns
  // 16nt + 4(c & 3) .. +3; with nt = 4a + u the chunk is 8a + ((2u + ((c & 3) >> 1)) ^ swz(row))
  int v_off[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 16 * h + 4 * g + (c >> 2);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v_off[h][u] = r * kRowBytes + (((2 * u + ((c & 3) >> 1)) ^ swz(r)) << 4) + ((c & 1) << 3);
  }

  f32x4 acc_o[kVTiles];   // O[head 4g + i][value column 16 nt + c] (PV accumulator layout)
#pragma unroll
  for (int nt = 0; nt < kVTiles; ++nt) acc_o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // running max (log2 units) of head c
  float l_part = 0.f;        // this lane's share of head c's softmax denominator

  // Score operands of K-steps 3b .. 3b+2 (rows c and 16 + c of the tile) and
  // their MFMAs into S^T: s0 rows 4g+i, s1 rows 16+4g+i, head c.
  constexpr int kKB = 3;                                 // K-steps per batch
  constexpr int kKBatches = kKSteps / kKB;               // 6
  auto read_k = [&](const uint8_t* kvt, int b, bf16x8 (&dst)[kKB][2]) {
#pragma unroll
    for (int u = 0; u < kKB; ++u) {
      const int ks = kKB * b + u;
      const int off = ((ks & 1) ? a_off1 : a_off0) + 128 * (ks >> 1);
      dst[u][0] = *reinterpret_cast<const bf16x8*>(kvt + off);
      dst[u][1] = *reinterpret_cast<const bf16x8*>(kvt + off + 16 * kRowBytes);
    }
  };
  auto mfma_k = [&](int b, const bf16x8 (&op)[kKB][2], f32x4& s0, f32x4& s1) {
#pragma unroll
    for (int u = 0; u < kKB; ++u) {
      s0 = mfma_bf16(op[u][0], qf[kKB * b + u], s0);
      s1 = mfma_bf16(op[u][1], qf[kKB * b + u], s1);
    }
  };
  // value operands of column tiles 8n .. 8n+7 (two transposing reads each)
  constexpr int kVB = 8;
  auto read_v = [&](const uint8_t* kvt, int n, i16x4 (&lo)[kVB], i16x4 (&hi)[kVB]) {
#pragma unroll
    for (int u = 0; u < kVB; ++u) {
      const int nt = kVB * n + u;
      const int imm = 128 * (nt >> 2);
      lo[u] = lds_read_tr16(kvt + v_off[0][nt & 3] + imm);
      hi[u] = lds_read_tr16(kvt + v_off[1][nt & 3] + imm);
    }
  };
  auto scores = [&](int tile, f32x4& s0, f32x4& s1) {   // (prologue only)
    const uint8_t* kvt = sh.kv[tile % kRing];
    s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    s1 = s0;
#pragma unroll
    for (int b = 0; b < kKBatches; ++b) {
      bf16x8 op[kKB][2];
      read_k(kvt, b, op);
      mfma_k(b, op, s0, s1);
    }
  };

  // ---- tile loop ----
  // Iteration j: wait for tile j + 1, barrier (every wave is done with tile
  // j - 1, whose slot takes tile j + 3), scores of tile j + 1, softmax and
  // P.V of tile j, with the copies of tile j + 3 spread over the iteration.
  // Tiles past the end are copied too (their rows all re-read the split's
  // first row, a few cache lines) and never used: the loop has no branches
  // around copies, waits or MFMAs, and every wait is the same.
  f32x4 cur0 = {0.f, 0.f, 0.f, 0.f}, cur1 = cur0;
  if (n_tiles > 0) {
    issue_tile(0);
    issue_tile(1);
    issue_tile(2);
    wait_vmcnt<2 * kPiecesPerWave>();
    __syncthreads();
    scores(0, cur0, cur1);
  }
  for (int tile = 0; tile < n_tiles; ++tile) {
    wait_vmcnt<kPiecesPerWave>();                        // tile + 1 has landed, tile + 2 may be in flight
    __syncthreads();
    int rid[kPiecesPerWave];
    fetch_rows(tile + 3, rid);
    issue_pieces(tile + 3, rid, 0, 3);

    // The iteration is one software pipeline, fenced so that the compiler
    // keeps it: operand reads of the next batch are issued before the MFMAs
    // of the current one, first over the six score batches of tile + 1, then
    // over the four value batches of tile. The softmax of tile (VALU) runs
    // while the first score operands are in flight. (The last iteration
    // scores a stale slot and discards the result.)
    const uint8_t* kvn = sh.kv[(tile + 1) % kRing];
    const uint8_t* kvt = sh.kv[tile % kRing];
    bf16x8 kop[2][kKB][2];
    i16x4 vlo[2][kVB], vhi[2][kVB];
    read_k(kvn, 0, kop[0]);
    __builtin_amdgcn_sched_barrier(0);

    // softmax of tile: lane (c, g) holds head c, rows 4g+i (cur0) and 16+4g+i (cur1)
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = cur0[i] * scale_log2;
      sv[4 + i] = cur1[i] * scale_log2;
    }
    const int rows_left = nvalid - tile * kMlaTile;      // padding rows (last tile only) -> -inf
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (4 * g + i < rows_left) ? sv[i] : -INFINITY;
      sv[4 + i] = (16 + 4 * g + i < rows_left) ? sv[4 + i] : -INFINITY;
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
    float pr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
      l_part += pr[i];
    }
    bf16x8 pa;                                           // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 two = __builtin_convertvector(f32x2{pr[2 * i], pr[2 * i + 1]}, bf16x2);
      pa[2 * i] = two[0];
      pa[2 * i + 1] = two[1];
    }
    if (__ballot(alpha != 1.f) != 0ull) {               // rare: rescale O rows (heads 4g + i)
      float a4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
      for (int nt = 0; nt < kVTiles; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc_o[nt][i] *= a4[i];
    }

    // scores of tile + 1
    f32x4 nxt0 = {0.f, 0.f, 0.f, 0.f}, nxt1 = nxt0;
#pragma unroll
    for (int b = 0; b < kKBatches; ++b) {
      if (b + 1 < kKBatches) read_k(kvn, b + 1, kop[(b + 1) & 1]);
      else read_v(kvt, 0, vlo[0], vhi[0]);
      if (b == 1) issue_pieces(tile + 3, rid, 3, 6);
      if (b == 3) issue_pieces(tile + 3, rid, 6, kPiecesPerWave);
      __builtin_amdgcn_sched_barrier(0);
      mfma_k(b, kop[b & 1], nxt0, nxt1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // O += P . V(tile)
#pragma unroll
    for (int n = 0; n < kVTiles / kVB; ++n) {
      if (n + 1 < kVTiles / kVB) read_v(kvt, n + 1, vlo[(n + 1) & 1], vhi[(n + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kVB; ++u) {
        const i16x8 v8 = __builtin_shufflevector(vlo[n & 1][u], vhi[n & 1][u], 0, 1, 2, 3, 4, 5, 6, 7);
        acc_o[kVB * n + u] = mfma_bf16(pa, __builtin_bit_cast(bf16x8, v8), acc_o[kVB * n + u]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    cur0 = nxt0;
    cur1 = nxt1;
  }
  wait_vmcnt<0>();                                       // no copy into LDS outlives the loop

  // ---- finish: denominators, lse, normalized output ----
  const float l = sum_over_groups(l_part);               // head c
  if (g == 0) {
    const float lse_val = (l > 0.f) ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
    if (S == 1) {
      if (p.lse) p.lse[(int64_t)t * Hm + head0 + c] = lse_val;
    } else {
      p.part_lse[((int64_t)t * S + s) * Hm + head0 + c] = lse_val;
    }
  }
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float li = __shfl(l, 4 * g + i, kWave);        // head 4g + i
    inv[i] = li > 0.f ? 1.f / li : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = head0 + 4 * g + i;
    if (S == 1) {
      uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * kMlaDl;
#pragma unroll
      for (int nt = 0; nt < kVTiles; ++nt) orow[16 * nt + c] = f32_to_bf16_bits(acc_o[nt][i] * inv[i]);
    } else {
      float* orow = p.part_o + (((int64_t)t * S + s) * Hm + h) * kMlaDl;
#pragma unroll
      for (int nt = 0; nt < kVTiles; ++nt) orow[16 * nt + c] = acc_o[nt][i] * inv[i];
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
