// Sparse MLA over an fp8 latent cache (vLLM MLA page, the decode path under
// fp8_attention: the absorbed query is quantized with the layer's q scale by
// scaled_fp8_quant and the cache is written in fp8 with the layer's k scale).
// q and the cached rows hold OCP E4M3 codes with one scale per tensor:
//
//   z_i  = softmax_scale * q_scale * kv_scale * (q8[t,h,:] . C8_i)
//   out  = kv_scale * sum_i softmax(z)_i * C8_i[:512]           (bf16)
//   lse  = log sum_i exp(z_i)
//
// The structure is that of the bf16 kernel (one work-group of eight waves per
// (row, split, 64 heads); four score waves and four value waves; gathered rows
// stream through a four-slot LDS ring with global_load_lds; online base-2
// softmax with lazy rescaling; P exchanged through LDS between two barriers),
// with what the one-byte rows change:
//   * a row is 576 bytes and a tile holds 64 rows (the same 36 KB, so the same
//     36 one-kilobyte copies and ring depth cover twice the rows);
//   * scores: v_mfma_f32_16x16x128_f8f6f4 with the rows as M (lane (c, g): row
//     16 rb + c, bytes 32 g .. 32 g + 31 of a 128-byte block) and the heads as
//     N (q codes held in registers): four blocks for the 512 latent bytes and
//     one for the 64 rope bytes, whose upper half is zero on both sides;
//   * values: the gfx950 8-bit transposing LDS read (ds_read_b64_tr_b8) gives
//     lane (c, g) one value column of rows 8 g .. 8 g + 7 of a 32-row block,
//     which converts exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8) and feeds
//     the bf16 MFMA with P^T as B, so P stays bf16 as in the bf16 kernel.
// Swizzle: inside row r the 16-byte chunk q sits at chunk q ^ ((r >> 2) & 3)
// (rows are 576 bytes apart). With it the transposing value reads (8 rows x
// 16 bytes per 16-lane block) run at ~234 B/clk per CU and the score reads at
// ~246 B/clk, the latter only because the sixteen M indices of a score row
// block are the tile rows k and k + 8 side by side (measured on gfx950 by a
// search over chunk swizzles and row orders: no swizzle serves both read
// patterns with the plain row order). P rows are padded to 72 elements so that
// the P^T reads of sixteen heads fall on distinct banks.
#include <cfloat>

#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kF8Threads = 512;
constexpr int kF8Waves = kF8Threads / kWave;            // 8
constexpr int kF8RoleWaves = kF8Waves / 2;              // 4 score, 4 value
constexpr int kF8Tile = 64;                             // rows per tile
constexpr int kF8RowBytes = kMlaDqk;                    // 576
constexpr int kF8Chunks = kF8RowBytes / 16;             // 36
constexpr int kF8TileBytes = kF8Tile * kF8RowBytes;     // 36864
constexpr int kF8Pieces = kF8TileBytes / 1024;          // 36
constexpr int kF8PiecesMax = (kF8Pieces + kF8Waves - 1) / kF8Waves;   // 5 (waves 0..3), else 4
constexpr int kF8Ring = 4;
constexpr int kF8EntriesPerThread = kMlaFp8MaxEntriesPerBlock / kF8Threads;   // 2
constexpr int kF8RowBlocks = kF8Tile / 16;              // 4
constexpr int kF8KBlocks = 5;                           // 4 latent blocks of 128 bytes + the rope half block
constexpr int kF8PStride = kF8Tile + 8;                 // bf16 per head row of P
constexpr int kF8PvNT = kMlaDl / kF8RoleWaves / 16;     // 8 value-column tiles per value wave
constexpr int kF8PvHT = kMlaHeadsPerGroup / 16;         // 4 head tiles
constexpr int kF8PvKB = kF8Tile / 32;                   // 2 contraction blocks of 32 rows
constexpr int kF8VAhead = 4;                            // value tiles read ahead of their MFMAs
constexpr float kF8RescaleThreshold = 8.0f;             // log2 units
constexpr float kF8Log2e = 1.4426950408889634f;
constexpr float kF8Ln2 = 0.6931471805599453f;
static_assert(kF8Pieces > (kF8PiecesMax - 1) * kF8Waves &&
              kF8Pieces <= kF8PiecesMax * kF8RoleWaves + (kF8PiecesMax - 1) * kF8RoleWaves,
              "waves 0..3 copy kF8PiecesMax pieces of a tile, waves 4..7 one fewer");

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct F8Shared {
  alignas(16) uint8_t kv[kF8Ring][kF8TileBytes];        // gathered rows, swizzled chunks
  alignas(16) uint16_t p[kMlaHeadsPerGroup * kF8PStride];   // P of one tile, [head][row] bf16
  alignas(16) float alpha[kMlaHeadsPerGroup];           // rescale factor of the tile; at the end 1 / l
  alignas(16) int flag[kF8RoleWaves];                   // some head of score wave w rescaled
  int32_t rowid[kMlaFp8MaxEntriesPerBlock];
  int wave_sum[kF8Waves];
};

__device__ __forceinline__ int swz8(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, const f32x4& c) {
  // format 0 = E4M3 for both operands, no block scales (the unscaled form)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8-bit transposing LDS read: lane 2 r + m of each 16-lane block names the 8
// bytes m of row r of an 8 x 16-byte block; lane i of the block receives byte i
// of every row, rows 0..7 in order (one column of eight rows)
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// eight E4M3 codes (byte j = element j) -> eight bf16 (exact)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(const i32x2& v) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)v[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Wait until at most `tiles` tiles of this wave's copies are outstanding.
__device__ __forceinline__ void wait_tiles8(int tiles, bool five) {
  if (five) {
    if (tiles >= 2) wait_vmcnt<2 * kF8PiecesMax>();
    else if (tiles == 1) wait_vmcnt<kF8PiecesMax>();
    else wait_vmcnt<0>();
  } else {
    if (tiles >= 2) wait_vmcnt<2 * (kF8PiecesMax - 1)>();
    else if (tiles == 1) wait_vmcnt<kF8PiecesMax - 1>();
    else wait_vmcnt<0>();
  }
}

template <bool kPosScale>
__global__ __launch_bounds__(kF8Threads) void mla_fp8_kernel(MlaParams p) {
  __shared__ F8Shared sh;
  const BatchView& bv = p.batch;
  const int T = bv.num_rows;
  const int HG = p.heads / kMlaHeadsPerGroup;
  const int S = p.splits;

  // work-group -> (row t, split s, head group hg), XCD-aware as in the bf16 kernel
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
  const bool scorer = wave < kF8RoleWaves;
  const int rw = wave & (kF8RoleWaves - 1);
  const bool five = wave + kF8Waves * (kF8PiecesMax - 1) < kF8Pieces;

  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  const int addressable = bv.max_pages_per_seq * P;
  if (seq_len > addressable) seq_len = addressable;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;

  const int Hm = p.heads;
  const int hbase = hg * kMlaHeadsPerGroup;
  const int hl_s = 16 * rw + c;               // score waves: this lane's head inside the group

  // ---- this split's entries -> compacted cache-row ids ----
  const int e_begin = s * p.entries_per_split;
  int e_cnt = p.k - e_begin;
  if (e_cnt > p.entries_per_split) e_cnt = p.entries_per_split;
  if (e_cnt < 0) e_cnt = 0;
  const int32_t* idx = p.topk_idx + (int64_t)t * p.k + e_begin;
  int pos[kF8EntriesPerThread], page[kF8EntriesPerThread];
#pragma unroll
  for (int q = 0; q < kF8EntriesPerThread; ++q) {
    const int e = kF8EntriesPerThread * tid + q;
    pos[q] = (e < e_cnt) ? idx[e] : -1;
  }
#pragma unroll
  for (int q = 0; q < kF8EntriesPerThread; ++q) {
    const bool in = pos[q] >= 0 && pos[q] < seq_len;
    page[q] = in ? bt[pos[q] / P] : -1;
  }
  int nmine = 0;
#pragma unroll
  for (int q = 0; q < kF8EntriesPerThread; ++q) nmine += (page[q] >= 0 && page[q] < bv.num_pages) ? 1 : 0;
  const int incl = (int)wave_inclusive_scan((uint32_t)nmine);
  if (lane == kWave - 1) sh.wave_sum[wave] = incl;
  __syncthreads();
  int nvalid = 0, w_off = 0;
#pragma unroll
  for (int w = 0; w < kF8Waves; ++w) {
    const int v = sh.wave_sum[w];
    w_off += (w < wave) ? v : 0;
    nvalid += v;
  }
  {
    int o = w_off + incl - nmine;
#pragma unroll
    for (int q = 0; q < kF8EntriesPerThread; ++q)
      if (page[q] >= 0 && page[q] < bv.num_pages) sh.rowid[o++] = page[q] * P + pos[q] % P;
  }
  __syncthreads();

  const float scale_log2 = p.softmax_scale * p.q_scale * p.kv_scale * kF8Log2e;
  const uint8_t* kvbase = static_cast<const uint8_t*>(p.kv);
  const int n_tiles = (nvalid + kF8Tile - 1) / kF8Tile;

  // ---- copies: copy i = wave + 8 j covers LDS chunks 64 i .. 64 i + 63 of the
  // dense tile; lane l takes chunk 64 i + l: row r = chunk / 36, LDS chunk
  // position col, holding the row's logical chunk col ^ swz8(r). Rows past
  // the split's valid entries re-read its first row (their scores are masked).
  auto fetch_rows = [&](int tile, int (&rid)[kF8PiecesMax]) {
    if ((tile + 1) * kF8Tile <= nvalid) {              // uniform: every row of the tile is valid
#pragma unroll
      for (int j = 0; j < kF8PiecesMax; ++j) {
        const int pc = min(wave + kF8Waves * j, kF8Pieces - 1);
        rid[j] = sh.rowid[tile * kF8Tile + (64 * pc + lane) / kF8Chunks];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kF8PiecesMax; ++j) {
        const int pc = min(wave + kF8Waves * j, kF8Pieces - 1);
        const int e = tile * kF8Tile + (64 * pc + lane) / kF8Chunks;
        rid[j] = sh.rowid[e < nvalid ? e : 0];
      }
    }
  };
  auto issue_pieces = [&](int tile, const int (&rid)[kF8PiecesMax], int j0, int j1) {
    const uint32_t dst = lds_offset(sh.kv[tile % kF8Ring]);
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      if (j == kF8PiecesMax - 1 && !five) break;
      const int pc = wave + kF8Waves * j;
      const int chunk = 64 * pc + lane;
      const int r = chunk / kF8Chunks;
      const int col = ((chunk - r * kF8Chunks) ^ swz8(r)) * 16;
      lds_dma16(kvbase + (int64_t)rid[j] * kF8RowBytes + col, dst + 1024 * pc);
    }
  };

  constexpr int kAhead = kF8Ring - 1;
  int rid_next[kF8PiecesMax];

  if (scorer) {
    // ================= score waves =================
    // q (the N operand: lane (c, g) holds head hbase + hl_s, bytes 32 g ..
    // 32 g + 31 of each 128-byte block; the rope block's upper half is zero),
    // loaded after the copies of tile 0 and consumed at once so that no
    // compiler vector-memory wait lands inside the tile loop.
    if (n_tiles > 0) {
      fetch_rows(0, rid_next);
      issue_pieces(0, rid_next, 0, kF8PiecesMax);
    }
    i32x8 qf[kF8KBlocks];
    {
      const uint8_t* qrow = static_cast<const uint8_t*>(p.q) + ((int64_t)t * Hm + hbase + hl_s) * kF8RowBytes;
#pragma unroll
      for (int kb = 0; kb < kF8KBlocks; ++kb) {
        const int off = kb < 4 ? 128 * kb + 32 * g : 512 + 32 * (g & 1);
        const i32x4 lo = *reinterpret_cast<const i32x4*>(qrow + off);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(qrow + off + 16);
        i32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (kb == 4 && g >= 2) v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        qf[kb] = v;
      }
#pragma unroll
      for (int kb = 0; kb < kF8KBlocks; ++kb) asm volatile("" : "+v"(qf[kb]));
    }
    for (int tl = 1; tl < kAhead && tl < n_tiles; ++tl) {
      fetch_rows(tl, rid_next);
      issue_pieces(tl, rid_next, 0, kF8PiecesMax);
    }
    if (n_tiles > kAhead) fetch_rows(kAhead, rid_next);

    float m_ref = -INFINITY;
    float l_part = 0.f;

    // row operand (A) of block kb: M index c of row block rb is tile row
    // 16 rb + (c >> 1) + 8 (c & 1) (rows k and k + 8 side by side: with the
    // chunk swizzle the sixteen 16-byte reads of a quarter wave then fall on
    // distinct banks, measured on gfx950, where rows 16 rb + c conflict two-way);
    // lane (c, g) reads logical chunks 8 kb + 2 g and + 1 of it (the rope
    // block: chunks 32 + 2 (g & 1), + 1, zeroed for g >= 2 after the read, so
    // every address stays in its row)
    const int lo_chunk = 2 * (g & 1);
    const int a_row = (c >> 1) + 8 * (c & 1);
    auto read_kb = [&](const uint8_t* kvt, int kb, i32x8 (&dst)[kF8RowBlocks]) {
#pragma unroll
      for (int rb = 0; rb < kF8RowBlocks; ++rb) {
        const int row = 16 * rb + a_row;
        const int q0 = kb < 4 ? 8 * kb + 2 * g : 32 + lo_chunk;
        const uint8_t* base = kvt + row * kF8RowBytes;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(base + ((q0 ^ swz8(row)) << 4));
        const i32x4 hi = *reinterpret_cast<const i32x4*>(base + (((q0 + 1) ^ swz8(row)) << 4));
        i32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (kb == 4 && g >= 2) v = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
        dst[rb] = v;
      }
    };
    // S[rows, head hl_s] of one tile: lane (c, g) ends with M indices 4 g + i
    // of each row block, i.e. tile rows 16 rb + 2 g + (i >> 1) + 8 (i & 1)
    auto scores = [&](const uint8_t* kvt, f32x4 (&sacc)[kF8RowBlocks], int copy_tile, int (&rid)[kF8PiecesMax]) {
      i32x8 op[2][kF8RowBlocks];
#pragma unroll
      for (int rb = 0; rb < kF8RowBlocks; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      read_kb(kvt, 0, op[0]);
#pragma unroll
      for (int kb = 0; kb < kF8KBlocks; ++kb) {
        if (kb + 1 < kF8KBlocks) read_kb(kvt, kb + 1, op[(kb + 1) & 1]);
        if (copy_tile >= 0 && kb < 3) issue_pieces(copy_tile, rid, 2 * kb, min(2 * kb + 2, kF8PiecesMax));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < kF8RowBlocks; ++rb) sacc[rb] = mfma_fp8_k128(op[kb & 1][rb], qf[kb], sacc[rb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // online softmax of one tile: the lane's 16 probabilities as bf16 pairs
    // (pa[rb][0]: tile rows 16 rb + 2 g, + 1; pa[rb][1]: 16 rb + 8 + 2 g, + 1)
    // and its head's rescale factor
    auto softmax = [&](int tile, const f32x4 (&sacc)[kF8RowBlocks], bf16x2 (&pa)[kF8RowBlocks][2], float* alpha) {
      // With a positive scale the scores stay unscaled here: rounding is
      // monotone, so the maximum of the scaled scores is the scaled maximum,
      // and the scale enters each exponent through one fma.
      const int rows_left = nvalid - tile * kF8Tile;
      float sv[4 * kF8RowBlocks];
#pragma unroll
      for (int rb = 0; rb < kF8RowBlocks; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * rb + i] = kPosScale ? sacc[rb][i] : sacc[rb][i] * scale_log2;
      if (rows_left < kF8Tile) {                         // uniform: the last, partial tile
#pragma unroll
        for (int rb = 0; rb < kF8RowBlocks; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * rb + 2 * g + (i >> 1) + 8 * (i & 1);
            sv[4 * rb + i] = (row < rows_left) ? sv[4 * rb + i] : -INFINITY;
          }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 4 * kF8RowBlocks; ++i) mx = fmaximum(mx, sv[i]);
      mx = max_over_groups(mx);                        // a NaN score makes the head's output NaN either way
      if (kPosScale) mx *= scale_log2;
      *alpha = 1.f;
      if (mx > m_ref + kF8RescaleThreshold) {
        *alpha = __builtin_amdgcn_exp2f(m_ref - mx);
        m_ref = mx;
        l_part *= *alpha;
      }
#pragma unroll
      for (int rb = 0; rb < kF8RowBlocks; ++rb) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(kPosScale ? fmaf(sv[4 * rb + i], scale_log2, -m_ref) : sv[4 * rb + i] - m_ref);
          l_part += pr[i];
        }
        pa[rb][0] = __builtin_convertvector(f32x2{pr[0], pr[2]}, bf16x2);   // rows 2 g, 2 g + 1
        pa[rb][1] = __builtin_convertvector(f32x2{pr[1], pr[3]}, bf16x2);   // rows 8 + 2 g, 8 + 2 g + 1
      }
    };
    auto publish = [&](const bf16x2 (&pa)[kF8RowBlocks][2], float alpha) {   // between B1 and B2
#pragma unroll
      for (int rb = 0; rb < kF8RowBlocks; ++rb) {
        *reinterpret_cast<bf16x2*>(&sh.p[hl_s * kF8PStride + 16 * rb + 2 * g]) = pa[rb][0];
        *reinterpret_cast<bf16x2*>(&sh.p[hl_s * kF8PStride + 16 * rb + 8 + 2 * g]) = pa[rb][1];
      }
      if (g == 0) sh.alpha[hl_s] = alpha;
      const bool any = __ballot(alpha != 1.f) != 0ull;
      if (lane == 0) sh.flag[rw] = any ? 1 : 0;
    };

    if (n_tiles > 0) {                                 // prologue: tile 0
      wait_tiles8(min(n_tiles, kAhead) - 1, five);
      __syncthreads();
      f32x4 sacc[kF8RowBlocks];
      scores(sh.kv[0], sacc, -1, rid_next);
      float alpha;
      bf16x2 pa[kF8RowBlocks][2];
      softmax(0, sacc, pa, &alpha);
      publish(pa, alpha);
      wait_tiles8(min(n_tiles, kAhead) - 2, five);
      __syncthreads();
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      const bool more = tile + 1 < n_tiles;
      bf16x2 pa[kF8RowBlocks][2];
      float alpha = 1.f;
      const int last = n_tiles - 1;
      const int copy_tile = tile + kAhead <= last ? tile + kAhead : -1;
      if (more) {
        f32x4 sacc[kF8RowBlocks];
        scores(sh.kv[(tile + 1) % kF8Ring], sacc, copy_tile, rid_next);
        softmax(tile + 1, sacc, pa, &alpha);
      } else if (copy_tile >= 0) {
        issue_pieces(copy_tile, rid_next, 0, kF8PiecesMax);
      }
      if (copy_tile >= 0 && copy_tile + 1 <= last) fetch_rows(copy_tile + 1, rid_next);
      __syncthreads();                                 // B1: every value wave holds P of the tile
      if (more) publish(pa, alpha);
      wait_tiles8(min(tile + kAhead, last) - (tile + 2), five);
      __syncthreads();                                 // B2
    }
    const float l = sum_over_groups(l_part);
    if (g == 0) {
      const float lse_val = (l > 0.f) ? (m_ref + log2f(l)) * kF8Ln2 : -INFINITY;
      if (S == 1) {
        if (p.lse) p.lse[(int64_t)t * Hm + hbase + hl_s] = lse_val;
      } else {
        p.part_lse[((int64_t)t * S + s) * Hm + hbase + hl_s] = lse_val;
      }
      sh.alpha[hl_s] = l > 0.f ? p.kv_scale / l : 0.f;
    }
    __syncthreads();
  } else {
    // ================= value waves =================
    for (int tl = 0; tl < kAhead && tl < n_tiles; ++tl) {
      fetch_rows(tl, rid_next);
      issue_pieces(tl, rid_next, 0, kF8PiecesMax);
    }
    if (n_tiles > kAhead) fetch_rows(kAhead, rid_next);
    f32x4 acc_o[kF8PvHT][kF8PvNT];   // O[head 16 hb + c][value column 128 rw + 16 nt + 4 g + i]
#pragma unroll
    for (int hb = 0; hb < kF8PvHT; ++hb)
#pragma unroll
      for (int nt = 0; nt < kF8PvNT; ++nt) acc_o[hb][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // value operand (A of O^T += V^T P^T): block g of 16 lanes reads rows
    // 32 kb + 8 g .. + 7, lane 2 r + m naming bytes 8 m of row 8 g + r's chunk
    // 8 rw + nt; with nt = 4 a + u the chunk sits at 8 rw + 4 a + (u ^ swz8(row)).
    const int vr = 8 * g + (c >> 1);
    int v_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v_off[u] = vr * kF8RowBytes + ((8 * rw + (u ^ swz8(vr))) << 4) + ((c & 1) << 3);
    // P^T operand (B): lane (c, g) reads P[head 16 hb + c][32 kb + 8 g .. + 7]
    const int p_off = c * kF8PStride + 8 * g;

    if (n_tiles > 0) {
      wait_tiles8(min(n_tiles, kAhead) - 1, five);
      __syncthreads();
      wait_tiles8(min(n_tiles, kAhead) - 2, five);
      __syncthreads();
    }
    for (int tile = 0; tile < n_tiles; ++tile) {
      const uint8_t* kvt = sh.kv[tile % kF8Ring];
      const int last = n_tiles - 1;
      const int copy_tile = tile + kAhead <= last ? tile + kAhead : -1;
      const i32x4 fl4 = *reinterpret_cast<const i32x4*>(sh.flag);
      bf16x8 pb[kF8PvKB][kF8PvHT];
#pragma unroll
      for (int kb = 0; kb < kF8PvKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < kF8PvHT; ++hb)
          pb[kb][hb] = *reinterpret_cast<const bf16x8*>(&sh.p[16 * hb * kF8PStride + p_off + 32 * kb]);
      if (__builtin_amdgcn_readfirstlane(fl4[0] | fl4[1] | fl4[2] | fl4[3])) {
#pragma unroll
        for (int hb = 0; hb < kF8PvHT; ++hb) {
          const float a = sh.alpha[16 * hb + c];
#pragma unroll
          for (int nt = 0; nt < kF8PvNT; ++nt) acc_o[hb][nt] *= a;
        }
      }
      // O += P . V(tile), the value reads kF8VAhead tiles ahead of their MFMAs
      constexpr int kSteps = kF8PvKB * kF8PvNT;        // (kb, nt) pairs, nt fastest
      i32x2 vraw[kF8VAhead];
      auto read_v = [&](int st) {
        const int kb = st / kF8PvNT, nt = st % kF8PvNT;
        vraw[st % kF8VAhead] = lds_read_tr8(kvt + v_off[nt & 3] + 64 * (nt >> 2) + 32 * kF8RowBytes * kb);
      };
#pragma unroll
      for (int st = 0; st < kF8VAhead; ++st) read_v(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const int kb = st / kF8PvNT, nt = st % kF8PvNT;
        const bf16x8 v8 = e4m3x8_to_bf16(vraw[st % kF8VAhead]);
        if (st + kF8VAhead < kSteps) read_v(st + kF8VAhead);
        if (copy_tile >= 0 && st < 2) issue_pieces(copy_tile, rid_next, 2 * st, 2 * st + 2);
        if (copy_tile >= 0 && st == 2) issue_pieces(copy_tile, rid_next, 4, kF8PiecesMax);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 0; hb < kF8PvHT; ++hb) acc_o[hb][nt] = mfma_bf16_k32(v8, pb[kb][hb], acc_o[hb][nt]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (copy_tile >= 0 && copy_tile + 1 <= last) fetch_rows(copy_tile + 1, rid_next);
      __syncthreads();                                 // B1: done with P and the tile's slot
      wait_tiles8(min(tile + kAhead, last) - (tile + 2), five);
      __syncthreads();                                 // B2
    }
    __syncthreads();                                   // kv_scale / l of every head is in LDS
#pragma unroll
    for (int hb = 0; hb < kF8PvHT; ++hb) {
      const float inv = sh.alpha[16 * hb + c];
      const int h = hbase + 16 * hb + c;
      const int col0 = 128 * rw + 4 * g;
      uint16_t* orow = (S == 1)
          ? static_cast<uint16_t*>(p.out) + ((int64_t)t * Hm + h) * kMlaDl + col0
          : p.part_o + (((int64_t)t * S + s) * Hm + h) * kMlaDl + col0;
#pragma unroll
      for (int nt = 0; nt < kF8PvNT; ++nt) {
        const f32x4 o = acc_o[hb][nt] * inv;
        *reinterpret_cast<bf16x4*>(orow + 16 * nt) = __builtin_convertvector(o, bf16x4);
      }
    }
  }
}

}  // namespace

hipError_t launch_mla_fp8(const MlaParams& p, hipStream_t s) {
  const int T = p.batch.num_rows;
  if (T == 0) return hipSuccess;
  const int HG = p.heads / kMlaHeadsPerGroup;
  const int units = T * p.splits;
  const int units_per_xcd = (units + 7) / 8;
  const int64_t blocks = 8LL * units_per_xcd * HG;
  // the positive-scale path needs a normal scale (the kernel's product, in
  // the same order): a padding row's -inf times a zero (flushed) scale would
  // give NaN in its exponent
  if (p.softmax_scale * p.q_scale * p.kv_scale * kF8Log2e >= FLT_MIN)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mla_fp8_kernel<true>), dim3((unsigned)blocks), dim3(kF8Threads), 0, s, p);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(mla_fp8_kernel<false>), dim3((unsigned)blocks), dim3(kF8Threads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_mla_combine_bf16(p, s);
}

}  // namespace dsa
