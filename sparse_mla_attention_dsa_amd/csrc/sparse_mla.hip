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
constexpr int kDmaPerTile = kTileBytes / 1024;          // 36 wave-wide 1 KB copies
constexpr int kRing = 3;                                // tiles resident: 1 computing, 2 landing
constexpr int kDmaWaves = kMlaWaves / 2;                // the second-half score waves issue the copies
constexpr int kDmaPerWave = kDmaPerTile / kDmaWaves;    // 9
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
  alignas(16) uint16_t pbuf[kMlaHeadsPerGroup * kPRow];     // [head][row] bf16 bits, padded rows
  alignas(16) f32x4 sx[kMlaWaves / 2][2][kWave];            // second-half partial scores
  alignas(16) float alpha[kMlaHeadsPerGroup];
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

// Copy 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at LDS offset lds_off + 16 * l (wave-uniform lds_off). M0 is set here
// explicitly; completion is tracked with vmcnt by the caller.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_off) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);   // LDS aperture: low 32 bits are the offset
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

  // One tile = 36 wave-wide 1 KB copies, issued by the four second-half score
  // waves (which have no softmax to run): wave 4 + j issues copies j, j + 4, ...
  // Copy i fills LDS chunks 64i .. 64i+63; the row and logical column of each
  // lane's chunk do not depend on the tile.
  int dma_row[kDmaPerWave], dma_col[kDmaPerWave];
#pragma unroll
  for (int q = 0; q < kDmaPerWave; ++q) {
    const int i = (wave & 3) + kDmaWaves * q;
    const int chunk = 64 * i + lane;
    const int r = chunk / kChunksPerRow;
    dma_row[q] = r;
    dma_col[q] = ((chunk % kChunksPerRow) ^ swz(r)) * 16;   // logical chunk stored at this position
  }
  auto issue_tile = [&](int tile) {                     // second-half waves only
    const uint32_t dst = lds_offset(sh.kv[tile % kRing]);
    int64_t rid[kDmaPerWave];
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {             // row ids first (LDS reads) ...
      const int e = tile * kMlaTile + dma_row[q];
      // rows past the end re-read the split's first row; their scores are masked
      rid[q] = sh.rowid[e < nvalid ? e : 0];
    }
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q)               // ... then the copies back to back
      lds_dma16(kvbase + rid[q] * kRowBytes + dma_col[q], dst + 1024 * ((wave & 3) + kDmaWaves * q));
  };

  // Consume q here: the compiler then knows its loads have completed, and it
  // places no vector-memory waits inside the tile loop, where they would also
  // drain the (to it invisible) tile copies in flight.
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) asm volatile("" :: "v"(qf[ks]));

  if (kh == 1) {
    if (n_tiles > 0) issue_tile(0);
    if (n_tiles > 1) issue_tile(1);
  }

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

  // tile 0 visible before the loop
  if (kh == 1) {
    if (n_tiles > 1) wait_vmcnt<kDmaPerWave>(); else wait_vmcnt<0>();
  }
  __syncthreads();

  // Per tile: scores -> [barrier B] -> copies of tile + 2, softmax, wait for
  // tile + 1 -> [barrier C] -> P.V. Barrier B also guarantees that every wave
  // has finished P.V of the previous tile, so its ring slot can be refilled.
  for (int tile = 0; tile < n_tiles; ++tile) {
    const uint8_t* kvt = sh.kv[tile % kRing];

    // ---- partial scores: 32 rows x 16 heads over this wave's half ----
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
    const f32x4 own0 = sa0 + sb0, own1 = sa1 + sb1;
    if (kh == 1) {
      sh.sx[ht][0][lane] = own0;
      sh.sx[ht][1][lane] = own1;
    }
    __syncthreads();                                     // barrier B
    if (kh == 1 && tile + 2 < n_tiles) issue_tile(tile + 2);   // slot of tile - 1: free after B

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
      if (__ballot(alpha != 1.f) != 0ull && lane == 0) sh.flag[tile & 1] = 1;
      float pr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(sv[i] - m_ref);
        l_part += pr[i];
      }
      bf16x2 pb[4];                                      // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = __builtin_convertvector(f32x2{pr[2 * i], pr[2 * i + 1]}, bf16x2);
      uint16_t* prow = sh.pbuf + (16 * ht + c) * kPRow;
      *reinterpret_cast<bf16x2*>(prow + 4 * g) = pb[0];
      *reinterpret_cast<bf16x2*>(prow + 4 * g + 2) = pb[1];
      *reinterpret_cast<bf16x2*>(prow + 16 + 4 * g) = pb[2];
      *reinterpret_cast<bf16x2*>(prow + 16 + 4 * g + 2) = pb[3];
      if (g == 0) sh.alpha[16 * ht + c] = alpha;
    }
    // tile + 1 has landed once at most tile + 2's copies are pending
    if (kh == 1 && tile + 1 < n_tiles) {
      if (tile + 2 < n_tiles) wait_vmcnt<kDmaPerWave>(); else wait_vmcnt<0>();
    }
    __syncthreads();                                     // barrier C

    // ---- O[64 heads x value columns 64w..64w+63] += P . V ----
    if (sh.flag[tile & 1]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(sh.alpha + 16 * mt + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc_o[mt][nt] *= a4;
      }
    }
    if (tid == 0) sh.flag[(tile + 1) & 1] = 0;
    bf16x8 pa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t* pr = sh.pbuf + (16 * mt + c) * kPRow;
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
  }

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
