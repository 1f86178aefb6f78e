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
// waves handles one (row, split of the top-k list, group of 64 heads):
//   * the split's positions are resolved once through the block table into
//     cache-row ids in LDS, skipping -1 / out-of-range entries (so the -1 tail
//     of short rows costs nothing);
//   * gathered rows arrive 32 at a time: global -> VGPR (issued one tile ahead)
//     -> LDS, with the row stride padded to 1168 bytes so that both LDS access
//     patterns below are free of bank conflicts;
//   * scores: wave w computes S^T[32 rows x 16 heads] = C_tile . Q_w^T with
//     v_mfma_f32_16x16x32_bf16 (rows = M from LDS, heads = N from registers:
//     each wave keeps its 16 heads x 576 of q in VGPRs);
//   * online softmax in fp32, base 2, with lazy rescaling: the running maximum
//     of a head only moves when a tile exceeds it by more than 2^8, so the
//     accumulator rescale is skipped on most tiles;
//   * probabilities (bf16) and the per-head rescale factors go through LDS so
//     that wave w can compute O[64 heads x 128 value columns] += P . V_tile,
//     again on 16x16x32 bf16 MFMA (heads = M, value columns = N);
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
constexpr int kRowBytes = kMlaDqk * 2;                  // 1152
constexpr int kLdsRowStride = kRowBytes + 16;           // 1168
constexpr int kChunksPerRow = kRowBytes / 16;           // 72
constexpr int kTileChunks = kMlaTile * kChunksPerRow;   // 2304
constexpr int kChunksPerThread = kTileChunks / kMlaThreads;  // 9
constexpr float kRescaleThreshold = 8.0f;               // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

static_assert(kTileChunks % kMlaThreads == 0, "tile must split evenly over the threads");

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

struct MlaShared {
  int32_t rowid[kMlaMaxEntriesPerBlock];
  alignas(16) uint8_t kv[kMlaTile * kLdsRowStride];
  alignas(16) uint16_t pbuf[kMlaHeadsPerGroup * kMlaTile];  // [head][row] bf16 bits
  alignas(16) float alpha[kMlaHeadsPerGroup];
  alignas(16) float lsum[kMlaHeadsPerGroup];
  int flag[2];
  int wave_cnt[2][kMlaThreads / kWave];
};

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__global__ __launch_bounds__(kMlaThreads, 1) void mla_bf16_kernel(MlaParams p) {
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
  const int lane = lane_id(), wave = wave_id();
  const int g = lane >> 4, c = lane & 15;

  int b, jrow, q_len;
  row_to_seq(t, bv.cu_seqlens_q, bv.num_seqs, &b, &jrow, &q_len);
  const int P = bv.page_size;
  int seq_len = bv.seq_lens_k[b];
  const int addressable = bv.max_pages_per_seq * P;
  if (seq_len > addressable) seq_len = addressable;
  const int32_t* bt = bv.block_table + (int64_t)b * bv.max_pages_per_seq;

  // ---- resolve this split's entries into cache-row ids (compacted) ----
  const int e_begin = s * p.entries_per_split;
  int e_cnt = p.k - e_begin;
  if (e_cnt > p.entries_per_split) e_cnt = p.entries_per_split;
  if (e_cnt < 0) e_cnt = 0;
  const int32_t* idx = p.topk_idx + (int64_t)t * p.k + e_begin;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nvalid = 0;
  for (int e0 = 0, it = 0; e0 < e_cnt; e0 += kMlaThreads, ++it) {
    const int e = e0 + tid;
    bool valid = false;
    int32_t rid = 0;
    if (e < e_cnt) {
      const int pos = idx[e];
      if (pos >= 0 && pos < seq_len) {
        const int page = bt[pos / P];
        if (page >= 0 && page < bv.num_pages) {
          valid = true;
          rid = page * P + pos % P;
        }
      }
    }
    const uint64_t m = __ballot(valid);
    const int buf = it & 1;
    if (lane == 0) sh.wave_cnt[buf][wave] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kMlaThreads / kWave; ++w) {
      const int v = sh.wave_cnt[buf][w];
      off += (w < wave) ? v : 0;
      tot += v;
    }
    if (valid) sh.rowid[nvalid + off + __popcll(m & lt_mask)] = rid;
    nvalid += tot;
  }
  if (tid < 2) sh.flag[tid] = 0;
  __syncthreads();

  const int head0 = hg * kMlaHeadsPerGroup;          // first head of the group
  const int Hm = p.heads;
  const float scale_log2 = p.softmax_scale * kLog2e;

  // ---- q of this wave's 16 heads (N operand of the score MFMA) ----
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                         ((int64_t)t * Hm + head0 + 16 * wave + c) * kMlaDqk;
  bf16x8 qf[kMlaDqk / 32];
#pragma unroll
  for (int ks = 0; ks < kMlaDqk / 32; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * g);

  f32x4 acc_o[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc_o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;   // running max (log2 units) of head 16*wave + c
  float l_part = 0.f;        // this lane's share of the softmax denominator

  const uint8_t* kvbase = static_cast<const uint8_t*>(p.kv);
  const int n_tiles = (nvalid + kMlaTile - 1) / kMlaTile;

  i32x4 stage[kChunksPerThread];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int cid = tid + kMlaThreads * i;
      const int r = cid / kChunksPerRow, col = cid % kChunksPerRow;
      const int e = tile * kMlaTile + r;
      if (e < nvalid) {
        const int64_t rid = sh.rowid[e];
        stage[i] = *reinterpret_cast<const i32x4*>(kvbase + rid * kRowBytes + col * 16);
      } else {
        stage[i] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int cid = tid + kMlaThreads * i;
      const int r = cid / kChunksPerRow, col = cid % kChunksPerRow;
      *reinterpret_cast<i32x4*>(sh.kv + r * kLdsRowStride + col * 16) = stage[i];
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    if (tile + 1 < n_tiles) load_tile(tile + 1);   // in flight during this tile

    // ---- scores for 32 rows x this wave's 16 heads ----
    f32x4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* r0 = sh.kv + c * kLdsRowStride + 16 * g;
    const uint8_t* r1 = r0 + 16 * kLdsRowStride;
#pragma unroll
    for (int ks = 0; ks < kMlaDqk / 32; ++ks) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(r0 + 64 * ks);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(r1 + 64 * ks);
      sc0 = mfma_bf16(a0, qf[ks], sc0);
      sc1 = mfma_bf16(a1, qf[ks], sc1);
    }
    // lane (c, g) holds head c, rows 4g+i (sc0) and 16+4g+i (sc1)
    const int rowbase = tile * kMlaTile;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (rowbase + 4 * g + i < nvalid) ? sc0[i] * scale_log2 : -INFINITY;
      sv[4 + i] = (rowbase + 16 + 4 * g + i < nvalid) ? sc1[i] * scale_log2 : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    float alpha = 1.f;
    if (mx > m_ref + kRescaleThreshold) {
      alpha = exp2f(m_ref - mx);
      m_ref = mx;
      l_part *= alpha;
    }
    if (__ballot(alpha != 1.f) != 0ull && lane == 0) sh.flag[tile & 1] = 1;
    uint16_t pb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pr = exp2f(sv[i] - m_ref);
      l_part += pr;
      pb[i] = f32_to_bf16_bits(pr);
    }
    uint16_t* prow = sh.pbuf + (16 * wave + c) * kMlaTile;
    *reinterpret_cast<u16x4*>(prow + 4 * g) = u16x4{pb[0], pb[1], pb[2], pb[3]};
    *reinterpret_cast<u16x4*>(prow + 16 + 4 * g) = u16x4{pb[4], pb[5], pb[6], pb[7]};
    if (g == 0) sh.alpha[16 * wave + c] = alpha;
    __syncthreads();

    // ---- O[64 heads x value columns 128w..128w+127] += P . V ----
    if (sh.flag[tile & 1]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(sh.alpha + 16 * mt + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc_o[mt][nt] *= a4;
      }
    }
    if (tid == 0) sh.flag[(tile + 1) & 1] = 0;
    bf16x8 pa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint16_t* pr = sh.pbuf + (16 * mt + c) * kMlaTile;
      const u16x4 lo = *reinterpret_cast<const u16x4*>(pr + 4 * g);
      const u16x4 hi = *reinterpret_cast<const u16x4*>(pr + 16 + 4 * g);
      const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      pa[mt] = __builtin_bit_cast(bf16x8, v);
    }
    const uint16_t* kv16 = reinterpret_cast<const uint16_t*>(sh.kv);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int dv = 128 * wave + 16 * nt + c;
      u16x8 v;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        v[jj] = kv16[(4 * g + jj) * (kLdsRowStride / 2) + dv];
        v[4 + jj] = kv16[(16 + 4 * g + jj) * (kLdsRowStride / 2) + dv];
      }
      const bf16x8 vb = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc_o[mt][nt] = mfma_bf16(pa[mt], vb, acc_o[mt][nt]);
    }
    __syncthreads();
    if (tile + 1 < n_tiles) store_tile();
    __syncthreads();
  }

  // ---- finish: denominators, lse, normalized output ----
  float l = l_part;
  l += shfl_xor_f(l, 16);
  l += shfl_xor_f(l, 32);
  const int hq = head0 + 16 * wave + c;     // head of this lane in the score layout
  const float lse_val = (l > 0.f) ? (m_ref + log2f(l)) * kLn2 : -INFINITY;
  if (g == 0) {
    sh.lsum[16 * wave + c] = l;
    if (S == 1) {
      if (p.lse) p.lse[(int64_t)t * Hm + hq] = lse_val;
    } else {
      p.part_lse[((int64_t)t * S + s) * Hm + hq] = lse_val;
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
        for (int nt = 0; nt < 8; ++nt)
          orow[128 * wave + 16 * nt + c] = f32_to_bf16_bits(acc_o[mt][nt][i] * inv);
      } else {
        float* orow = p.part_o + (((int64_t)t * S + s) * Hm + h) * kMlaDl;
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) orow[128 * wave + 16 * nt + c] = acc_o[mt][nt][i] * inv;
      }
    }
  }
}

// LSE merge of the split partials (merge_attn_states generalised to S parts).
template <bool kBf16Out>
__global__ __launch_bounds__(128) void mla_combine_kernel(MlaParams p) {
  const int t = blockIdx.x, h = blockIdx.y;
  const int S = p.splits, Hm = p.heads, Dl = p.d_latent;
  const float* pl = p.part_lse + (int64_t)t * S * Hm + h;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[(int64_t)s * Hm]);
  float tot = 0.f;
  for (int s = 0; s < S; ++s) {
    const float v = pl[(int64_t)s * Hm];
    tot += (v == -INFINITY) ? 0.f : expf(v - mx);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if (threadIdx.x == 0 && p.lse) p.lse[(int64_t)t * Hm + h] = tot > 0.f ? mx + logf(tot) : -INFINITY;
  for (int d = threadIdx.x; d < Dl; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float v = pl[(int64_t)s * Hm];
      if (v == -INFINITY) continue;
      acc += expf(v - mx) * p.part_o[(((int64_t)t * S + s) * Hm + h) * Dl + d];
    }
    acc *= inv;
    if (kBf16Out) static_cast<uint16_t*>(p.out)[((int64_t)t * Hm + h) * Dl + d] = f32_to_bf16_bits(acc);
    else static_cast<float*>(p.out)[((int64_t)t * Hm + h) * Dl + d] = acc;
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
  const int max_splits = (k + 2 * kMlaTile - 1) / (2 * kMlaTile);   // >= 2 tiles per split
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
  hipLaunchKernelGGL(mla_combine_kernel<true>, dim3(T, p.heads), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mla_f32(const MlaParams& p, hipStream_t s) {
  if (p.batch.num_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(mla_f32_kernel, dim3(p.batch.num_rows, p.heads), dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
