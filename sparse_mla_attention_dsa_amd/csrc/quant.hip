// fp8 quantization of the indexer's inputs, the step just before the scores
// (SGLang indexer page, "dsa_indexer.py": Indexer.forward_cuda turns the bf16
// index query into (q_fp8, q_scale) with act_quant and _get_logits_head_gate
// multiplies the head gates by q_scale; Indexer._store_index_k_cache
// quantizes the new index keys the same way and writes (k_fp8, k_scale) into
// the paged index-K buffer at out_cache_loc).
//
// One block is one 128-wide head row of q or one key:
//   s = max(max_d |x_d|, 1e-30) / 448          fp32
//   code_d = E4M3FN(x_d / s)                   the fp32 quotient (IEEE division),
//                                              nearest code, ties to even
// The gate of a head row becomes w * s, so the scores use the codes directly.
//
// Memory-bound and tiny next to the scores: a 16-lane quarter of a wave takes
// one block (16 bytes of bf16 per lane in, 8 bytes of codes per lane out),
// and the block maximum is four lane exchanges inside the quarter.
#include "device_common.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantBlocksPerWg = kQuantThreads / 16;

// fp32 -> OCP E4M3FN code, nearest, ties to even mantissa. E4M3FN has no
// infinity: a magnitude that rounds past 448 (onto the step that would be
// 480) or lies beyond it, infinity and NaN all give the NaN code 0x7F; the
// sign bit is kept.
__device__ __forceinline__ uint32_t e4m3fn_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t mag;
  if (a >= 0x43f00000u) {                                        // >= 480, inf, NaN
    mag = 0x7fu;
  } else if (a < 0x3c800000u) {                                  // below 2^-6: multiples of 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling; rint: half to even
  } else {
    // drop 20 of the 23 mantissa bits, rounding to nearest even (a carry
    // moves into the exponent), then rebias the exponent from 127 to 7
    const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
    mag = r - (120u << 3);
    mag = mag > 0x7fu ? 0x7fu : mag;
  }
  return sign | mag;
}

// Quantizes the block whose elements 8 l .. 8 l + 7 this lane of a 16-lane
// quarter holds (16 bytes of bf16 at src): returns the lane's 8 codes packed
// little-endian and the block's scale. Any NaN in the block makes the scale
// NaN (the maximum is taken on the magnitude bits, where NaN is largest).
__device__ __forceinline__ uint2 quant_block(const uint16_t* src, float* scale) {
  const i32x4 raw = *reinterpret_cast<const i32x4*>(src);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
    x[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xffff0000u);
  }
  uint32_t m = __float_as_uint(1e-30f);                          // the floor, as magnitude bits
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 16));
  const float s = __uint_as_float(m) / 448.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= e4m3fn_code(x[i] / s) << (8 * i);
    hi |= e4m3fn_code(x[4 + i] / s) << (8 * i);
  }
  *scale = s;
  return make_uint2(lo, hi);
}

__global__ __launch_bounds__(kQuantThreads) void quant_index_q_kernel(QuantQParams p) {
  const int64_t row = (int64_t)blockIdx.x * kQuantBlocksPerWg + threadIdx.x / 16;   // (t, h)
  if (row >= p.rows) return;
  const int l = threadIdx.x & 15;
  float s;
  const uint2 codes = quant_block(p.q + row * kIdxDim + 8 * l, &s);
  *reinterpret_cast<uint2*>(p.q8 + row * kIdxDim + 8 * l) = codes;
  if (l == 0) p.w_eff[row] = p.w[row] * s;
}

__global__ __launch_bounds__(kQuantThreads) void store_index_k_kernel(StoreKParams p) {
  const int64_t i = (int64_t)blockIdx.x * kQuantBlocksPerWg + threadIdx.x / 16;
  if (i >= p.num_tokens) return;
  const int64_t slot = p.slot_mapping[i];
  if (slot < 0 || slot >= (int64_t)p.num_pages * p.page_size) return;   // uniform in the quarter
  const int l = threadIdx.x & 15;
  float s;
  const uint2 codes = quant_block(p.key + i * kIdxDim + 8 * l, &s);
  const int64_t page = slot / p.page_size;
  const int pos = (int)(slot - page * p.page_size);
  uint8_t* pg = p.cache + page * p.page_bytes;
  *reinterpret_cast<uint2*>(pg + (int64_t)pos * kIdxDim + 8 * l) = codes;
  if (l == 0) *reinterpret_cast<float*>(pg + (int64_t)p.page_size * kIdxDim + 4 * pos) = s;
}

}  // namespace

hipError_t launch_quant_index_q(const QuantQParams& p, hipStream_t s) {
  if (p.rows == 0) return hipSuccess;
  const int64_t wgs = (p.rows + kQuantBlocksPerWg - 1) / kQuantBlocksPerWg;
  hipLaunchKernelGGL(quant_index_q_kernel, dim3((unsigned)wgs), dim3(kQuantThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_store_index_k(const StoreKParams& p, hipStream_t s) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t wgs = (p.num_tokens + kQuantBlocksPerWg - 1) / kQuantBlocksPerWg;
  hipLaunchKernelGGL(store_index_k_kernel, dim3((unsigned)wgs), dim3(kQuantThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa
