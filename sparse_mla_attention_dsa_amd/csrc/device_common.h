// Device helpers shared by the DSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Row t of a batch -> (request b, index j of the row inside the request, rows of
// the request). cu == nullptr means one row per request (decode).
__device__ __forceinline__ void row_to_seq(int t, const int32_t* __restrict__ cu, int num_seqs,
                                           int* b, int* j, int* q_len) {
  if (cu == nullptr) {
    *b = t; *j = 0; *q_len = 1;
    return;
  }
  // largest b with cu[b] <= t (cu is non-decreasing; empty requests are skipped)
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  *b = lo;
  *j = t - cu[lo];
  *q_len = cu[lo + 1] - cu[lo];
}

// Keys the row may see under bottom-right causal alignment, clamped to what the
// block table and the caller's buffers can address.
__device__ __forceinline__ int visible_keys(int seq_len_k, int q_len, int j, int cap) {
  int v = seq_len_k - q_len + j + 1;
  v = v < 0 ? 0 : v;
  return v < cap ? v : cap;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Order-preserving map of a float to an unsigned key: a < b  <=>  key(a) < key(b),
// with -0 mapped onto +0 so that equal floats get equal keys.
__device__ __forceinline__ uint32_t ordered_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// max / sum of v over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane
// groups), with the gfx950 lane swaps (VALU, no LDS round trip); every lane
// gets the result
// The maximum is IEEE 754-2019 `maximum` (a NaN input gives NaN), which
// gfx950 has as v_maximum3_f32; fmaxf would first quiet each input with an
// extra v_max_f32.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// IEEE 754-2019 maximum of two floats (NaN propagates; v_maximum3_f32)
__device__ __forceinline__ float fmaximum(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Reduce-scatter over the four 16-lane groups: p[u] is this lane's partial
// of quantity u; lane group g (lanes 16g .. 16g + 15) gets the sum over the
// four groups of quantity g. The swaps pair rows (0, 1) and (2, 3) first
// (v_permlane16_swap exchanges the odd rows of its first operand with the
// even rows of its second), then the halves (v_permlane32_swap: upper half of
// the first with lower half of the second). Quantity u ends as
// (p_0[u] + p_1[u]) + (p_2[u] + p_3[u]), the association of sum_over_groups,
// so both give the same floats.
__device__ __forceinline__ float sum_scatter_over_groups(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);   // rows 0, 2: quantity 0; rows 1, 3: 1
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);   // rows 0, 2: quantity 2; rows 1, 3: 3
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave, on DPP lane moves (no LDS
// round trip): shifts of 1, 2, 4, 8 lanes inside each 16-lane row, then the
// last lane of row 0 / row 2 is added to rows 1 / 3, and the last lane of
// row 1 to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  // dpp_ctrl: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143;
  // bound_ctrl = true makes lanes without a source read 0.
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>(p);   // LDS aperture: low 32 bits are the offset
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at M0 + 16 l (M0 = the wave-uniform destination). Completion is counted by
// vmcnt like any other vector load.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_addr) : "memory", "m0");
}

// fp8 (E4M3) 16x16x128 MFMA with fp32 accumulate. All-zero scale operands
// select the unscaled form of v_mfma_f32_16x16x128_f8f6f4: the plain fp8
// product (the same values as unit E8M0 scales), under which the wave can issue
// independent VALU work far better than under the scaled form.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// relu as an integer max with 0 on the float's bits (negative floats are
// negative integers); no NaN quieting is needed.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

}  // namespace dsa
