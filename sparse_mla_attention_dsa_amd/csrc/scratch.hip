// sparse_mla_decode_noalloc: sparse_mla_decode with its split-KV partials in a
// static device array of the library instead of a caller workspace, for
// callers that cannot allocate device memory.
//
// The array lives in this file as a file-scope __device__ variable. In host
// code its name is a host-side stand-in, not a device address, so the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in a per-device
// table; only those addresses are ever handed to kernels. The call itself
// allocates nothing: it sizes the plan, rejects plans larger than the array,
// and calls sparse_mla_decode with the array as its workspace. Every partial
// the kernels read is written first by the same call (each split writes its
// own partials, an empty split included), so nothing needs clearing between
// calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa.h"
#include "dsa_internal.h"

namespace {

constexpr size_t kScratchBytes = 32u << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

extern "C" dsa_status_t sparse_mla_decode_noalloc(const dsa_batch_t* batch, const void* q,
                                                  const void* kv_cache, dsa_dtype_t dtype,
                                                  const int32_t* topk_idx, int32_t k, int32_t num_heads,
                                                  int32_t d_latent, int32_t d_rope, float softmax_scale,
                                                  void* out, float* lse, dsa_stream_t stream) {
  const size_t need = dsa_workspace_bytes(DSA_OP_MLA_DECODE, batch, k, num_heads, d_latent, dtype);
  if (need == (size_t)-1)   // invalid or unsupported: the plain call reports which, before any launch
    return sparse_mla_decode(batch, q, kv_cache, dtype, topk_idx, k, num_heads, d_latent, d_rope, softmax_scale,
                             out, lse, nullptr, 0, stream);
  if (need > kScratchBytes)
    return dsa::set_error(DSA_ERR_UNSUPPORTED,
                          "sparse_mla_decode_noalloc: the split partials of this batch need %zu bytes, more "
                          "than the %zu-byte static scratch (use sparse_mla_decode with a workspace)",
                          need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return dsa::set_error(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
      return dsa::set_error(DSA_ERR_UNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev,
                            kMaxDevices - 1);
    // once per device, with that device current: the device address of its copy
    std::call_once(g_once[dev], [dev] { g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch)); });
    if (g_err[dev] != hipSuccess || g_ptr[dev] == nullptr)
      return dsa::set_error(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(g_err[dev]));
    ws = g_ptr[dev];
  }
  return sparse_mla_decode(batch, q, kv_cache, dtype, topk_idx, k, num_heads, d_latent, d_rope, softmax_scale,
                           out, lse, ws, ws ? kScratchBytes : 0, stream);
}
