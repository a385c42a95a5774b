// mlra_decode_noalloc: the whole decode step of mlra_decode with its workspace in a fixed
// device array of this library, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). It launches the
// same kernels as mlra_decode on the same arguments.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "mlra_device.h"

namespace mlra {
namespace {

constexpr size_t kScratchBytes = size_t(MLRA_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "scratch size");

// The workspace of every mlra_decode_noalloc call on a device. Each device that loads this
// library holds its own copy until the process ends. In host code the name is only a handle
// for hipGetSymbolAddress, never a device address.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
int scratch_on_current_device(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MLRA_ERR_UNSUPPORTED, "device ordinal %d is past the %d devices the scratch table holds", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return set_error(MLRA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a NULL address");
    ptrs[dev] = ptr;
  }
  *out = ptrs[dev];
  return MLRA_OK;
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_decode_noalloc(const void* q_nope, const void* q_rope, const void* latent_cache,
                                   const void* rope_cache, const int32_t* block_table, const int32_t* seqlens,
                                   const float* W_UV, float* out, const mlra_decode_params* p, void* stream) {
  size_t need = 0;
  int rc = mlra_decode_workspace_size(p, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return set_error(MLRA_ERR_WORKSPACE,
                     "this call needs %zu bytes of workspace; mlra_decode_noalloc holds %zu (use mlra_decode with "
                     "a caller workspace)",
                     need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_on_current_device(&ws);
  if (rc) return rc;
  return mlra_decode(q_nope, q_rope, latent_cache, rope_cache, block_table, seqlens, W_UV, out, p, ws,
                     kScratchBytes, stream);
}
