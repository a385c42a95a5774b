// Plan dump and HBM bandwidth probes (a plain copy and a non-temporal read) that the
// benchmark uses as achievable-bandwidth context and as the byte-counter calibration.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mlra_device.h"

namespace mlra {
namespace {

// ------------------------------------------------------------------ plan dump and copy probe

__global__ __launch_bounds__(64) void plan_kernel(const int32_t* seqlens, int B, int G_req, int max_seg,
                                                  int32_t* out) {
  const int g = blockIdx.x;
  const int lane = threadIdx.x;
  int32_t* row = out + int64_t(g) * max_seg * 3;
  for (int k = lane; k < max_seg * 3; k += 64) row[k] = -1;
  const Lens lens = load_lens(seqlens, B);
  const Plan plan = make_plan(lens, G_req);
  if (g == 0 && lane == 0) {
    out[int64_t(G_req) * max_seg * 3] = int32_t(plan.T);
    out[int64_t(G_req) * max_seg * 3 + 1] = plan.G;
  }
  if (g >= plan.G) return;
  SegmentWalk walk = begin_walk(lens, g, plan);
  int b, ta, te, L, k = 0;
  while (next_segment(lens, walk, b, ta, te, L)) {
    if (lane == 0 && k < max_seg) {
      row[3 * k] = b;
      row[3 * k + 1] = ta;
      row[3 * k + 2] = te;
    }
    ++k;
  }
}

// Read-only stream: each workgroup reads one contiguous chunk with non-temporal 16-byte
// loads, 16 per thread in flight; the XOR of every word goes to sink[0] once per wave.
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n, int64_t per_wg,
                                                   uint32_t* sink) {
  const int64_t begin = int64_t(blockIdx.x) * per_wg;
  const int64_t end = begin + per_wg < n ? begin + per_wg : n;
  u32x4 x = {};
  int64_t i = begin + threadIdx.x;
  for (; i + (kReadUnroll - 1) * 256 < end; i += kReadUnroll * 256) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u];
  }
  for (; i < end; i += 256) x ^= __builtin_nontemporal_load(src + i);
  uint32_t r = x[0] ^ x[1] ^ x[2] ^ x[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) r ^= __shfl_xor(r, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, r);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_decode_plan(const int32_t* seqlens, int32_t batch, int32_t num_splits, int32_t max_segments,
                                int32_t* plan, void* stream) {
  if (batch < 0 || num_splits < 1 || max_segments < 1)
    return set_error(MLRA_ERR_SHAPE, "batch >= 0, num_splits >= 1 and max_segments >= 1 required");
  if (!plan || (batch > 0 && !seqlens)) return set_error(MLRA_ERR_NULL, "seqlens and plan must be non-NULL");
  hipLaunchKernelGGL(plan_kernel, dim3(num_splits), dim3(64), 0, static_cast<hipStream_t>(stream), seqlens, batch,
                     num_splits, max_segments, plan);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
  return MLRA_OK;
}

extern "C" int mlra_read_bandwidth_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return set_error(MLRA_ERR_NULL, "src and sink must be non-NULL");
  if (!aligned16(src) || bytes % 16 != 0) return set_error(MLRA_ERR_ALIGN, "src and bytes must be 16-byte aligned");
  if (bytes == 0) return MLRA_OK;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  const int64_t n = int64_t(bytes / 16);
  const int64_t blocks = int64_t(cus) * 4;
  const int64_t per_wg = (n + blocks - 1) / blocks;
  hipLaunchKernelGGL(read_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), n, per_wg, sink);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "read kernel launch");
  return MLRA_OK;
}

extern "C" int mlra_copy_bandwidth_probe(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return set_error(MLRA_ERR_NULL, "src and dst must be non-NULL");
  if (!aligned16(src) || !aligned16(dst) || bytes % 16 != 0)
    return set_error(MLRA_ERR_ALIGN, "src, dst and bytes must be 16-byte aligned");
  if (bytes == 0) return MLRA_OK;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "device query");
  const int64_t n = int64_t(bytes / 16);
  int64_t blocks = (n + 255) / 256;
  if (blocks > int64_t(cus) * 16) blocks = int64_t(cus) * 16;
  hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "copy kernel launch");
  return MLRA_OK;
}
