// Query-side absorption (decode step 1) for the MLRA / MLA decode.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mlra_device.h"

namespace mlra {
namespace {

constexpr int kAbsorbSeqs = 32;  // sequences per workgroup (the MFMA M dimension)
// ------------------------------------------------------------------ query-side absorption
//
// q_nope[b][i][j*DL + c] = sum_n W_UK[j][i][c][n] * q_pre[b][i][j][n] (decode step 1: the
// NoPE key of head i in latent head j is C_j @ W_UK[j][i], so its dot with q_pre equals the
// dot of C_j with W_UK[j][i] @ q_pre). One single-wave workgroup per (query head i, 32 of the
// 512 latent channels, group of 32 sequences); fp32 MFMA with M = sequences, N = latent
// channels, K = d_nope = 128, both operands loaded from global memory with 16-byte loads.

struct AbsorbArgs {
  const unsigned char* q_pre;
  const float* W_UK;  // [NB][h][DL][128]
  unsigned char* q_nope;
  int B, h, NB, DL;             // DL: channels per latent head
  int64_t qp_sb, qp_sh, qp_sj;  // bytes
  int64_t qn_sb, qn_sh;         // bytes
};

constexpr int kDNope = 128;
constexpr int kAbsorbRows = 32;  // latent rows per workgroup (one wave, the MFMA N dimension)

// Eight consecutive query channels as fp32.
__device__ __forceinline__ void load8(const __bf16* p, float* out) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = float(v[e]);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  const floatx4 v0 = *reinterpret_cast<const floatx4*>(p), v1 = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = v0[e];
    out[4 + e] = v1[e];
  }
}

// One wave per (query head i, 32 latent rows, group of 32 sequences): y[b][c] = sum_n
// q_pre[b][n] W_UK[c][n] on fp32 MFMA 32x32x2 with M = sequences, N = latent rows, K = d_nope.
// Lane half hh supplies channels 64*hh .. 64*hh + 63, in order, one per MFMA step; both
// operands come straight from global memory in that order (no LDS).
template <typename T>
__global__ __launch_bounds__(64) void absorb_kernel(AbsorbArgs a) {
  const int lane = threadIdx.x;
  const int n = lane & 31, hh = lane >> 5;
  const int i = blockIdx.x;
  const int rb = blockIdx.y;
  const int grp = blockIdx.z;
  const int DL = a.DL;
  const int j = (rb * kAbsorbRows) / DL;
  const int c0 = (rb * kAbsorbRows) % DL;
  const int b0 = grp * kAbsorbSeqs;
  const int nb = min(kAbsorbSeqs, a.B - b0);

  float qa[64], wb[64];
  const float* wrow = a.W_UK + ((int64_t(j) * a.h + i) * DL + c0 + n) * kDNope + 64 * hh;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(wrow + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) wb[4 * u + e] = v[e];
  }
  if (n < nb) {
    const T* qrow = reinterpret_cast<const T*>(a.q_pre + int64_t(b0 + n) * a.qp_sb + int64_t(i) * a.qp_sh +
                                               int64_t(j) * a.qp_sj) + 64 * hh;
#pragma unroll
    for (int u = 0; u < 8; ++u) load8(qrow + 8 * u, qa + 8 * u);
  } else {
#pragma unroll
    for (int e = 0; e < 64; ++e) qa[e] = 0.f;
  }
  // Two accumulators (even and odd steps) halve the dependent MFMA chain; added at the end.
  floatx16 y0 = {}, y1 = {};
#pragma unroll
  for (int s2 = 0; s2 < 64; s2 += 2) {
    y0 = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s2], wb[s2], y0, 0, 0, 0);
    y1 = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s2 + 1], wb[s2 + 1], y1, 0, 0, 0);
  }
  const floatx16 y = y0 + y1;
  // y[rr]: sequence 8*(rr>>2) + 4*hh + (rr&3), latent channel c0 + n.
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int bl = 8 * (rr >> 2) + 4 * hh + (rr & 3);
    if (bl < nb) {
      T* dst = reinterpret_cast<T*>(a.q_nope + int64_t(b0 + bl) * a.qn_sb + int64_t(i) * a.qn_sh);
      dst[j * DL + c0 + n] = T(y[rr]);
    }
  }
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_absorb_query(const void* q_pre, const float* W_UK, void* q_nope, const mlra_decode_params* p,
                                 int32_t d_nope, int64_t qpre_stride_b, int64_t qpre_stride_h,
                                 int64_t qpre_stride_j, void* stream) {
  int rc = mlra_check_params(p);
  if (rc) return rc;
  if (d_nope != kDNope) return set_error(MLRA_ERR_UNSUPPORTED, "d_nope must be %d (got %d)", kDNope, d_nope);
  if (qpre_stride_b < 0 || qpre_stride_h < 0 || qpre_stride_j < 0)
    return set_error(MLRA_ERR_SHAPE, "query strides must be >= 0");
  if (p->batch == 0) return MLRA_OK;
  if (!q_pre || !W_UK || !q_nope) return set_error(MLRA_ERR_NULL, "q_pre, W_UK and q_nope must be non-NULL");
  const int64_t esz = p->dtype == MLRA_BF16 ? 2 : 4;
  if (!aligned16(q_pre) || !aligned16(W_UK) || (qpre_stride_b * esz) % 16 || (qpre_stride_h * esz) % 16 ||
      (qpre_stride_j * esz) % 16)
    return set_error(MLRA_ERR_ALIGN, "q_pre, W_UK and the q_pre strides must be 16-byte aligned");
  AbsorbArgs a;
  a.q_pre = static_cast<const unsigned char*>(q_pre);
  a.W_UK = W_UK;
  a.q_nope = static_cast<unsigned char*>(q_nope);
  a.B = p->batch;
  a.h = p->num_heads;
  a.NB = p->num_branches;
  a.DL = p->d_latent;
  a.qp_sb = qpre_stride_b * esz;
  a.qp_sh = qpre_stride_h * esz;
  a.qp_sj = qpre_stride_j * esz;
  a.qn_sb = p->q_stride_b * esz;
  a.qn_sh = p->q_stride_h * esz;
  static_assert(kShardLatent % kAbsorbRows == 0, "latent heads are whole row blocks");
  const dim3 grid(p->num_heads, latent_total(*p) / kAbsorbRows, (p->batch + kAbsorbSeqs - 1) / kAbsorbSeqs);
  if (p->dtype == MLRA_BF16)
    hipLaunchKernelGGL(absorb_kernel<__bf16>, grid, dim3(64), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(64), 0, static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "absorb kernel launch");
  return MLRA_OK;
}

