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
// dot of C_j with W_UK[j][i] @ q_pre). One workgroup per (query head i, 128-row block r of the
// 512 latent channels, group of 32 sequences); fp32 MFMA with M = sequences, N = latent
// channels (32 per wave), K = d_nope = 128. The query block is staged in LDS k-major.

struct AbsorbArgs {
  const unsigned char* q_pre;
  const float* W_UK;  // [NB][h][DL][128]
  unsigned char* q_nope;
  int B, h, NB;
  int64_t qp_sb, qp_sh, qp_sj;  // bytes
  int64_t qn_sb, qn_sh;         // bytes
};

constexpr int kDNope = 128;

template <typename T>
__global__ __launch_bounds__(256) void absorb_kernel(AbsorbArgs a) {
  __shared__ float qs[kDNope][kAbsorbSeqs];  // q_pre block, k-major: qs[n][b]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int i = blockIdx.x;
  const int r = blockIdx.y;
  const int grp = blockIdx.z;
  const int DL = kLatentTotal / a.NB;
  const int j = (r * 128) / DL;
  const int c0 = (r * 128) % DL;
  const int b0 = grp * kAbsorbSeqs;
  const int nb = min(kAbsorbSeqs, a.B - b0);

  // W_UK rows c0 + 32*wave + n, pairs of columns (k = 4*kp + 2*hh + e, e = 0, 1).
  const float* wrow = a.W_UK + ((int64_t(j) * a.h + i) * DL + c0 + 32 * wave + n) * kDNope + 2 * hh;
  floatx2 wv[kDNope / 4];
#pragma unroll
  for (int kp = 0; kp < kDNope / 4; ++kp) wv[kp] = *reinterpret_cast<const floatx2*>(wrow + 4 * kp);

  for (int idx = tid; idx < kAbsorbSeqs * kDNope; idx += 256) {
    const int bl = idx / kDNope, k = idx % kDNope;
    float v = 0.f;
    if (bl < nb) {
      const unsigned char* src = a.q_pre + int64_t(b0 + bl) * a.qp_sb + int64_t(i) * a.qp_sh + int64_t(j) * a.qp_sj;
      v = float(reinterpret_cast<const T*>(src)[k]);
    }
    qs[k][bl] = v;
  }
  __syncthreads();

  floatx16 y = {};
#pragma unroll
  for (int kp = 0; kp < kDNope / 4; ++kp) {
    y = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[4 * kp + 2 * hh][n], wv[kp][0], y, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[4 * kp + 2 * hh + 1][n], wv[kp][1], y, 0, 0, 0);
  }
  // y[rr]: sequence 8*(rr>>2) + 4*hh + (rr&3), latent channel c0 + 32*wave + n.
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int bl = 8 * (rr >> 2) + 4 * hh + (rr & 3);
    if (bl < nb) {
      T* dst = reinterpret_cast<T*>(a.q_nope + int64_t(b0 + bl) * a.qn_sb + int64_t(i) * a.qn_sh);
      dst[j * DL + c0 + 32 * wave + n] = T(y[rr]);
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
  AbsorbArgs a;
  a.q_pre = static_cast<const unsigned char*>(q_pre);
  a.W_UK = W_UK;
  a.q_nope = static_cast<unsigned char*>(q_nope);
  a.B = p->batch;
  a.h = p->num_heads;
  a.NB = p->num_branches;
  a.qp_sb = qpre_stride_b * esz;
  a.qp_sh = qpre_stride_h * esz;
  a.qp_sj = qpre_stride_j * esz;
  a.qn_sb = p->q_stride_b * esz;
  a.qn_sh = p->q_stride_h * esz;
  const dim3 grid(p->num_heads, kLatentTotal / 128, (p->batch + kAbsorbSeqs - 1) / kAbsorbSeqs);
  if (p->dtype == MLRA_BF16)
    hipLaunchKernelGGL(absorb_kernel<__bf16>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(256), 0, static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "absorb kernel launch");
  return MLRA_OK;
}

