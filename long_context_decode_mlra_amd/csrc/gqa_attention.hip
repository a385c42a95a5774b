// Grouped-query (GQA) split-KV decode attention on gfx950: the comparator the MLRA paper
// measures its decode kernel against (page "Multi-Head Low-Rank Attention", ai.info summary
// of arXiv 2603.02188, "Key Contributions" #4), at the shape it analyses GQA with (64 query
// heads over 8 KV heads of 128 channels, "Methodology in Plain English", 4th paragraph).
//
// Kernels
//   gqa_decode_kernel  one single-wave workgroup per (token split, KV head). It streams
//                      32-token tiles of that head's K and V rows straight from HBM into its
//                      own LDS ring (no workgroup barrier: the wave owns its buffers), computes
//                      S^T = K Q^T and O^T += V^T P^T on bf16 MFMA 16x16x32 with the group's
//                      query heads as the N dimension (up to 16), keeps an fp32 online softmax
//                      per query head, and writes one partial per sequence it touches.
//   gqa_merge_kernel   log-sum-exp merge of each sequence's partials into the output.
// The split plan over the flattened tiles of all sequences is the one in mlra_device.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "mlra_device.h"

namespace mlra {
namespace {

constexpr int kGRow = kGqaHeadDim * 2;       // bytes of one token's K (or V) row of one KV head
constexpr int kGHalf = kTile * kGRow;        // 8 KiB: the K (or V) rows of one tile
constexpr int kGTile = 2 * kGHalf;           // 16 KiB: K rows, then V rows
constexpr int kGLoads = kGTile / 1024;       // 16 loads of 64 lanes x 16 bytes per tile
#ifndef MLRA_GQA_STAGES
#define MLRA_GQA_STAGES 3
#endif
constexpr int kGStages = MLRA_GQA_STAGES;    // tiles in flight while the wave waits for the oldest
constexpr int kGStreamPolicy = 2;            // non-temporal: every cache byte is read once
constexpr float kGRescaleSlack = 8.0f;       // see the MLRA kernel: raise the max only by > 8 (log2)
static_assert((kGStages - 1) * kGLoads < 64, "vmcnt immediate");

struct GqaArgs {
  const unsigned char* q;
  const unsigned char* k;
  const unsigned char* v;
  const int32_t* block_table;
  const int32_t* seqlens;
  float* part_o;    // [slots][Hq][128]
  float* part_ml;   // [slots][Hq][2]
  int64_t* prefix;  // [B + 3], written by workgroup (0, 0)
  int B, Hq, group, G_req, page_size, max_seqlen, max_pages;
  int64_t q_sb, q_sh, k_st, k_sh, v_st, v_sh;  // bytes
  float c;                                      // sm_scale * log2(e)
};

template <int N>
__device__ __forceinline__ void gqa_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until the loads of the oldest tile in flight have landed, `later` (< S) younger
// tiles' loads still allowed in flight (kGLoads each).
template <int S>
__device__ __forceinline__ void gqa_wait_tile(int later) {
  if constexpr (S > 1) {
    if (later == S - 1) {
      gqa_wait_vmcnt<(S - 1) * kGLoads>();
      return;
    }
    gqa_wait_tile<S - 1>(later);
  } else {
    gqa_wait_vmcnt<0>();
  }
}

// The 16-byte chunk c of row t sits at chunk position c ^ (t & 15) in LDS, so 16 rows read
// at one logical chunk hit 16 distinct bank groups (rows are 256 bytes apart).
__device__ __forceinline__ int gqa_swz(int t) { return t & 15; }

// This wave's K and V rows of one tile, HBM -> LDS. Load i covers rows 4*(i%8) .. +3 of the
// K half (i < 8) or the V half; lane l lands at LDS row 4*(i%8) + l/16, chunk position l%16.
// Rows past the sequence end re-read its last row (their logits are masked).
__device__ __forceinline__ void gqa_issue_tile(const GqaArgs& a, int b, int L, int tile, int kh, int lane,
                                               unsigned char* buf) {
  const int tok0 = tile * kTile;
  int64_t row0;
  if (a.block_table) {
    // Pages hold a multiple of kTile tokens, so a tile never straddles two pages.
    const int page = scalar_read(a.block_table + int64_t(b) * a.max_pages + tok0 / a.page_size);
    row0 = int64_t(page) * a.page_size + tok0 % a.page_size;
  } else {
    row0 = int64_t(b) * a.max_seqlen + tok0;
  }
  const int last = min(kTile, L - tok0) - 1;
  const unsigned char* kb = a.k + row0 * a.k_st + int64_t(kh) * a.k_sh;
  const unsigned char* vb = a.v + row0 * a.v_st + int64_t(kh) * a.v_sh;
#pragma unroll
  for (int i = 0; i < kGLoads; ++i) {
    const int r = 4 * (i & 7) + (lane >> 4);
    const int c = (lane & 15) ^ gqa_swz(r);
    const unsigned char* src = (i < 8 ? kb + min(r, last) * int(a.k_st) : vb + min(r, last) * int(a.v_st)) + c * 16;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, 0,
                                     kGStreamPolicy);
  }
}

__global__ __launch_bounds__(64) void gqa_decode_kernel(GqaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kGStages * kGTile];
  const int lane = threadIdx.x;
  const int n16 = lane & 15;  // MFMA column: query head kh*group + n16
  const int g4 = lane >> 4;   // MFMA K group
  const int kh = blockIdx.y;
  const int gs = blockIdx.x;
  const bool head_ok = n16 < a.group;
  const int head = kh * a.group + n16;

  const Lens lens = load_lens(a.seqlens, a.B);
  const Plan plan = make_plan(lens, a.G_req);
  if (gs == 0 && kh == 0) write_prefix(lens, plan, a.prefix);
  if (gs >= plan.G) return;
  SegmentWalk walk = begin_walk(lens, gs, plan);

  int b, ta, te, L;
  while (next_segment(lens, walk, b, ta, te, L)) {
    b = __builtin_amdgcn_readfirstlane(b);
    ta = __builtin_amdgcn_readfirstlane(ta);
    te = __builtin_amdgcn_readfirstlane(te);
    L = __builtin_amdgcn_readfirstlane(L);

    // Query operand of K step st: channels 32*st + 8*g4 .. +8 of this lane's head.
    bf16x8 qv[4];
    {
      const unsigned char* qp = a.q + int64_t(b) * a.q_sb + int64_t(head_ok ? head : 0) * a.q_sh;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        qv[st] = head_ok ? *reinterpret_cast<const bf16x8*>(qp + (32 * st + 8 * g4) * 2) : bf16x8{};
    }
    floatx4 O[8] = {};
    float m_run = -INFINITY;
    float l_run = 0.f;

#pragma unroll
    for (int st = 0; st < kGStages - 1; ++st)
      if (ta + st < te) gqa_issue_tile(a, b, L, ta + st, kh, lane, smem + st * kGTile);
    for (int k = ta; k < te; ++k) {
      const unsigned char* buf = smem + ((k - ta) % kGStages) * kGTile;
      if (k + kGStages - 1 < te) {
        // Tile k+S-1 reuses tile k-1's buffer: this wave's reads of it have returned.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        gqa_issue_tile(a, b, L, k + kGStages - 1, kh, lane, smem + ((k - ta + kGStages - 1) % kGStages) * kGTile);
      }
      gqa_wait_tile<kGStages>(min(kGStages - 1, te - 1 - k));

      // S^T for tokens 16*mb + n16 (A rows) and the group's heads (B columns). Row
      // 16*mb + n16 has swizzle n16, so chunk 4*st + g4 sits at (4*st + g4) ^ n16.
      floatx4 s2[2] = {};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8 kk = *reinterpret_cast<const bf16x8*>(buf + (16 * mb + n16) * kGRow +
                                                             (((4 * st + g4) ^ n16) << 4));
          s2[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qv[st], s2[mb], 0, 0, 0);
        }
      // Lane (n16, g4) holds tokens 16*(e>>2) + 4*g4 + (e&3) of head n16 in sv[e].
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = s2[e >> 2][e & 3];
      const int n_valid = L - k * kTile;
      if (n_valid < kTile) {
        const int lim = n_valid - 4 * g4;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (16 * (e >> 2) + (e & 3) >= lim) sv[e] = -INFINITY;
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * a.c;
      const bool raise = mt > m_run + kGRescaleSlack;
      if (__ballot(raise)) {
        const float mnew = raise ? mt : m_run;
        const float alpha = (mnew == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int o = 0; o < 8; ++o) O[o] *= alpha;
        m_run = mnew;
      }
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[e], a.c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[e + 1], a.c, -m_run));
        psum += p0 + p1;
        const bf16x2 pv = __builtin_convertvector((floatx2{p0, p1}), bf16x2);
        pb[e] = pv[0];
        pb[e + 1] = pv[1];
      }
      l_run += psum;

      // O^T[channel][head] += V^T P^T; K index 8*g4 + e is token 16*(e>>2) + 4*g4 + (e&3).
      // M-block 4*blk + qq holds channel 64*blk + 4*m + qq in row m = n16: each lane reads
      // four consecutive channels (8 bytes) of its eight tokens and regroups them.
      const unsigned char* vbuf = buf + kGHalf;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int chunk = 8 * blk + (n16 >> 1);
        u32x2 d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tau = 16 * (e >> 2) + 4 * g4 + (e & 3);
          d[e] = *reinterpret_cast<const u32x2*>(vbuf + tau * kGRow + ((chunk ^ gqa_swz(tau)) << 4) +
                                                 ((n16 & 1) << 3));
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint32_t sel = (qq & 1) ? 0x07060302u : 0x05040100u;
          u32x4 av;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const uint32_t lo = (qq < 2) ? d[2 * pp][0] : d[2 * pp][1];
            const uint32_t hi = (qq < 2) ? d[2 * pp + 1][0] : d[2 * pp + 1][1];
            av[pp] = __builtin_amdgcn_perm(hi, lo, sel);
          }
          O[4 * blk + qq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb,
                                                                    O[4 * blk + qq], 0, 0, 0);
        }
      }
    }

    // Partial of split gs for sequence b, slot gs + b. Lane (n16, g4) holds channels
    // 64*blk + 16*g4 + 4*r + qq in O[4*blk + qq][r].
    const int64_t pslot = int64_t(gs) + b;
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (head_ok) {
      float* dst = a.part_o + (pslot * a.Hq + head) * kGqaHeadDim;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<floatx4*>(dst + 64 * blk + 16 * g4 + 4 * r) =
              floatx4{O[4 * blk][r], O[4 * blk + 1][r], O[4 * blk + 2][r], O[4 * blk + 3][r]};
      if (g4 == 0) {
        float* ml = a.part_ml + (pslot * a.Hq + head) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    // Stores drained and LDS reads returned before the next segment reuses the ring.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }
}

// out[b][i][4*q4 .. +4] from the partials of the splits holding part of sequence b.
struct GqaMergeArgs {
  const float* part_o;
  const float* part_ml;
  const int64_t* prefix;
  float* out;
  int B, Hq;
};

__global__ __launch_bounds__(256) void gqa_merge_kernel(GqaMergeArgs a) {
  constexpr int kQuads = kGqaHeadDim / 4;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= int64_t(a.B) * a.Hq * kQuads) return;
  const int q4 = int(idx % kQuads);
  const int head = int((idx / kQuads) % a.Hq);
  const int b = int(idx / (int64_t(kQuads) * a.Hq));
  const Plan plan{a.prefix[a.B + 1], int(a.prefix[a.B + 2])};
  const int64_t P0 = a.prefix[b], P1 = a.prefix[b + 1];
  float M = -INFINITY, den = 0.f;
  floatx4 acc = {};
  if (P1 > P0) {
    const int64_t gf = split_of_tile(P0, plan), gl = split_of_tile(P1 - 1, plan);
    for (int64_t g = gf; g <= gl; ++g) {
      const int64_t row = (g + b) * a.Hq + head;
      const float m = a.part_ml[row * 2], l = a.part_ml[row * 2 + 1];
      const floatx4 o = *reinterpret_cast<const floatx4*>(a.part_o + row * kGqaHeadDim + 4 * q4);
      if (m == -INFINITY) continue;
      if (m > M) {
        const float sc = __builtin_amdgcn_exp2f(M - m);  // 0 when M is -inf
        den *= sc;
        acc *= sc;
        M = m;
      }
      const float w = __builtin_amdgcn_exp2f(m - M);
      den = fmaf(w, l, den);
      acc += w * o;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  *reinterpret_cast<floatx4*>(a.out + (int64_t(b) * a.Hq + head) * kGqaHeadDim + 4 * q4) = acc * inv;
}

// Resident single-wave GQA workgroups on the current device, cached per device.
int gqa_resident(int32_t* out) {
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] > 0) {
      *out = cache[dev];
      return MLRA_OK;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(gqa_decode_kernel), 64, 0);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  const int n = cus * (per_cu < 1 ? 1 : per_cu);
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = n;
  }
  *out = n;
  return MLRA_OK;
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_gqa_num_splits(const mlra_gqa_params* p, int32_t* num_splits) {
  const int rc = mlra_gqa_check_params(p);
  if (rc) return rc;
  if (!num_splits) return set_error(MLRA_ERR_NULL, "num_splits output pointer is NULL");
  if (p->num_splits > 0) {
    *num_splits = p->num_splits;
    return MLRA_OK;
  }
  int32_t n = 0;
  const int r = gqa_resident(&n);
  if (r) return r;
  *num_splits = n / p->num_kv_heads > 0 ? n / p->num_kv_heads : 1;
  return MLRA_OK;
}

extern "C" int mlra_gqa_workspace_size(const mlra_gqa_params* p, size_t* bytes) {
  if (!bytes) return set_error(MLRA_ERR_NULL, "bytes output pointer is NULL");
  int32_t G = 0;
  const int rc = mlra_gqa_num_splits(p, &G);
  if (rc) return rc;
  *bytes = gqa_layout(*p, G).total;
  return MLRA_OK;
}

extern "C" int mlra_gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                               const int32_t* seqlens, float* out, const mlra_gqa_params* p, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int32_t G = 0;
  GqaLayout lay;
  int rc = gqa_prepare(p, seqlens, workspace, workspace_bytes, &G, &lay);
  if (rc) return rc;
  if (p->batch == 0) return MLRA_OK;
  if (!q || !k_cache || !v_cache || !out)
    return set_error(MLRA_ERR_NULL, "q, k_cache, v_cache and out must be non-NULL");
  if ((p->page_size > 0) != (block_table != nullptr))
    return set_error(MLRA_ERR_NULL, "block_table must be given exactly when page_size > 0");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return set_error(MLRA_ERR_ALIGN, "q, k_cache, v_cache and out must be 16-byte aligned");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  GqaArgs a;
  a.q = static_cast<const unsigned char*>(q);
  a.k = static_cast<const unsigned char*>(k_cache);
  a.v = static_cast<const unsigned char*>(v_cache);
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.part_o = reinterpret_cast<float*>(ws + lay.part_o_off);
  a.part_ml = reinterpret_cast<float*>(ws + lay.part_ml_off);
  a.prefix = reinterpret_cast<int64_t*>(ws + lay.prefix_off);
  a.B = p->batch;
  a.Hq = p->num_q_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.G_req = G;
  a.page_size = p->page_size > 0 ? p->page_size : 1;
  a.max_seqlen = p->max_seqlen;
  a.max_pages = p->max_pages_per_seq;
  a.q_sb = p->q_stride_b * 2;
  a.q_sh = p->q_stride_h * 2;
  a.k_st = p->k_stride_tok * 2;
  a.k_sh = p->k_stride_head * 2;
  a.v_st = p->v_stride_tok * 2;
  a.v_sh = p->v_stride_head * 2;
  a.c = p->sm_scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(gqa_decode_kernel, dim3(G, p->num_kv_heads), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "GQA decode kernel launch");
  GqaMergeArgs m;
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.prefix = a.prefix;
  m.out = out;
  m.B = p->batch;
  m.Hq = p->num_q_heads;
  const int64_t n = int64_t(p->batch) * p->num_q_heads * (kGqaHeadDim / 4);
  hipLaunchKernelGGL(gqa_merge_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, m);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "GQA merge kernel launch");
  return MLRA_OK;
}
