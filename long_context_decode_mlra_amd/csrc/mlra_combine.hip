// Split-KV combine for the decode of mlra_attention.hip: log-sum-exp merge of each
// sequence's split partials, the W_UV up-projection on fp32 MFMA per block of latent
// channels, and the branch sum with the output scale (page "Multi-Head Low-Rank
// Attention", ai.info summary of arXiv 2603.02188, "Key Contributions" #2, #3).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "mlra_device.h"

namespace mlra {
namespace {

// ------------------------------------------------------------------ combine kernel
//
// One workgroup per (query head i, block q of kCombBlock of the NB * d_latent latent channels
// (512, or 128 in the shard form), run z of `sub` sequences). Block q lies in latent head j =
// q*kCombBlock / d_latent, channels c0..c0+kCombBlock-1 of it, c0 = q*kCombBlock % d_latent.
// The runs tile the 32-sequence groups of the ypart layout (sub is 32, 16, 8 or 4).
//  1. merge:   obar[b][k] = sum_s 2^{m_s-M} O_s[c0+k] / sum_s 2^{m_s-M} l_s over the splits
//              s holding part of sequence b (slots g + b, g in [g_first, g_last]), into LDS.
//  2. project: y_q[b][d] = sum_k obar[b][k] * W_UV[j][i][c0+k][d] on fp32 MFMA
//              (M = sequences, N = 128 output channels, K = kCombBlock). Every W_UV row is
//              read by exactly one workgroup of the grid.
//  3. branch sum: y_q goes to the workspace with stores that reach the device's coherence
//              point (sc1), and once they are complete the workgroup counts itself in the
//              arrival counter of (i, z). The last of the head's NBLK block workgroups to arrive
//              reads every y_q' of the run back (sc1 loads, which do not hit a stale L2 line of
//              its own XCD), adds them in the fixed order q' = 0, 1, ..., applies out_scale and
//              stores out, then resets the counter. The sum is the same whichever workgroup
//              arrives last. No workgroup waits for another. (Fences at device scope would
//              write back and invalidate the XCD's whole L2 instead of these few lines.)

struct CombineArgs {
  const void* part_o;   // fp32, or fp16 scaled per 64-channel block (bf16 caches)
  const int* part_e;    // the block exponents of fp16 partials
  const float* part_ml;
  const int64_t* prefix;
  const float* W_UV;
  float* ypart;    // [groups][h][nblk][32][128]
  int* counters;   // [h][runs]: arrivals per (query head, run); zero before the launch
  float* out;      // [B][h][128]
  int B, h;
  int sub;         // sequences per workgroup: a power of two dividing kCombSeqs
  float out_scale;
};

constexpr int kCombSeqs = 32;
constexpr int kCombTPS = kCombBlock / 16;  // merge threads per sequence, 4 channel quads each
constexpr int kSc1 = 16;                   // cache-policy bits of the buffer builtins: sc1

struct MergeState {
  float M, den;
  floatx4 acc[4];
};

// Fold one unnormalised partial (max m, sum l, four channel quads o stored as O * 2^-e) into st.
__device__ __forceinline__ void merge_in(MergeState& st, float m, float l, const floatx4 (&o)[4], int e = 0) {
  if (m == -INFINITY) return;
  if (m > st.M) {
    const float sc = __builtin_amdgcn_exp2f(st.M - m);  // 0 when st.M is -inf
    st.den *= sc;
#pragma unroll
    for (int u = 0; u < 4; ++u) st.acc[u] *= sc;
    st.M = m;
  }
  const float w = __builtin_amdgcn_exp2f(m - st.M);
  st.den = fmaf(w, l, st.den);
  const float wo = __builtin_amdgcn_ldexpf(w, e);
#pragma unroll
  for (int u = 0; u < 4; ++u) st.acc[u] += wo * o[u];
}

typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));

// Workgroup barrier that orders LDS only (the W_UV loads issued first stay in flight).
__device__ __forceinline__ void comb_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Buffer resource over `bytes` bytes at p (raw buffer, range-checked: reads past it return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t comb_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), bytes, 0x00020000);
}

template <int NB, int DL, typename P>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int kBatch = 4;  // slots loaded together
  constexpr int kSteps = kCombBlock / 2;  // K steps of the 32x32x2 MFMA
  constexpr int NBLK = NB * DL / kCombBlock;
  constexpr int kBlockFloats = kCombSeqs * kDV;
  __shared__ float ob[kCombBlock][kCombSeqs];  // merged block, k-major: ob[k][b]
  __shared__ float st_red[18 * 128];            // per (receiving slot part, pair): M, den, acc[16]
  __shared__ int last_arrival;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i = blockIdx.x;
  const int q = blockIdx.y;
  const int b0 = blockIdx.z * a.sub;  // first sequence of this workgroup's run
  const int grp = b0 / kCombSeqs;       // its 32-sequence group ...
  const int s0 = b0 % kCombSeqs;        // ... and its first row there
  const int j = (q * kCombBlock) / DL;
  const int c0 = (q * kCombBlock) % DL;
  const int nb = min(a.sub, a.B - b0);
  const int n = lane & 31, hh = lane >> 5;

  // ---- 1. merge. kCombTPS threads per sequence, each owning channel quads cq0 + kCombTPS*v
  // (v < 4); with nbp = nb rounded up to a power of two, S = 256 / (nbp * kCombTPS) slot
  // parts share a sequence.
  int nbp = 1;
  while (nbp < nb) nbp <<= 1;
  const int NPP = nbp * kCombTPS;  // threads per slot part
  const int S = 256 / NPP;
  const int r = tid / NPP;
  const int rem = tid % NPP;
  const int bl = rem / kCombTPS;
  const int cq0 = rem % kCombTPS;
  const bool live = bl < nb;
  const int b = b0 + (live ? bl : 0);

  // The sequence's first and end tiles, then its first batch of partials, then the W_UV slice
  // this wave multiplies by (rows c0 + 2kb + hh, column 32*wave + n). Vector loads retire in
  // order, so the W_UV loads go out after the first partials, which the merge waits for while
  // W_UV is still on its way.
  const int64_t P0 = a.prefix[b], P1 = a.prefix[b + 1];
  const Plan plan{a.prefix[a.B + 1], int(a.prefix[a.B + 2])};
  // Splits gf..gl hold the tiles of sequence b (none when it is empty or the thread idle).
  int64_t gf = 0, gl = -1;
  if (live && P1 > P0) {
    gf = split_of_tile(P0, plan);
    gl = split_of_tile(P1 - 1, plan);
  }
  // Slots g, g + S, ... of the sequence; past the last one the last is read again (slot 0 of
  // the head when there is none) and skipped through m = -inf.
  floatx2 ml[kBatch];
  floatx4 o[kBatch][4];
  int ex[kBatch];
  auto load_batch = [&](int64_t g) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t gg = g + int64_t(u) * S;
      const int64_t slot = gl >= 0 ? min(gg, gl) + b : 0;
      const int64_t row = (slot * NB + j) * a.h + i;
      ml[u] = *reinterpret_cast<const floatx2*>(a.part_ml + row * 2);
      if constexpr (sizeof(P) == 2) {
        ex[u] = a.part_e[row * (DL / kPartBlock) + c0 / kPartBlock];
        const _Float16* po = static_cast<const _Float16*>(a.part_o) + row * DL + c0;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          o[u][v] = __builtin_convertvector(*reinterpret_cast<const halfx4*>(po + 4 * (cq0 + kCombTPS * v)), floatx4);
      } else {
        ex[u] = 0;
        const float* po = static_cast<const float*>(a.part_o) + row * DL + c0;
#pragma unroll
        for (int v = 0; v < 4; ++v) o[u][v] = *reinterpret_cast<const floatx4*>(po + 4 * (cq0 + kCombTPS * v));
      }
      if (gg > gl) ml[u][0] = -INFINITY;
    }
  };
  load_batch(gf + r);
  const float* wcol = a.W_UV + ((int64_t(j) * a.h + i) * DL + c0) * kDV + 32 * wave + n;
  float wv[kSteps];
#pragma unroll
  for (int kb = 0; kb < kSteps; ++kb) wv[kb] = wcol[(2 * kb + hh) * kDV];
  __builtin_amdgcn_sched_barrier(0);

  MergeState st;
  st.M = -INFINITY;
  st.den = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) st.acc[u] = floatx4{};
#pragma unroll
  for (int u = 0; u < kBatch; ++u) merge_in(st, ml[u][0], ml[u][1], o[u], ex[u]);
  for (int64_t g = gf + r + kBatch * S; g <= gl; g += kBatch * S) {
    load_batch(g);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) merge_in(st, ml[u][0], ml[u][1], o[u], ex[u]);
  }
  if (S > 1) {
    // Tree over the slot parts in a fixed order: at each level, part r + half hands its state
    // (M, den, 16 accumulators; each an unnormalised partial of the same form as a split's)
    // to part r < half through st_red[(r * 18 + f) * NPP + rem]. The barriers wait on LDS only,
    // so the W_UV loads stay in flight.
    for (int half = S >> 1; half >= 1; half >>= 1) {
      if (live && r >= half && r < 2 * half) {
        float* sw = st_red + (r - half) * 18 * NPP + rem;
        sw[0] = st.M;
        sw[NPP] = st.den;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) sw[(2 + 4 * u + e) * NPP] = st.acc[u][e];
      }
      comb_lds_barrier();
      if (live && r < half) {
        const float* sr = st_red + r * 18 * NPP + rem;
        floatx4 o1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o1[u] = floatx4{sr[(2 + 4 * u) * NPP], sr[(3 + 4 * u) * NPP], sr[(4 + 4 * u) * NPP], sr[(5 + 4 * u) * NPP]};
        merge_in(st, sr[0], sr[NPP], o1);
      }
      comb_lds_barrier();
    }
  }
  if (r == 0) {
    const float inv = (live && st.den > 0.f) ? 1.f / st.den : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int k = 4 * (cq0 + kCombTPS * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[k + e][s0 + bl] = live ? st.acc[v][e] * inv : 0.f;
    }
  }
  // Rows of the 32-sequence group outside this run read as zero (their outputs are not stored).
  for (int idx = tid; idx < kCombBlock * kCombSeqs; idx += 256) {
    const int col = idx % kCombSeqs;
    if (col < s0 || col >= s0 + nbp) ob[idx / kCombSeqs][col] = 0.f;
  }
  __syncthreads();

  // ---- 2. project: wave w computes output channels [32w, 32w+32) for the group's 32 rows.
  floatx16 y = {};
#pragma unroll
  for (int kb = 0; kb < kSteps; ++kb) y = __builtin_amdgcn_mfma_f32_32x32x2f32(ob[2 * kb + hh][n], wv[kb], y, 0, 0, 0);

  // ---- 3. hand y_q over (rows of this run only) and count the arrival.
  float* yhead = a.ypart + (int64_t(grp) * a.h + i) * NBLK * kBlockFloats;
  float* yq = yhead + q * kBlockFloats;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int row = 8 * (rr >> 2) + 4 * hh + (rr & 3);
    if (unsigned(row - s0) < unsigned(nb))
      __hip_atomic_store(yq + row * kDV + 32 * wave + n, y[rr], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every store of the workgroup has reached the coherence point before the count.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* counter = a.counters + int64_t(i) * gridDim.z + blockIdx.z;
  if (tid == 0)
    last_arrival = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == NBLK - 1;
  __syncthreads();
  if (!last_arrival) return;

  // ---- 4. the last arrival: out[b0 + t][i][:] = out_scale * (y_0 + y_1 + ...)[s0 + t][:].
  const __amdgpu_buffer_rsrc_t yr = comb_rsrc(yhead, NBLK * kBlockFloats * int(sizeof(float)));
  constexpr int kQuads = kDV / 4;
  for (int idx = tid; idx < nb * kQuads; idx += 256) {
    const int t = idx / kQuads, d4 = idx % kQuads;
    const int off = ((s0 + t) * kDV + 4 * d4) * int(sizeof(float));
    floatx4 v[NBLK];
#pragma unroll
    for (int qq = 0; qq < NBLK; ++qq)
      v[qq] = __builtin_amdgcn_raw_buffer_load_b128(yr, off + qq * kBlockFloats * int(sizeof(float)), 0, kSc1);
    floatx4 sum = v[0];
#pragma unroll
    for (int qq = 1; qq < NBLK; ++qq) sum += v[qq];
    *reinterpret_cast<floatx4*>(a.out + (int64_t(b0 + t) * a.h + i) * kDV + 4 * d4) = a.out_scale * sum;
  }
  // Ready for a later combine on the same workspace (the attention kernel clears it as well).
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sequences per combine workgroup: 32 (or B rounded up to a power of two, at least 4),
// halved while the grid holds fewer workgroups than the device has compute units. The
// one-latent-head shard form has a quarter of the channel blocks, so its 32 query heads give
// 64 workgroups at 32 sequences and 256 at 8. Measured on MI355X, B=32, h=32, L=32K, whole
// steps: the shard form 83.4 us at 32 sequences, 80.6 at 8; MLRA-4 and MLA, whose grids
// already fill the device, lose 2 us or more at 16 (each run then reads the W_UV slices again).
int combine_sub(int B, int h, int nblk, int cus) {
  int sub = 4;
  while (sub < kCombSeqs && sub < B) sub <<= 1;
  while (sub > 4 && int64_t(h) * nblk * ((B + sub - 1) / sub) < cus) sub >>= 1;
  return sub;
}

// Compute units of the current device, cached per device.
int device_cus(int* cus) {
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev] > 0) {
      *cus = cache[dev];
      return MLRA_OK;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = *cus;
  }
  return MLRA_OK;
}

using CombineFn = void (*)(CombineArgs);

// The partials of bf16 caches are fp16 (with block exponents), those of fp32 caches fp32.
template <typename P>
CombineFn pick_combine_p(int nb, int dl) {
  if (nb == 4) return combine_kernel<4, 128, P>;
  if (nb == 2) return combine_kernel<2, 256, P>;
  return dl == kShardLatent ? combine_kernel<1, kShardLatent, P> : combine_kernel<1, 512, P>;
}

CombineFn pick_combine(int dtype, int nb, int dl) {
  return dtype == MLRA_BF16 ? pick_combine_p<_Float16>(nb, dl) : pick_combine_p<float>(nb, dl);
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_decode_combine(const int32_t* seqlens, const float* W_UV, float* out,
                                   const mlra_decode_params* p, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int32_t G = 0;
  WorkspaceLayout lay;
  int rc = prepare(p, seqlens, workspace, workspace_bytes, &G, &lay);
  if (rc) return rc;
  if (p->batch == 0) return MLRA_OK;
  if (!W_UV || !out) return set_error(MLRA_ERR_NULL, "W_UV and out must be non-NULL");
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(W_UV) & 3) != 0)
    return set_error(MLRA_ERR_ALIGN, "out must be 16-byte and W_UV 4-byte aligned");
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  CombineArgs c;
  c.part_o = ws + lay.part_o_off;
  c.part_e = reinterpret_cast<const int*>(ws + lay.part_e_off);
  c.part_ml = reinterpret_cast<const float*>(ws + lay.part_ml_off);
  c.prefix = reinterpret_cast<const int64_t*>(ws + lay.prefix_off);
  c.W_UV = W_UV;
  c.ypart = reinterpret_cast<float*>(ws + lay.ypart_off);
  c.counters = reinterpret_cast<int*>(ws + lay.counters_off);
  c.out = out;
  c.B = p->batch;
  c.h = p->num_heads;
  c.out_scale = p->out_scale;
  const int nblk = latent_total(*p) / kCombBlock;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc) return rc;
  c.sub = combine_sub(p->batch, p->num_heads, nblk, cus);
  const dim3 grid(p->num_heads, nblk, (p->batch + c.sub - 1) / c.sub);
  hipLaunchKernelGGL(pick_combine(p->dtype, p->num_branches, p->d_latent), grid, dim3(256), 0,
                     static_cast<hipStream_t>(stream), c);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return MLRA_OK;
}

extern "C" int mlra_decode(const void* q_nope, const void* q_rope, const void* latent_cache, const void* rope_cache,
                           const int32_t* block_table, const int32_t* seqlens, const float* W_UV, float* out,
                           const mlra_decode_params* p, void* workspace, size_t workspace_bytes, void* stream) {
  if (p && p->batch > 0 && (!W_UV || !out)) return set_error(MLRA_ERR_NULL, "W_UV and out must be non-NULL");
  if (p && p->batch > 0 && (!aligned16(out) || (reinterpret_cast<uintptr_t>(W_UV) & 3) != 0))
    return set_error(MLRA_ERR_ALIGN, "out must be 16-byte and W_UV 4-byte aligned");
  int rc = mlra_decode_splitkv(q_nope, q_rope, latent_cache, rope_cache, block_table, seqlens, p, workspace,
                               workspace_bytes, stream);
  if (rc) return rc;
  return mlra_decode_combine(seqlens, W_UV, out, p, workspace, workspace_bytes, stream);
}

