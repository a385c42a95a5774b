// Split-KV decode attention for MLRA (NB latent heads per token) and absorbed MLA
// on gfx950, behind the C ABI of include/mlra.h.
//
// The computation (page "Multi-Head Low-Rank Attention", ai.info summary of
// arXiv 2603.02188): absorbed decode is MQA-style attention of every query head
// over the latent cache followed by the value up-projection ("Main Findings"
// bullet 4). MLRA runs that attention once per latent head with its own softmax
// and sums the per-head up-projected outputs, scaled for the branch count
// ("Key Contributions" #2, #3). Each branch's logit adds the shared RoPE logit
// (per-branch logit space 128 + 64, "Key Contributions" #2).
//
// Kernels (the split partials they write are merged by mlra_combine.hip)
//   decode_branch_kernel  MLRA-4 bf16 with up to 32 query heads: one workgroup per split,
//                     one wave per latent head (branch). Each wave streams its branch's
//                     slice of 32-token tiles (latent channels + RoPE rows) HBM -> LDS
//                     into a private ring, computes S^T = K Q^T and O^T += V^T P^T on bf16
//                     MFMA for all query heads, keeps an fp32 online softmax per query
//                     head, and writes one partial (unnormalised O, running max, running
//                     sum) per sequence it touches; a split that spans sequences keeps its
//                     first partial in registers and stores it after its loads are done.
//                     No workgroup barrier.
//   decode_kernel     the same computation with whole tiles shared by the workgroup's waves
//                     (workgroup barriers per tile): MLRA-4 bf16 with more than 32 query
//                     heads, and every fp32 form.
//   decode_hs_kernel  bf16 with one or two latent heads (MLA, MLRA-2), with the query
//                     heads split across wave pairs.
//   decode_shard_kernel  the shard form, one latent head of 128 channels (bf16, up to 32 query
//                     heads): the branch-wave computation with a split per wave.
// Splitting is balanced over the flattened tiles of all sequences (the plan in mlra_device.h),
// and each XCD runs a contiguous run of splits (xcd_major_split).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "mlra_device.h"

namespace mlra {
namespace {

// Cache policy of the cache-tile loads: non-temporal. Every cache byte is read once per
// step, so allocating it in L2 / the Infinity Cache only evicts useful lines; streaming
// loads measured about 7 TB/s against about 6.1 TB/s for default-policy loads on MI355X.
constexpr int kStreamPolicy = 2;

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's loads of the oldest tile in flight have landed, with `later`
// (0 <= later < S, wave-uniform) tiles issued after it still allowed in flight. Wave w
// issues Q + 1 loads per tile if w < R, else Q.
template <int S, int Q, int R>
__device__ __forceinline__ void wait_tile(int later, int wave) {
  if constexpr (S > 1) {
    if (later == S - 1) {
      if (R > 0 && wave < R)
        wait_vmcnt<(S - 1) * (Q + 1)>();
      else
        wait_vmcnt<(S - 1) * Q>();
      return;
    }
    wait_tile<S - 1, Q, R>(later, wave);
  } else {
    wait_vmcnt<0>();
  }
}

// A running max is only raised once the tile max exceeds it by this many
// log2 units, so exp2 arguments stay <= 8 and unneeded rescales are skipped.
// The final result is exact either way: numerator and denominator share the max.
constexpr float kRescaleSlack = 8.0f;

// ------------------------------------------------------------------ decode kernel

// Workgroup barrier that orders LDS only. __syncthreads() also waits for every
// outstanding global load of the wave (its release fence drains vmcnt), which
// would drain the prefetch of the next tile; here only LDS traffic is drained.
// The asm statement is also a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Splits shorter than this many tiles pay their fixed costs (query loads, one 64 KiB
// partial per sequence touched, the combine's share) on too few cache bytes: below it, with
// two resident workgroups per compute unit, one split per unit streams as fast and halves
// the partials. Measured on MI355X: B=4 L=64K-128K (24 tiles per split at 512 splits) and
// B=64 L=1K-64K (48) run faster with 256 splits, B=32 L=32K (64) with 512.
constexpr int kMinTilesPerSplit = 56;

struct DecodeArgs {
  const unsigned char* q_nope;
  const unsigned char* q_rope;
  const unsigned char* latent;
  const unsigned char* rope;
  const int32_t* block_table;
  const int32_t* seqlens;
  void* part_o;     // fp32 (fp32 caches) or fp16 with per-64-channel-block exponents (bf16 caches)
  int* part_e;      // those exponents (bf16 caches)
  float* part_ml;
  int64_t* prefix;  // [B + 3]: first global tile of each sequence, then T, T, G (written by workgroup 0)
  int* counters;    // [n_counters]: the combine kernel's arrival counters, cleared here
  int n_counters;
  int B, h, G_req, page_size, max_seqlen, max_pages;
  int G_small;                       // > 0: use this many splits when splits would be short (see split_plan)
  int64_t q_sb, q_sh, qr_sb, qr_sh;  // bytes
  int64_t lat_stride, rope_stride;   // bytes
  float c;                           // sm_scale * log2(e)
};

// Clears this workgroup's share of the arrival counters that the combine kernel after it on the
// stream counts its workgroups in (every launched workgroup takes an equal slice; the kernel
// boundary makes the zeros visible to the combine).
__device__ __forceinline__ void clear_counters(const DecodeArgs& a) {
  const int per = (a.n_counters + int(gridDim.x) - 1) / int(gridDim.x);
  const int lo = int(blockIdx.x) * per;
  const int hi = min(a.n_counters, lo + per);
  for (int k = lo + int(threadIdx.x); k < hi; k += int(blockDim.x)) a.counters[k] = 0;
}

// The split plan of a launch of G_req workgroups, switched to G_small splits when the tiles
// would give fewer than kMinTilesPerSplit per split. Workgroups g >= G exit at once; the first
// G_small of them land one per compute unit (workgroups are dealt round-robin over the XCDs).
__device__ __forceinline__ Plan split_plan(const DecodeArgs& a, const Lens& lens) {
  Plan p = make_plan(lens, a.G_req);
  if (a.G_small > 0 && p.T < int64_t(kMinTilesPerSplit) * a.G_req) p.G = int(p.T < a.G_small ? p.T : a.G_small);
  return p;
}

// ---- partials of bf16 caches: fp16 values, one exponent e per 64-channel block, the block
// stored as x * 2^-e. With e taken so that the block's largest magnitude is below 2^(e + 15), no
// stored value can overflow, whatever the cache holds, and each keeps 11 significant bits
// relative to its block's largest value (rounded to nearest even). Halving the partials
// halves the bytes the attention kernel writes at its end and the combine reads.
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int part_exp(float mx) { return __builtin_amdgcn_frexp_expf(mx) - 15; }

__device__ __forceinline__ halfx8 half8_scaled(const float* v, int e) {
  halfx8 h;
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(v[k], -e));
  return h;
}

// The two block exponents of a 128-channel slice held as in tile_pv (lane (n, hh) holds channel
// 32*gg + 16*hh + 4*i + mb in O[mb][4*gg + i]; gg < 2 is block 0). Every lane of the wave calls
// it: a block's largest magnitude combines both lane halves.
__device__ __forceinline__ void slice_exps(const floatx16 (&O)[4], int (&e)[2]) {
  float mx[2] = {0.f, 0.f};
#pragma unroll
  for (int gg = 0; gg < 4; ++gg)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) mx[gg >> 1] = fmaxf(mx[gg >> 1], fabsf(O[mb][4 * gg + i]));
#pragma unroll
  for (int k = 0; k < 2; ++k) e[k] = part_exp(fmaxf(mx[k], __shfl_xor(mx[k], 32, 64)));
}

// Store the slice (dst: its first channel; dst_e: its first block's exponent).
__device__ __forceinline__ void store_slice_f16(_Float16* dst, int* dst_e, const floatx16 (&O)[4], int hh,
                                                const int (&e)[2]) {
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) v[4 * i + mb] = O[mb][4 * gg + i];
    *reinterpret_cast<halfx8*>(dst + 32 * gg + 16 * hh) = half8_scaled(v, e[gg >> 1]);
    *reinterpret_cast<halfx8*>(dst + 32 * gg + 16 * hh + 8) = half8_scaled(v + 8, e[gg >> 1]);
  }
  if (hh == 0) {
    dst_e[0] = e[0];
    dst_e[1] = e[1];
  }
}

// Split run by workgroup wg of the n active ones. Workgroups are dealt round-robin over the
// 8 XCDs (wg % 8), so this gives XCD x a contiguous run of splits, and every XCD reads every
// region of the caches. With split wg on workgroup wg, XCD x read the same eighth of every
// sequence (the same 4 MiB-aligned blocks at B=32, L=32K), and on MI355X the odd XCDs then
// finished 3-5 us after the even ones; with contiguous runs their finish times agree to 0.5 us.
__device__ __forceinline__ int xcd_major_split(int wg, int n) {
  const int x = wg & 7, i = wg >> 3;
  const int q = n >> 3, r = n & 7;
  return x * q + min(x, r) + i;
}

// Tile geometry. The LDS copy of a tile keeps the cache row order; within each row the
// 16-byte chunk c of token t sits at chunk position c ^ lat_swizzle(t) (latent rows) or
// c ^ rope_swizzle(t) (RoPE rows), so the MFMA operand reads hit distinct banks: 16
// consecutive rows read at one logical chunk land on 16 different 16-byte bank groups
// (latent rows are 1 KiB or 2 KiB apart: only the chunk position picks the banks), rows
// 4 apart read as 8-byte column groups land in different 128-byte halves, and two 128-byte
// bf16 RoPE rows that share a 256-byte bank span never collide.
__device__ __forceinline__ int lat_swizzle(int t) { return (t & 7) | ((((t >> 3) ^ (t >> 2)) & 1) << 3); }
template <int kRopeRowBytes>
__device__ __forceinline__ int rope_swizzle(int t) {
  return kRopeRowBytes == 128 ? ((t >> 1) & 7) : (t & 15);
}
template <typename T, int NB, int HB>
struct Geo {
  static constexpr int kEsz = int(sizeof(T));
  static constexpr int kLatRow = kLatentTotal * kEsz;  // bytes of one token's latent row
  static constexpr int kRopeRow = kDRope * kEsz;       // bytes of one token's RoPE row
  static constexpr int kLatTile = kTile * kLatRow;
  static constexpr int kTileBytes = kLatTile + kTile * kRopeRow;
  static constexpr int kWaves = 4 * HB;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kInst = kTileBytes / 1024;  // 64 lanes x 16 bytes per load
  static constexpr int kInstPerWave = (kInst + kWaves - 1) / kWaves;
  static constexpr int kWPB = 4 / NB;  // waves sharing one latent head (each owns 128 channels)
  static constexpr int kDL = kLatentTotal / NB;
  // Loads go straight into LDS unless the idle tile buffer is needed for the
  // logit exchange between the waves that share one latent head.
  static constexpr bool kDirect = (kWPB == 1);
  static constexpr int kStages = 2;  // tile buffers
  static constexpr int kLds = kStages * kTileBytes;
  static_assert(kLatTile % 1024 == 0 && kTileBytes % 1024 == 0, "tile must be whole 1 KiB loads");
  static_assert(kWaves * 4096 <= kTileBytes, "logit exchange must fit the idle tile buffer");
  // Wave w issues the tile load instructions w, w + kWaves, ... below kInst: kLoadsQ + 1
  // of them if w < kLoadsR, else kLoadsQ.
  static constexpr int kLoadsQ = kInst / kWaves;
  static constexpr int kLoadsR = kInst % kWaves;
};

// Per-lane MFMA operands of the query: lane (n, hh) supplies query head 32*hb + n.
template <typename T, int NB>
struct QOps;

template <int NB>
struct QOps<__bf16, NB> {
  static constexpr int kRopeSteps = NB;  // 16-channel RoPE k-steps per wave: 64 / 16 / (4 / NB)
  bf16x8 lat[8];
  bf16x8 rope[kRopeSteps];
};

template <int NB>
struct QOps<float, NB> {
  static constexpr int kRopeGroups = 2 * NB;  // 8-channel RoPE groups per wave: 64 / 8 / (4 / NB)
  floatx4 lat[16];
  floatx4 rope[kRopeGroups];
};

template <typename T, int NB, int HB>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int head, bool head_ok, int wq, int sub, int hh,
                                       QOps<T, NB>& q) {
  using G = Geo<T, NB, HB>;
  const unsigned char* qn = a.q_nope + int64_t(b) * a.q_sb + int64_t(head) * a.q_sh + 128 * wq * G::kEsz;
  const unsigned char* qr = a.q_rope + int64_t(b) * a.qr_sb + int64_t(head) * a.qr_sh;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      q.lat[ks] = head_ok ? *reinterpret_cast<const bf16x8*>(qn + (16 * ks + 8 * hh) * 2) : bf16x8{};
#pragma unroll
    for (int rs = 0; rs < QOps<T, NB>::kRopeSteps; ++rs) {
      const int ks = sub * QOps<T, NB>::kRopeSteps + rs;
      q.rope[rs] = head_ok ? *reinterpret_cast<const bf16x8*>(qr + (16 * ks + 8 * hh) * 2) : bf16x8{};
    }
  } else {
#pragma unroll
    for (int g = 0; g < 16; ++g)
      q.lat[g] = head_ok ? *reinterpret_cast<const floatx4*>(qn + (8 * g + 4 * hh) * 4) : floatx4{};
#pragma unroll
    for (int rg = 0; rg < QOps<T, NB>::kRopeGroups; ++rg) {
      const int g = sub * QOps<T, NB>::kRopeGroups + rg;
      q.rope[rg] = head_ok ? *reinterpret_cast<const floatx4*>(qr + (8 * g + 4 * hh) * 4) : floatx4{};
    }
  }
}

// Where tile `tile` of sequence b starts in the caches (through the block table when paged).
struct TileRows {
  const unsigned char* lat;  // latent row of the tile's first token
  const unsigned char* rope; // RoPE row of the tile's first token
  int last;                  // index of the tile's last valid token
};

__device__ __forceinline__ TileRows tile_rows(const DecodeArgs& a, int b, int L, int tile) {
  const int tok0 = tile * kTile;
  int64_t row0;
  if (a.block_table) {
    // Pages hold a multiple of kTile tokens, so a tile never straddles two pages.
    const int page = scalar_read(a.block_table + int64_t(b) * a.max_pages + tok0 / a.page_size);
    row0 = int64_t(page) * a.page_size + tok0 % a.page_size;
  } else {
    row0 = int64_t(b) * a.max_seqlen + tok0;
  }
  TileRows r;
  r.lat = a.latent + row0 * a.lat_stride;
  r.rope = a.rope + row0 * a.rope_stride;
  r.last = min(kTile, L - tok0) - 1;
  return r;
}

// Source of 16-byte load `inst` (0 .. kInst-1) of a tile for lane `lane`: the
// load fills LDS bytes [inst*1024 + 16*lane, +16) of the tile. Tokens past the
// end of the sequence re-read its last token (valid data; their logits are masked).
template <typename T, int NB, int HB>
__device__ __forceinline__ const unsigned char* load_src(const DecodeArgs& a, const TileRows& tr, int inst,
                                                         int lane) {
  using G = Geo<T, NB, HB>;
  const int off = inst * 1024 + lane * 16;
  // Offsets inside one tile fit 32 bits: 32 rows times a stride below 2^25 bytes.
  if (off < G::kLatTile) {
    const int t = off / G::kLatRow;
    const int c = ((off % G::kLatRow) >> 4) ^ lat_swizzle(t);
    return tr.lat + (min(t, tr.last) * int(a.lat_stride) + c * 16);
  }
  const int o2 = off - G::kLatTile;
  const int t = o2 / G::kRopeRow;
  const int c = ((o2 % G::kRopeRow) >> 4) ^ rope_swizzle<G::kRopeRow>(t);
  return tr.rope + (min(t, tr.last) * int(a.rope_stride) + c * 16);
}

// Register-staged loader: this wave's loads of one tile into registers.
template <typename T, int NB, int HB>
__device__ __forceinline__ void issue_tile_loads(const DecodeArgs& a, int b, int L, int tile, int wave, int lane,
                                                 u32x4 (&stg)[Geo<T, NB, HB>::kInstPerWave]) {
  using G = Geo<T, NB, HB>;
  const TileRows tr = tile_rows(a, b, L, tile);
#pragma unroll
  for (int i = 0; i < G::kInstPerWave; ++i) {
    const int inst = wave + i * G::kWaves;
    if (inst < G::kInst)
      stg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(load_src<T, NB, HB>(a, tr, inst, lane)));
  }
}

// One 16-byte non-temporal load per lane straight into LDS; the wave's 64 lanes fill
// [dst, dst + 1024) in lane order.
__device__ __forceinline__ void dma16(const unsigned char* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, kStreamPolicy);
}

// Direct loader: this wave's loads of one tile go straight from HBM into LDS
// (each load writes 64 lanes x 16 bytes contiguously at the given LDS address).
// Completion is tracked by the wave's vector-memory counter. (Whole-tile offsets computed
// once, as decode_branch_kernel does, measured 2 us slower in decode_hs_kernel.)
template <typename T, int NB, int HB>
__device__ __forceinline__ void issue_tile_dma(const DecodeArgs& a, int b, int L, int tile, int wave, int lane,
                                               unsigned char* buf) {
  using G = Geo<T, NB, HB>;
  const TileRows tr = tile_rows(a, b, L, tile);
#pragma unroll
  for (int i = 0; i < G::kInstPerWave; ++i) {
    const int inst = wave + i * G::kWaves;
    if (inst < G::kInst) dma16(load_src<T, NB, HB>(a, tr, inst, lane), buf + inst * 1024);
  }
}

template <typename T, int NB, int HB>
__device__ __forceinline__ void store_tile(unsigned char* buf, int wave, int lane,
                                           const u32x4 (&stg)[Geo<T, NB, HB>::kInstPerWave]) {
  using G = Geo<T, NB, HB>;
#pragma unroll
  for (int i = 0; i < G::kInstPerWave; ++i) {
    const int inst = wave + i * G::kWaves;
    if (inst < G::kInst) *reinterpret_cast<u32x4*>(buf + inst * 1024 + lane * 16) = stg[i];
  }
}

// S^T[token][head] partial over this wave's 128 latent channels and its share of the RoPE channels.
template <typename T, int NB, int HB>
__device__ __forceinline__ floatx16 tile_logits(const unsigned char* buf, int wq, int n, int hh,
                                                const QOps<T, NB>& q) {
  using G = Geo<T, NB, HB>;
  floatx16 s = {};
  const unsigned char* row = buf + n * G::kLatRow;
  const unsigned char* rrow = buf + G::kLatTile + n * G::kRopeRow;
  const int sw = lat_swizzle(n);
  const int rsw = rope_swizzle<G::kRopeRow>(n);
  const int sub = wq % G::kWPB;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 k = *reinterpret_cast<const bf16x8*>(row + ((16 * wq + ((2 * ks + hh) ^ sw)) << 4));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, q.lat[ks], s, 0, 0, 0);
    }
#pragma unroll
    for (int rs = 0; rs < QOps<T, NB>::kRopeSteps; ++rs) {
      const int ks = sub * QOps<T, NB>::kRopeSteps + rs;
      const bf16x8 k = *reinterpret_cast<const bf16x8*>(rrow + (((2 * ks + hh) ^ rsw) << 4));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, q.rope[rs], s, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const floatx4 k = *reinterpret_cast<const floatx4*>(row + ((32 * wq + ((2 * g + hh) ^ sw)) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(k[e], q.lat[g][e], s, 0, 0, 0);
    }
#pragma unroll
    for (int rg = 0; rg < QOps<T, NB>::kRopeGroups; ++rg) {
      const int g = sub * QOps<T, NB>::kRopeGroups + rg;
      const floatx4 k = *reinterpret_cast<const floatx4*>(rrow + (((2 * g + hh) ^ rsw) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(k[e], q.rope[rg][e], s, 0, 0, 0);
    }
  }
  return s;
}

// O^T[channel][head] += V^T P^T over the tile. Register r of lane half hh holds
// the weight of token tau = 8*(r/4) + 4*hh + r%4; output row m of M-block mb is
// latent channel 4*m + mb of this wave's 128 channels.
template <typename T, int NB, int HB>
__device__ __forceinline__ void tile_pv(const unsigned char* buf, int wq, int n, int hh, const floatx16& p,
                                        floatx16 (&O)[4]) {
  using G = Geo<T, NB, HB>;
  if constexpr (sizeof(T) == 2) {
    // Token tau = 16*ks + 8*(e>>2) + 4*hh + (e&3): its swizzle depends on e and hh only, so
    // there is one lane-dependent base per e and the ks part of the row is an immediate.
    const unsigned char* vb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t0 = 8 * (e >> 2) + 4 * hh + (e & 3);
      vb[e] = buf + t0 * G::kLatRow + (((16 * wq + (n >> 1)) ^ lat_swizzle(t0)) << 4) + ((n & 1) << 3);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const floatx2 f = {p[8 * ks + e], p[8 * ks + e + 1]};
        const bf16x2 v = __builtin_convertvector(f, bf16x2);
        pb[e] = v[0];
        pb[e + 1] = v[1];
      }
      u32x2 d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        d[e] = *reinterpret_cast<const u32x2*>(vb[e] + 16 * ks * G::kLatRow);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint32_t sel = (mb & 1) ? 0x07060302u : 0x05040100u;
        u32x4 av;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t lo = (mb < 2) ? d[2 * pp][0] : d[2 * pp][1];
          const uint32_t hi = (mb < 2) ? d[2 * pp + 1][0] : d[2 * pp + 1][1];
          av[pp] = __builtin_amdgcn_perm(hi, lo, sel);
        }
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, O[mb], 0, 0, 0);
      }
    }
  } else {
    // Token tau = 8*(r>>2) + 4*hh + (r&3); lat_swizzle(tau) repeats with period 16 in tau.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tau = 8 * (r >> 2) + 4 * hh + (r & 3);
      const floatx4 v =
          *reinterpret_cast<const floatx4*>(buf + tau * G::kLatRow + (((32 * wq + n) ^ lat_swizzle(tau)) << 4));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) O[mb] = __builtin_amdgcn_mfma_f32_32x32x2f32(v[mb], p[r], O[mb], 0, 0, 0);
    }
  }
}

template <typename T, int NB, int HB>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 256 * HB),
                          amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 2)))
void decode_kernel(DecodeArgs a) {
  using G = Geo<T, NB, HB>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[G::kLds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: lets tile addressing stay scalar
  const int hb = wave >> 2;       // block of 32 query heads
  const int wq = wave & 3;        // which 128 of the 512 latent channels this wave owns
  const int j = wq / G::kWPB;     // latent head (branch)
  const int sub = wq % G::kWPB;   // part of the branch
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int head = hb * kHeadBlock + n;
  const bool head_ok = head < a.h;

  clear_counters(a);
  const Lens lens = load_lens(a.seqlens, a.B);
  const Plan plan = split_plan(a, lens);
  if (blockIdx.x == 0 && wave == 0) write_prefix(lens, plan, a.prefix);
  if (int(blockIdx.x) >= plan.G) return;
  const int g = xcd_major_split(blockIdx.x, plan.G);
  SegmentWalk walk = begin_walk(lens, g, plan);

  int b, ta, te, L;
  while (next_segment(lens, walk, b, ta, te, L)) {
    // Segment bounds are the same in every lane: keep them (and the loop) scalar.
    b = __builtin_amdgcn_readfirstlane(b);
    ta = __builtin_amdgcn_readfirstlane(ta);
    te = __builtin_amdgcn_readfirstlane(te);
    L = __builtin_amdgcn_readfirstlane(L);
    QOps<T, NB> q;
    floatx16 O[4] = {};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // kStages LDS tile buffers. Direct loads: tile k+kStages-1 is issued before the wave
    // waits for tile k, so kStages tiles are on their way while it waits and kStages-1
    // while tile k is computed. Register staging: tile k+1 is in registers while tile k
    // is computed.
    [[maybe_unused]] u32x4 stg[G::kDirect ? 1 : G::kInstPerWave];
    if constexpr (G::kDirect) {
#pragma unroll
      for (int st = 0; st < G::kStages - 1; ++st)
        if (ta + st < te) issue_tile_dma<T, NB, HB>(a, b, L, ta + st, wave, lane, smem + st * G::kTileBytes);
    } else {
      issue_tile_loads<T, NB, HB>(a, b, L, ta, wave, lane, stg);
    }
    // The queries load while the first tile is on its way.
    load_q<T, NB, HB>(a, b, head, head_ok, wq, sub, hh, q);
    for (int k = ta; k < te; ++k) {
      const int slot = (k - ta) % G::kStages;
      unsigned char* buf = smem + slot * G::kTileBytes;
      unsigned char* idle = smem + ((k - ta + 1) % G::kStages) * G::kTileBytes;
      if constexpr (G::kDirect) {
        if (k + G::kStages - 1 < te) {
          // Tile k+kStages-1 reuses the buffer of tile k-1: every wave must be done with it.
          if (k > ta) lds_barrier();
          issue_tile_dma<T, NB, HB>(a, b, L, k + G::kStages - 1, wave, lane,
                                    smem + ((k - ta + G::kStages - 1) % G::kStages) * G::kTileBytes);
        }
        // This wave's loads of tile k have landed once only the later tiles' loads are pending.
        wait_tile<G::kStages, G::kLoadsQ, G::kLoadsR>(min(G::kStages - 1, te - 1 - k), wave);
        lds_barrier();  // every wave's part of tile k landed
      } else {
        store_tile<T, NB, HB>(buf, wave, lane, stg);
        if (k + 1 < te) issue_tile_loads<T, NB, HB>(a, b, L, k + 1, wave, lane, stg);
        lds_barrier();  // tile k visible to every wave; tile k+1 stays in flight
      }

      floatx16 s = tile_logits<T, NB, HB>(buf, wq, n, hh, q);
      if constexpr (G::kWPB > 1) {
        // Sum the partial logits of the waves that share this latent head, in a fixed order,
        // so every one of them holds bit-identical logits.
        floatx4* red = reinterpret_cast<floatx4*>(idle);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          red[(wave * 4 + qq) * 64 + lane] = floatx4{s[4 * qq], s[4 * qq + 1], s[4 * qq + 2], s[4 * qq + 3]};
        lds_barrier();
        floatx16 tot = {};
#pragma unroll
        for (int w2 = 0; w2 < G::kWPB; ++w2) {
          const int src = hb * 4 + j * G::kWPB + w2;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const floatx4 v = red[(src * 4 + qq) * 64 + lane];
            tot[4 * qq] += v[0];
            tot[4 * qq + 1] += v[1];
            tot[4 * qq + 2] += v[2];
            tot[4 * qq + 3] += v[3];
          }
        }
        lds_barrier();  // exchange area free again before the next tile is stored there
        s = tot;
      }

      const int n_valid = L - k * kTile;
      if (n_valid < kTile) {
        // Register r of lane half hh holds token 8*(r>>2) + 4*hh + (r&3).
        const int lim = n_valid - 4 * hh;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
      }

      // Online softmax in log2 units: x = s * sm_scale * log2(e).
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mt = mx * a.c;
      const bool raise = mt > m_run + kRescaleSlack;
      if (__ballot(raise)) {
        const float mnew = raise ? mt : m_run;
        const float alpha = (mnew == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) O[mb] *= alpha;
        m_run = mnew;
      }
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -m_run));
        psum += s[r];
      }
      l_run += psum;
      tile_pv<T, NB, HB>(buf, wq, n, hh, s, O);
    }
    lds_barrier();  // both tile buffers free before the next segment

    // Partial of split g for sequence b, slot g + b.
    const int64_t pslot = int64_t(g) + b;
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    [[maybe_unused]] int e[2];
    if constexpr (sizeof(T) == 2) slice_exps(O, e);
    if (head_ok) {
      const int64_t row = (pslot * NB + j) * a.h + head;
      if constexpr (sizeof(T) == 2) {
        store_slice_f16(static_cast<_Float16*>(a.part_o) + row * G::kDL + sub * 128,
                        a.part_e + row * (G::kDL / kPartBlock) + 2 * sub, O, hh, e);
      } else {
        float* dst = static_cast<float*>(a.part_o) + row * G::kDL + sub * 128;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            *reinterpret_cast<floatx4*>(dst + 32 * gg + 16 * hh + 4 * i) =
                floatx4{O[0][4 * gg + i], O[1][4 * gg + i], O[2][4 * gg + i], O[3][4 * gg + i]};
      }
      if (hh == 0 && sub == 0) {
        float* ml = a.part_ml + ((pslot * NB + j) * a.h + head) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    // The partial stores share the vector-memory counter with the next segment's tile loads.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// ------------------------------------------------------------------ one wave per branch (MLRA-4, bf16, h <= 32)
//
// Four waves per workgroup; wave j owns latent head (branch) j outright. It streams its own
// slice of every tile, the 128 channels of latent head j in the 32 latent rows (8 KiB) plus
// the 32 RoPE rows (4 KiB), into a private LDS ring of kBranchStages tiles, and computes its
// branch's logits (latent and RoPE channels), softmax and PV alone. No wave waits for another:
// there is no workgroup barrier, and while a wave computes one tile the next kBranchStages-1
// of its own are in flight. All four waves load the same RoPE rows, non-temporally like the
// latent slices; most of the repeats are still served by L2 (measured: 4 % more HBM reads
// than one copy). An L2-allocating policy for the RoPE rows removes that 4 % on clean caches
// but made the kernel up to 1.5x slower on MI355X when the work before it left the caches
// full of dirty lines (a write of 128 MiB or more). The ring takes 144 KiB, so one workgroup
// runs per compute unit, and the split count (one split per resident workgroup) is half that
// of decode_kernel, which halves the partials. MFMA layout as in decode_kernel: S^T = K Q^T
// and O^T += V^T P^T on bf16 32x32x16, tokens as M and the 32 query heads as N.
constexpr int kBranchStages = 3;
constexpr int kBrLatRow = 128 * 2;                 // bytes: one latent head of one token
constexpr int kBrRopeRow = kDRope * 2;             // bytes: one RoPE row
constexpr int kBrLat = kTile * kBrLatRow;          // 8 KiB
constexpr int kBrTile = kBrLat + kTile * kBrRopeRow;  // 12 KiB per wave and tile
constexpr int kBrLoads = kBrTile / 1024;           // 12 loads of 64 lanes x 16 bytes
static_assert(kBrLat == 8 * 1024 && kBrLoads == 12, "branch tile geometry");
static_assert((kBranchStages - 1) * kBrLoads < 64, "vmcnt immediate");
static_assert(4 * kBranchStages * kBrTile <= 160 * 1024, "LDS");

// s_waitcnt immediates for __builtin_amdgcn_s_waitcnt (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8). Unlike inline asm, the builtin is seen by the compiler's
// own wait insertion, which then knows the waited-for loads are complete.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm0Lgkm0 = (7 << 4);

// x combined with the value of lane l ^ 32, in every lane, by one v_permlane32_swap with both
// operands x: result 0 then holds the low half of x in both halves and result 1 the high half,
// so every lane combines the same two values in the same order. (In the kernels with two
// workgroups per CU the LDS shuffle measured as fast or faster, so they keep it.)
__device__ __forceinline__ floatx2 halves_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return floatx2{__builtin_bit_cast(float, uint32_t(r[0])), __builtin_bit_cast(float, uint32_t(r[1]))};
}
__device__ __forceinline__ float halves_max(float x) {
  const floatx2 p = halves_pair(x);
  return fmaxf(p[0], p[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
  const floatx2 p = halves_pair(x);
  return p[0] + p[1];
}

// Latent slice rows: chunk c (of 16) of token t sits at chunk position c ^ (t & 15).
__device__ __forceinline__ int br_lat_swizzle(int t) { return t & 15; }

// Wave j's 12 loads of one tile: 8 latent loads (rows 4i .. 4i+3; lane l -> row 4i + l/16,
// chunk position l%16), then 4 RoPE loads (rows 8i .. 8i+7; lane l -> row 8i + l/8, chunk
// position l%8). Rows past the sequence end re-read its last row (their logits are masked).
// Byte offset of load i for this lane from the tile's first row, clamped to row `last`.
__device__ __forceinline__ uint32_t br_load_offset(const DecodeArgs& a, int i, int j, int lane, int last) {
  if (i < 8) {
    const int r = 4 * i + (lane >> 4);
    return uint32_t(min(r, last) * int(a.lat_stride) + j * kBrLatRow + (((lane & 15) ^ br_lat_swizzle(r)) << 4));
  }
  const int r = 8 * (i - 8) + (lane >> 3);
  return uint32_t(min(r, last) * int(a.rope_stride) + (((lane & 7) ^ rope_swizzle<kBrRopeRow>(r)) << 4));
}

// `full` holds this lane's offsets for a whole tile (computed once): a tile that does not end
// a sequence is then addressed as scalar row base + 32-bit lane offset, with no vector
// arithmetic. Offsets inside one tile fit 32 bits (32 rows, strides below 2^25 bytes).
__device__ __forceinline__ void br_issue_tile(const DecodeArgs& a, int b, int L, int tile, int j, int lane,
                                              unsigned char* buf, const uint32_t (&full)[kBrLoads]) {
  const TileRows tr = tile_rows(a, b, L, tile);
  if (tr.last == kTile - 1) {
#pragma unroll
    for (int i = 0; i < kBrLoads; ++i) dma16((i < 8 ? tr.lat : tr.rope) + full[i], buf + i * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < kBrLoads; ++i)
      dma16((i < 8 ? tr.lat : tr.rope) + br_load_offset(a, i, j, lane, tr.last), buf + i * 1024);
  }
}

// Wait until this wave's loads of the oldest tile in flight have landed, with `later`
// (0 <= later < S, wave-uniform) tiles issued after it still in flight.
template <int S>
__device__ __forceinline__ void br_wait_tile(int later) {
  if constexpr (S > 1) {
    if (later == S - 1) {
      wait_vmcnt<(S - 1) * kBrLoads>();
      return;
    }
    br_wait_tile<S - 1>(later);
  } else {
    wait_vmcnt<0>();
  }
}

// Online-softmax state of one wave for one segment: unnormalised O (channel 32*gg + 16*hh +
// 4*i + mb of the wave's latent head is O[mb][4*gg + i]), running max m in log2 units, and
// the lane half's share l of the denominator.
struct BrAcc {
  floatx16 O[4];
  float m, l;
};

// Tiles [ta, te) of sequence b for latent head j, from the queries to the softmax state.
__device__ __forceinline__ void br_segment(const DecodeArgs& a, int b, int L, int ta, int te, int j, int lane,
                                           bool head_ok, unsigned char* ring, const uint32_t (&full)[kBrLoads],
                                           BrAcc& acc) {
  const int n = lane & 31;
  const int hh = lane >> 5;
  // Query operands: latent K step ks covers channels 16*ks + 8*hh .. +8 of latent head j,
  // RoPE K step rs channels 16*rs + 8*hh .. +8. Lanes past h load head 0 and are zeroed.
  bf16x8 ql[8], qr[4];
  {
    const unsigned char* qn = a.q_nope + int64_t(b) * a.q_sb + int64_t(head_ok ? n : 0) * a.q_sh + 256 * j;
    const unsigned char* qp = a.q_rope + int64_t(b) * a.qr_sb + int64_t(head_ok ? n : 0) * a.qr_sh;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ql[ks] = *reinterpret_cast<const bf16x8*>(qn + (16 * ks + 8 * hh) * 2);
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) qr[rs] = *reinterpret_cast<const bf16x8*>(qp + (16 * rs + 8 * hh) * 2);
  }
  floatx16 (&O)[4] = acc.O;
  float& m_run = acc.m;
  float& l_run = acc.l;
  for (int mb = 0; mb < 4; ++mb) O[mb] = floatx16{};
  m_run = -INFINITY;
  l_run = 0.f;

  // The first kBranchStages-1 tiles go out while the queries are in flight; then wait for
  // the queries only. The wait is a builtin so that the compiler, too, knows the query
  // registers complete: it places no wait of its own on them inside the tile loop.
  int issued = 0;
#pragma unroll
  for (int st = 0; st < kBranchStages - 1; ++st)
    if (ta + st < te) {
      br_issue_tile(a, b, L, ta + st, j, lane, ring + st * kBrTile, full);
      ++issued;
    }
  if (issued == kBranchStages - 1)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((kBranchStages - 1) * kBrLoads));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (!head_ok) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ql[ks] = bf16x8{};
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) qr[rs] = bf16x8{};
  }

  for (int k = ta; k < te; ++k) {
    const unsigned char* buf = ring + ((k - ta) % kBranchStages) * kBrTile;
    if (k + kBranchStages - 1 < te) {
      // Tile k+S-1 reuses tile k-1's buffer: this wave's reads of it have returned.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      br_issue_tile(a, b, L, k + kBranchStages - 1, j, lane,
                    ring + ((k - ta + kBranchStages - 1) % kBranchStages) * kBrTile, full);
    }
    br_wait_tile<kBranchStages>(min(kBranchStages - 1, te - 1 - k));

    // S^T[token][head]: row n of the A operand is token n; chunk 2*ks + hh of latent row n
    // sits at (2*ks + hh) ^ br_lat_swizzle(n), of RoPE row n at (2*rs + hh) ^ rope_swizzle(n).
    floatx16 s = {};
    {
      const unsigned char* lrow = buf + n * kBrLatRow;
      const unsigned char* rrow = buf + kBrLat + n * kBrRopeRow;
      const int sw = br_lat_swizzle(n);
      const int rsw = rope_swizzle<kBrRopeRow>(n);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kk = *reinterpret_cast<const bf16x8*>(lrow + (((2 * ks + hh) ^ sw) << 4));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, ql[ks], s, 0, 0, 0);
      }
#pragma unroll
      for (int rs = 0; rs < 4; ++rs) {
        const bf16x8 kk = *reinterpret_cast<const bf16x8*>(rrow + (((2 * rs + hh) ^ rsw) << 4));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qr[rs], s, 0, 0, 0);
      }
    }
    const int n_valid = L - k * kTile;
    if (n_valid < kTile) {
      // Register r of lane half hh holds token 8*(r>>2) + 4*hh + (r&3).
      const int lim = n_valid - 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) >= lim) s[r] = -INFINITY;
    }
    // Online softmax in log2 units: x = s * sm_scale * log2(e).
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    const float mt = mx * a.c;
    const bool raise = mt > m_run + kRescaleSlack;
    if (__ballot(raise)) {
      const float mnew = raise ? mt : m_run;
      const float alpha = (mnew == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) O[mb] *= alpha;
      m_run = mnew;
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -m_run));
      psum += s[r];
    }
    l_run += psum;

    // O^T[channel][head] += V^T P^T: K step ks covers tokens 16*ks .. +16; lane (n, hh)
    // takes token 16*ks + 8*(e>>2) + 4*hh + (e&3) as K index 8*hh + e. Output row m of
    // M-block mb is channel 4*m + mb: each lane reads channels 4n .. 4n+3 (8 bytes).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 v = __builtin_convertvector((floatx2{s[8 * ks + e], s[8 * ks + e + 1]}), bf16x2);
        pb[e] = v[0];
        pb[e + 1] = v[1];
      }
      u32x2 d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tau = 16 * ks + 8 * (e >> 2) + 4 * hh + (e & 3);
        d[e] = *reinterpret_cast<const u32x2*>(buf + tau * kBrLatRow + (((n >> 1) ^ br_lat_swizzle(tau)) << 4) +
                                               ((n & 1) << 3));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint32_t sel = (mb & 1) ? 0x07060302u : 0x05040100u;
        u32x4 av;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t lo = (mb < 2) ? d[2 * pp][0] : d[2 * pp][1];
          const uint32_t hi = (mb < 2) ? d[2 * pp + 1][0] : d[2 * pp + 1][1];
          av[pp] = __builtin_amdgcn_perm(hi, lo, sel);
        }
        O[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pb, O[mb], 0, 0, 0);
      }
    }
  }
}

// The partial of latent head j (of NB) at slot pslot. Called by every lane of the wave; lanes of
// heads past h store nothing.
template <int NB>
__device__ __forceinline__ void br_store_partial(const DecodeArgs& a, int64_t pslot, int j, int n, int hh,
                                                 bool head_ok, const BrAcc& acc, float l_tot) {
  int e[2];
  slice_exps(acc.O, e);
  if (!head_ok) return;
  const int64_t row = (pslot * NB + j) * a.h + n;
  store_slice_f16(static_cast<_Float16*>(a.part_o) + row * 128, a.part_e + row * 2, acc.O, hh, e);
  if (hh == 0) {
    float* ml = a.part_ml + row * 2;
    ml[0] = acc.m;
    ml[1] = l_tot;
  }
}

// Split g of latent head j (of NB) by one wave, through the ring `ring`: the partial for
// sequence b goes to slot g + b. A store issued while tiles stream in delays every later tile
// wait (the vector-memory counter retires loads and stores in order), so when a split spans
// sequences the first segment's partial stays in registers until the last segment ends, and
// both are stored with no loads in flight. The first segment runs in its own copy of the tile
// loop, free of the held registers.
template <int NB>
__device__ __forceinline__ void br_run_split(const DecodeArgs& a, const Lens& lens, const Plan& plan, int g, int j,
                                             int lane, bool head_ok, unsigned char* ring,
                                             const uint32_t (&full)[kBrLoads]) {
  const int n = lane & 31;
  const int hh = lane >> 5;
  SegmentWalk walk = begin_walk(lens, g, plan);
  int b, ta, te, L;
  if (!next_segment(lens, walk, b, ta, te, L)) return;
  b = __builtin_amdgcn_readfirstlane(b);
  BrAcc first;
  br_segment(a, b, __builtin_amdgcn_readfirstlane(L), __builtin_amdgcn_readfirstlane(ta),
             __builtin_amdgcn_readfirstlane(te), j, lane, head_ok, ring, full, first);
  const int64_t slot0 = int64_t(g) + b;
  const float l0 = halves_sum(first.l);
  if (walk.cur >= walk.end) {
    br_store_partial<NB>(a, slot0, j, n, hh, head_ok, first, l0);
    return;
  }
  while (next_segment(lens, walk, b, ta, te, L)) {
    // LDS reads returned before this segment's loads reuse the ring (a builtin: the
    // compiler's own wait tracking then starts the segment clean).
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    asm volatile("" ::: "memory");
    b = __builtin_amdgcn_readfirstlane(b);
    BrAcc cur;
    br_segment(a, b, __builtin_amdgcn_readfirstlane(L), __builtin_amdgcn_readfirstlane(ta),
               __builtin_amdgcn_readfirstlane(te), j, lane, head_ok, ring, full, cur);
    const float l_tot = halves_sum(cur.l);
    const bool last = walk.cur >= walk.end;
    if (last) br_store_partial<NB>(a, slot0, j, n, hh, head_ok, first, l0);
    br_store_partial<NB>(a, int64_t(g) + b, j, n, hh, head_ok, cur, l_tot);
    if (last) return;
  }
  // Reached only if the walk ended on a segment short of the split's end.
  br_store_partial<NB>(a, slot0, j, n, hh, head_ok, first, l0);
}

// Launch bounds allow one wave per SIMD (the LDS ring admits no more). Built with the MFMA
// VGPR form (-amdgpu-mfma-vgpr-form): otherwise the compiler keeps the accumulators in AGPRs
// and copies them to and from VGPRs every tile.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_branch_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kBranchStages * kBrTile];
  const int lane = threadIdx.x & 63;
  const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // latent head of this wave
  const bool head_ok = (lane & 31) < a.h;  // lane's query head (MFMA column)
  unsigned char* ring = smem + j * (kBranchStages * kBrTile);
  uint32_t full[kBrLoads];
#pragma unroll
  for (int i = 0; i < kBrLoads; ++i) full[i] = br_load_offset(a, i, j, lane, kTile - 1);

  clear_counters(a);
  const Lens lens = load_lens(a.seqlens, a.B);
  const Plan plan = split_plan(a, lens);
  if (blockIdx.x == 0 && j == 0) write_prefix(lens, plan, a.prefix);
  if (int(blockIdx.x) >= plan.G) return;
  br_run_split<4>(a, lens, plan, xcd_major_split(blockIdx.x, plan.G), j, lane, head_ok, ring, full);
}

// ------------------------------------------------------------------ one latent head (shard form)
//
// The shard form caches one latent head of 128 channels plus the RoPE rows: one GPU's share of
// MLRA-4 when the latent heads are spread over four GPUs ("Key Contributions" #2; the branch
// sum then becomes a sum across GPUs). Each wave of a workgroup runs a split of its own, as one
// branch wave of decode_branch_kernel runs its split, so a workgroup runs four consecutive
// splits and the split count is four per resident workgroup.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void decode_shard_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * kBranchStages * kBrTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool head_ok = (lane & 31) < a.h;
  unsigned char* ring = smem + wave * (kBranchStages * kBrTile);
  uint32_t full[kBrLoads];
#pragma unroll
  for (int i = 0; i < kBrLoads; ++i) full[i] = br_load_offset(a, i, 0, lane, kTile - 1);

  clear_counters(a);
  const Lens lens = load_lens(a.seqlens, a.B);
  const Plan plan = split_plan(a, lens);
  if (blockIdx.x == 0 && wave == 0) write_prefix(lens, plan, a.prefix);
  const int wgs = (plan.G + 3) / 4;  // workgroups holding at least one split
  if (int(blockIdx.x) >= wgs) return;
  const int g = 4 * xcd_major_split(blockIdx.x, wgs) + wave;
  if (g >= plan.G) return;
  br_run_split<1>(a, lens, plan, g, 0, lane, head_ok, ring, full);
}

// ------------------------------------------------------------------ split-head decode (NB = 1, 2; bf16)
//
// For one or two latent heads of 512 or 256 channels, splitting the logit channels over all
// four waves would need every wave's partial logits summed each tile. Instead each wave
// (cp, hq) takes 16 query heads hq and accumulates PV for latent channels [256*cp, +256).
// NB = 2: that is latent head j = cp, and the wave computes its full logits (256 latent +
// 64 RoPE channels) itself. NB = 1: the two waves of a head group each compute half of the
// 576-channel logit (256 latent + 32 RoPE channels) and add the other half from a small LDS
// exchange, in a fixed order so both hold identical logits. Tiles go straight into LDS.
// MFMA 16x16x32 bf16, tokens as M (two blocks of 16), heads as N, 32 channels as K:
// lane (n16, g) holds head 16*hq + n16 and tokens 16*mb + 4*g + r (mb < 2, r < 4).

template <int NB, int HB>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 256 * HB), amdgpu_waves_per_eu(2, 2)))
void decode_hs_kernel(DecodeArgs a) {
  static_assert(NB == 1 || NB == 2, "split-head decode is for one or two latent heads");
  using G = Geo<__bf16, NB, HB>;
  constexpr int kLatSteps = 8;                   // 32-channel K steps over 256 latent channels
  constexpr int kRopeSteps = NB == 2 ? 2 : 1;    // over 64 or 32 RoPE channels
  constexpr int kSteps = kLatSteps + kRopeSteps;
  constexpr int DL = kLatentTotal / NB;
  constexpr int kXchBytes = NB == 1 ? 4 * HB * 2 * 64 * 16 : 0;  // per wave: 2 M-blocks x 64 lanes x 16 B
  // Two waves per SIMD: two workgroups per compute unit of one head block, one of two.
  static_assert(2 * G::kTileBytes + kXchBytes <= 81920 * HB, "LDS for two waves per SIMD");
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * G::kTileBytes + kXchBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cp = wave & 1;   // PV channels [256*cp, 256*cp + 256); logit channels, see above
  const int hq = wave >> 1;  // query heads [16*hq, 16*hq + 16)
  const int j = NB == 2 ? cp : 0;
  const int qk_c0 = 256 * cp;  // first latent channel of this wave's logit K steps
  const int n16 = lane & 15;
  const int g = lane >> 4;
  const int head = 16 * hq + n16;
  const bool head_ok = head < a.h;

  clear_counters(a);
  const Lens lens = load_lens(a.seqlens, a.B);
  const Plan plan = split_plan(a, lens);
  if (blockIdx.x == 0 && wave == 0) write_prefix(lens, plan, a.prefix);
  if (int(blockIdx.x) >= plan.G) return;
  const int gsplit = xcd_major_split(blockIdx.x, plan.G);
  SegmentWalk walk = begin_walk(lens, gsplit, plan);

  int b, ta, te, L;
  while (next_segment(lens, walk, b, ta, te, L)) {
    b = __builtin_amdgcn_readfirstlane(b);
    ta = __builtin_amdgcn_readfirstlane(ta);
    te = __builtin_amdgcn_readfirstlane(te);
    L = __builtin_amdgcn_readfirstlane(L);

    // The first tile is on its way while the queries load.
    issue_tile_dma<__bf16, NB, HB>(a, b, L, ta, wave, lane, smem);
    // Query operands: K step st < 8 covers latent channels qk_c0 + 32*st + 8*g .. +8; the RoPE
    // steps cover RoPE channels 32*rs + 8*g (NB = 2: rs = 0, 1; NB = 1: rs = cp).
    bf16x8 qv[kSteps];
    {
      const unsigned char* qn = a.q_nope + int64_t(b) * a.q_sb + int64_t(head) * a.q_sh;
      const unsigned char* qr = a.q_rope + int64_t(b) * a.qr_sb + int64_t(head) * a.qr_sh;
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const int rs = NB == 2 ? st - kLatSteps : cp;
        const unsigned char* src = st < kLatSteps ? qn + (qk_c0 + 32 * st + 8 * g) * 2 : qr + (32 * rs + 8 * g) * 2;
        qv[st] = head_ok ? *reinterpret_cast<const bf16x8*>(src) : bf16x8{};
      }
    }
    floatx4 O[16] = {};
    float m_run = -INFINITY;
    float l_run = 0.f;

    for (int k = ta; k < te; ++k) {
      unsigned char* buf = smem + ((k - ta) & 1) * G::kTileBytes;
      unsigned char* idle = smem + (((k - ta) & 1) ^ 1) * G::kTileBytes;
      // Tile k+1 goes into tile k-1's buffer once every wave is done with it, before this
      // wave waits for tile k: two tiles in flight during the wait.
      if (k + 1 < te) {
        if (k > ta) lds_barrier();
        issue_tile_dma<__bf16, NB, HB>(a, b, L, k + 1, wave, lane, idle);
      }
      wait_tile<2, G::kLoadsQ, G::kLoadsR>(k + 1 < te ? 1 : 0, wave);  // this wave's part of tile k landed
      lds_barrier();  // every wave's part of tile k landed

      // S^T for tokens 16*mb + n16 (A rows) and this wave's 16 heads.
      // K step st = 4u + v reads chunk qk_c0/8 + 16u + ((4v + g) ^ sw) of row 16*mb + n16: the
      // swizzle only permutes the low four bits, so four lane-dependent bases (one per v) and
      // immediate offsets cover every step; the swizzle of both rows is lat_swizzle(n16).
      floatx4 s2[2] = {};
      const int sw = lat_swizzle(n16);
      const int rsw = rope_swizzle<G::kRopeRow>(n16);
      const unsigned char* kb[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) kb[v] = buf + n16 * G::kLatRow + qk_c0 * 2 + (((4 * v + g) ^ sw) << 4);
      const unsigned char* rb[kRopeSteps];
#pragma unroll
      for (int v = 0; v < kRopeSteps; ++v) {
        const int rs = NB == 2 ? v : cp;
        rb[v] = buf + G::kLatTile + n16 * G::kRopeRow + (((4 * rs + g) ^ rsw) << 4);
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          bf16x8 kk;
          if (st < kLatSteps)
            kk = *reinterpret_cast<const bf16x8*>(kb[st & 3] + 16 * mb * G::kLatRow + (st >> 2) * 256);
          else
            kk = *reinterpret_cast<const bf16x8*>(rb[st - kLatSteps] + 16 * mb * G::kRopeRow);
          s2[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qv[st], s2[mb], 0, 0, 0);
        }
      }
      if constexpr (NB == 1) {
        // Add the other half of the logit from the partner wave (wave ^ 1), half 0 first.
        floatx4* xch = reinterpret_cast<floatx4*>(smem + 2 * G::kTileBytes);
        xch[(wave * 2 + 0) * 64 + lane] = s2[0];
        xch[(wave * 2 + 1) * 64 + lane] = s2[1];
        lds_barrier();
        const floatx4 o0 = xch[((wave ^ 1) * 2 + 0) * 64 + lane];
        const floatx4 o1 = xch[((wave ^ 1) * 2 + 1) * 64 + lane];
        s2[0] = cp == 0 ? s2[0] + o0 : o0 + s2[0];
        s2[1] = cp == 0 ? s2[1] + o1 : o1 + s2[1];
      }
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = s2[e >> 2][e & 3];  // token 16*(e>>2) + 4*g + (e&3)
      const int n_valid = L - k * kTile;
      if (n_valid < kTile) {
        const int lim = n_valid - 4 * g;
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
      const bool raise = mt > m_run + kRescaleSlack;
      if (__ballot(raise)) {
        const float mnew = raise ? mt : m_run;
        const float alpha = (mnew == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
        l_run *= alpha;
#pragma unroll
        for (int o = 0; o < 16; ++o) O[o] *= alpha;
        m_run = mnew;
      }
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[e], a.c, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[e + 1], a.c, -m_run));
        psum += p0 + p1;
        const bf16x2 v = __builtin_convertvector((floatx2{p0, p1}), bf16x2);
        pb[e] = v[0];
        pb[e + 1] = v[1];
      }
      l_run += psum;

      // O^T[channel][head] += V^T P^T. K index 8*g + e is token 16*(e>>2) + 4*g + (e&3).
      // M-block 4*blk + q holds channel 256*cp + 64*blk + 4*m + q in row m = n16.
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int chunk = ((256 * cp + 64 * blk) >> 3) + (n16 >> 1);
        u32x2 d[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int tau = 16 * (e >> 2) + 4 * g + (e & 3);
          d[e] = *reinterpret_cast<const u32x2*>(buf + tau * G::kLatRow + ((chunk ^ lat_swizzle(tau)) << 4) +
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
    lds_barrier();  // both tile buffers free before the next segment

    // Partial of split gsplit for sequence b, slot gsplit + b. Lane (n16, g) holds channels
    // 256*cp + 64*blk + 16*g + 4*r + qq in O[4*blk + qq][r].
    const int64_t pslot = int64_t(gsplit) + b;
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    // One exponent per 64-channel block blk of the wave's 256: its channels sit in the four lane
    // groups g (lanes 16 apart), so the block's largest magnitude takes two exchanges.
    int e[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      float mx = 0.f;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(O[4 * blk + qq][r]));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      e[blk] = part_exp(mx);
    }
    if (head_ok) {
      const int64_t prow = (pslot * NB + j) * a.h + head;
      const int c0 = NB == 1 ? 256 * cp : 0;  // the wave's first channel of the latent head
      _Float16* dst = static_cast<_Float16*>(a.part_o) + prow * DL + c0;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) v[4 * r + qq] = O[4 * blk + qq][r];  // channel 64*blk + 16*g + 4*r + qq
        *reinterpret_cast<halfx8*>(dst + 64 * blk + 16 * g) = half8_scaled(v, e[blk]);
        *reinterpret_cast<halfx8*>(dst + 64 * blk + 16 * g + 8) = half8_scaled(v + 8, e[blk]);
      }
      if (g == 0) {
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) a.part_e[prow * (DL / kPartBlock) + c0 / kPartBlock + blk] = e[blk];
      }
      if (g == 0 && (NB == 2 || cp == 0)) {
        float* ml = a.part_ml + ((pslot * NB + j) * a.h + head) * 2;
        ml[0] = m_run;
        ml[1] = l_tot;
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// ------------------------------------------------------------------ host side

using DecodeFn = void (*)(DecodeArgs);

DecodeFn pick_decode(int dtype, int nb, int dl, int hb) {
#define MLRA_PICK(T, NB_)                                                        \
  if (nb == NB_) return hb == 1 ? decode_kernel<T, NB_, 1> : decode_kernel<T, NB_, 2>;
  if (dl * nb != kLatentTotal) return (dtype == MLRA_BF16 && nb == 1 && dl == kShardLatent && hb == 1)
                                          ? decode_shard_kernel : nullptr;
  if (dtype == MLRA_BF16) {
    if (nb == 4) return hb == 1 ? decode_branch_kernel : decode_kernel<__bf16, 4, 2>;
    if (nb == 2) return hb == 1 ? decode_hs_kernel<2, 1> : decode_hs_kernel<2, 2>;
    if (nb == 1) return hb == 1 ? decode_hs_kernel<1, 1> : decode_hs_kernel<1, 2>;
  } else {
    MLRA_PICK(float, 4)
    MLRA_PICK(float, 2)
    MLRA_PICK(float, 1)
  }
#undef MLRA_PICK
  return nullptr;
}

// Resident decode workgroups per device, cached per (device, kernel); *cus_out (optional)
// receives the compute units of the device.
int resident_splits(const mlra_decode_params& p, int32_t* out, int* cus_out = nullptr) {
  static std::mutex mu;
  static int cache[64][2][4][2];  // device, dtype, log2 NB (3: the shard form), HB-1
  static int cus_cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const int hb = head_blocks(p.num_heads);
  const int nbi = is_shard(p) ? 3 : p.num_branches == 4 ? 2 : p.num_branches == 2 ? 1 : 0;
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    if (cache[dev][p.dtype][nbi][hb - 1] > 0) {
      *out = cache[dev][p.dtype][nbi][hb - 1];
      if (cus_out) *cus_out = cus_cache[dev];
      return MLRA_OK;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
  int per_cu = 0;
  const void* kernel = reinterpret_cast<const void*>(pick_decode(p.dtype, p.num_branches, p.d_latent, hb));
  if (!kernel) return set_error(MLRA_ERR_UNSUPPORTED, "no decode kernel for this configuration");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256 * hb, 0);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (per_cu < 1) per_cu = 1;
  const int n = cus * per_cu * (is_shard(p) ? 4 : 1);  // the shard kernel runs a split per wave
  if (dev >= 0 && dev < 64) {
    std::lock_guard<std::mutex> lk(mu);
    cache[dev][p.dtype][nbi][hb - 1] = n;
    cus_cache[dev] = cus;
  }
  *out = n;
  if (cus_out) *cus_out = cus;
  return MLRA_OK;
}

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" int mlra_decode_num_splits(const mlra_decode_params* p, int32_t* num_splits) {
  const int rc = mlra_check_params(p);
  if (rc) return rc;
  if (!num_splits) return set_error(MLRA_ERR_NULL, "num_splits output pointer is NULL");
  if (p->num_splits > 0) {
    *num_splits = p->num_splits;
    return MLRA_OK;
  }
  return resident_splits(*p, num_splits);
}

extern "C" int mlra_decode_workspace_size(const mlra_decode_params* p, size_t* bytes) {
  if (!bytes) return set_error(MLRA_ERR_NULL, "bytes output pointer is NULL");
  int32_t G = 0;
  const int rc = mlra_decode_num_splits(p, &G);
  if (rc) return rc;
  *bytes = workspace_layout(*p, G).total;
  return MLRA_OK;
}

extern "C" int mlra_decode_splitkv(const void* q_nope, const void* q_rope, const void* latent_cache,
                                   const void* rope_cache, const int32_t* block_table, const int32_t* seqlens,
                                   const mlra_decode_params* p, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  int32_t G = 0;
  WorkspaceLayout lay;
  int rc = prepare(p, seqlens, workspace, workspace_bytes, &G, &lay);
  if (rc) return rc;
  if (p->batch == 0) return MLRA_OK;
  if (!q_nope || !q_rope || !latent_cache || !rope_cache)
    return set_error(MLRA_ERR_NULL, "q_nope, q_rope, latent_cache and rope_cache must be non-NULL");
  if ((p->page_size > 0) != (block_table != nullptr))
    return set_error(MLRA_ERR_NULL, "block_table must be given exactly when page_size > 0");
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(latent_cache) || !aligned16(rope_cache))
    return set_error(MLRA_ERR_ALIGN, "q_nope, q_rope, latent_cache and rope_cache must be 16-byte aligned");

  const int64_t esz = p->dtype == MLRA_BF16 ? 2 : 4;
  DecodeArgs a;
  a.q_nope = static_cast<const unsigned char*>(q_nope);
  a.q_rope = static_cast<const unsigned char*>(q_rope);
  a.latent = static_cast<const unsigned char*>(latent_cache);
  a.rope = static_cast<const unsigned char*>(rope_cache);
  a.block_table = block_table;
  a.seqlens = seqlens;
  a.part_o = static_cast<unsigned char*>(workspace) + lay.part_o_off;
  a.part_e = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + lay.part_e_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + lay.part_ml_off);
  a.prefix = reinterpret_cast<int64_t*>(static_cast<unsigned char*>(workspace) + lay.prefix_off);
  a.counters = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + lay.counters_off);
  a.n_counters = int(lay.n_counters);
  a.B = p->batch;
  a.h = p->num_heads;
  a.G_req = G;
  a.G_small = 0;
  if (p->num_splits == 0) {
    // Default split count: allow one split per compute unit instead of two for short splits.
    int32_t resident = 0;
    int cus = 0;
    rc = resident_splits(*p, &resident, &cus);
    if (rc) return rc;
    if (cus > 0 && G >= 2 * cus && !is_shard(*p)) a.G_small = cus;
  }
  a.page_size = p->page_size > 0 ? p->page_size : 1;
  a.max_seqlen = p->max_seqlen;
  a.max_pages = p->max_pages_per_seq;
  a.q_sb = p->q_stride_b * esz;
  a.q_sh = p->q_stride_h * esz;
  a.qr_sb = p->qr_stride_b * esz;
  a.qr_sh = p->qr_stride_h * esz;
  a.lat_stride = p->lat_stride_tok * esz;
  a.rope_stride = p->rope_stride_tok * esz;
  a.c = p->sm_scale * kLog2e;

  const int hb = head_blocks(p->num_heads);
  DecodeFn fn = pick_decode(p->dtype, p->num_branches, p->d_latent, hb);
  if (!fn) return set_error(MLRA_ERR_UNSUPPORTED, "no decode kernel for this configuration");
  const int wgs = is_shard(*p) ? (G + 3) / 4 : G;  // the shard kernel runs four splits per workgroup
  hipLaunchKernelGGL(fn, dim3(wgs), dim3(256 * hb), 0, static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return MLRA_OK;
}

