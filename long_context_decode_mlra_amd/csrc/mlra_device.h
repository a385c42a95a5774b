// Device-side pieces shared by the decode translation units: vector types, scalar
// metadata reads, and the split plan that both the attention kernel and the combine
// kernel follow. Header-only; every translation unit gets its own copy.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mlra_internal.h"

namespace mlra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Wave-uniform read of read-only metadata through the scalar data cache. Scalar loads
// are counted by lgkmcnt, so they never wait on the tile loads in flight.
__device__ __forceinline__ int32_t scalar_read(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

inline int hip_fail(hipError_t e, const char* what) {
  return set_error(MLRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------------ split plan
// All sequences are cut into tiles of kTile tokens; the T tiles, taken in
// sequence order, are cut into G = min(G_req, T) contiguous ranges of
// floor/ceil(T/G) tiles. Range g = [g*T/G, (g+1)*T/G). Split g writes its
// partial for sequence b into slot g + b: ranges are ordered, so the sequences
// split g touches are >= those of any earlier split, which makes g + b unique.

__device__ __forceinline__ int64_t tiles_of(int L) { return (int64_t(L) + kTile - 1) / kTile; }

struct Plan {
  int64_t T;
  int G;
};

__device__ __forceinline__ int64_t wave_sum(int64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The batch's sequence lengths, read from memory once per wave: lane l holds seqlens[l] for
// l < min(B, 64), so the plan and the walk of a batch of up to 64 sequences cost one load
// instead of a chain of dependent ones. Lengths past the first 64 are read when asked for.
struct Lens {
  const int32_t* p;
  int B;
  int32_t reg;
};

__device__ __forceinline__ Lens load_lens(const int32_t* __restrict__ p, int B) {
  const int lane = threadIdx.x & 63;
  Lens s;
  s.p = p;
  s.B = B;
  s.reg = lane < B ? p[lane] : 0;
  return s;
}

// Length of sequence base + lane in every lane (0 past B); base is a multiple of 64.
__device__ __forceinline__ int lane_len(const Lens& s, int base) {
  const int b = base + (threadIdx.x & 63);
  return base == 0 ? s.reg : (b < s.B ? s.p[b] : 0);
}

// Length of sequence b, 0 <= b < B, the same b in every lane.
__device__ __forceinline__ int len_of(const Lens& s, int b) {
  return b < 64 ? __builtin_amdgcn_readlane(s.reg, b) : scalar_read(s.p + b);
}

// Every lane of the calling wave gets the same plan.
__device__ inline Plan make_plan(const Lens& s, int G_req) {
  int64_t t = 0;
  for (int base = 0; base < s.B; base += 64) t += tiles_of(lane_len(s, base));
  Plan p;
  p.T = wave_sum(t);
  p.G = int(p.T < G_req ? p.T : G_req);
  return p;
}

__device__ __forceinline__ int64_t split_begin(int64_t g, const Plan& p) { return g * p.T / p.G; }

// Largest split g whose range starts at or before tile x (x < T): the split holding tile x.
__device__ __forceinline__ int64_t split_of_tile(int64_t x, const Plan& p) {
  return ((x + 1) * p.G - 1) / p.T;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// The sequence b holding global tile x (< T) and its first global tile P_b.
__device__ inline void find_sequence(const Lens& s, int64_t x, int& b_out, int64_t& P_out) {
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  for (int base = 0; base < s.B; base += 64) {
    const int b = base + lane;
    const int64_t t = tiles_of(lane_len(s, base));
    const int64_t incl = wave_inclusive_scan(t);
    const int64_t excl = carry + incl - t;
    const unsigned long long hit = __ballot(b < s.B && t > 0 && excl <= x && x < excl + t);
    if (hit) {
      const int src = __ffsll(hit) - 1;
      b_out = base + src;
      P_out = __shfl(excl, src, 64);
      return;
    }
    carry += __shfl(incl, 63, 64);
  }
  b_out = s.B;
  P_out = carry;
}

// prefix[b] = first global tile of sequence b (b <= B), prefix[B+1] = T, prefix[B+2] = G.
// Called by one whole wave.
__device__ inline void write_prefix(const Lens& s, const Plan& p, int64_t* prefix) {
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  for (int base = 0; base < s.B; base += 64) {
    const int b = base + lane;
    const int64_t t = tiles_of(lane_len(s, base));
    const int64_t incl = wave_inclusive_scan(t);
    if (b < s.B) prefix[b] = carry + incl - t;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) {
    prefix[s.B] = carry;
    prefix[s.B + 1] = p.T;
    prefix[s.B + 2] = p.G;
  }
}

struct SegmentWalk {
  int b;       // current sequence
  int64_t Pb;  // its first global tile
  int64_t cur; // next global tile to hand out
  int64_t end; // end of this split's range
};

__device__ inline SegmentWalk begin_walk(const Lens& s, int64_t g, const Plan& p) {
  SegmentWalk w;
  w.cur = split_begin(g, p);
  w.end = split_begin(g + 1, p);
  find_sequence(s, w.cur, w.b, w.Pb);
  return w;
}

// Next (sequence, first tile, end tile) of the split, tiles local to the sequence, and the
// sequence's length L.
__device__ inline bool next_segment(const Lens& s, SegmentWalk& w, int& b, int& ta, int& te, int& L) {
  while (w.cur < w.end && w.b < s.B) {
    const int len = len_of(s, __builtin_amdgcn_readfirstlane(w.b));
    const int64_t n = tiles_of(len);
    const int64_t seg_end = w.end < w.Pb + n ? w.end : w.Pb + n;
    if (n > 0 && w.cur < seg_end) {
      b = w.b;
      ta = int(w.cur - w.Pb);
      te = int(seg_end - w.Pb);
      L = len;
      w.cur = seg_end;
      if (seg_end == w.Pb + n) {
        w.Pb += n;
        ++w.b;
      }
      return true;
    }
    w.Pb += n;
    ++w.b;
  }
  return false;
}

}  // namespace mlra
