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

// Every lane of the calling wave gets the same plan.
__device__ inline Plan make_plan(const int32_t* __restrict__ seqlens, int B, int G_req) {
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
  for (int b = lane; b < B; b += 64) s += tiles_of(seqlens[b]);
  Plan p;
  p.T = wave_sum(s);
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
__device__ inline void find_sequence(const int32_t* __restrict__ seqlens, int B, int64_t x, int& b_out,
                              int64_t& P_out) {
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int64_t t = b < B ? tiles_of(seqlens[b]) : 0;
    const int64_t incl = wave_inclusive_scan(t);
    const int64_t excl = carry + incl - t;
    const unsigned long long hit = __ballot(b < B && t > 0 && excl <= x && x < excl + t);
    if (hit) {
      const int src = __ffsll(hit) - 1;
      b_out = base + src;
      P_out = __shfl(excl, src, 64);
      return;
    }
    carry += __shfl(incl, 63, 64);
  }
  b_out = B;
  P_out = carry;
}

// prefix[b] = first global tile of sequence b (b <= B), prefix[B+1] = T, prefix[B+2] = G.
// Called by one whole wave.
__device__ inline void write_prefix(const int32_t* __restrict__ seqlens, int B, const Plan& p, int64_t* prefix) {
  const int lane = threadIdx.x & 63;
  int64_t carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int64_t t = b < B ? tiles_of(seqlens[b]) : 0;
    const int64_t incl = wave_inclusive_scan(t);
    if (b < B) prefix[b] = carry + incl - t;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) {
    prefix[B] = carry;
    prefix[B + 1] = p.T;
    prefix[B + 2] = p.G;
  }
}

struct SegmentWalk {
  int b;       // current sequence
  int64_t Pb;  // its first global tile
  int64_t cur; // next global tile to hand out
  int64_t end; // end of this split's range
};

__device__ inline SegmentWalk begin_walk(const int32_t* __restrict__ seqlens, int B, int64_t g, const Plan& p) {
  SegmentWalk w;
  w.cur = split_begin(g, p);
  w.end = split_begin(g + 1, p);
  find_sequence(seqlens, B, w.cur, w.b, w.Pb);
  return w;
}

// Next (sequence, first tile, end tile) of the split, tiles local to the sequence.
__device__ inline bool next_segment(const int32_t* __restrict__ seqlens, int B, SegmentWalk& w, int& b, int& ta,
                             int& te) {
  while (w.cur < w.end && w.b < B) {
    const int64_t n = tiles_of(seqlens[w.b]);
    const int64_t seg_end = w.end < w.Pb + n ? w.end : w.Pb + n;
    if (n > 0 && w.cur < seg_end) {
      b = w.b;
      ta = int(w.cur - w.Pb);
      te = int(seg_end - w.Pb);
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
