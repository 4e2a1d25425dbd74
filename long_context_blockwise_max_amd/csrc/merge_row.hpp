// Exact log-sum-exp merge of one query row's partial results, done by one wave.
//
// "Dropping the Anchor ..." Section 2.2: an online-softmax merge of the
// gathered per-shard results gives exact attention over all retained shards.
// The Star Attention review states the corrected update: part h contributes
// exp(s_h - s_global) * A_h, where A_h is the part's normalised output and s_h
// its log-sum-exp.  Hence, per query row and head,
//   lse = ln sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) * o_p.
// Parts with lse = -inf (no keys) contribute nothing.
//
// The lanes read the parts' LSEs in parallel (lane p takes parts p, p + 64, ...)
// and reduce max and sum across the wave; the weighted sum of the part outputs
// then runs over 8 parts at a time with independent loads (lane l owns D/64
// adjacent output columns), the weight of each part broadcast from the lane
// that computed it.  A part with lse = -inf is excluded by a select, so
// whatever its output row holds (0/0 included) never reaches the sum.
#pragma once
#include <math.h>

#include "common.hpp"

namespace pulsar {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
struct Cols;
template <>
struct Cols<128> {
  typedef float2 T;
  static __device__ __forceinline__ void fma(float w, T x, T& a) {
    a.x = fmaf(w, x.x, a.x);
    a.y = fmaf(w, x.y, a.y);
  }
  static __device__ __forceinline__ T zero() { return make_float2(0.f, 0.f); }
  static __device__ __forceinline__ T scale(T a, float s) { return make_float2(a.x * s, a.y * s); }
  static __device__ __forceinline__ T load(const float* p) { return *reinterpret_cast<const T*>(p); }
};
template <>
struct Cols<64> {
  typedef float T;
  static __device__ __forceinline__ void fma(float w, T x, T& a) { a = fmaf(w, x, a); }
  static __device__ __forceinline__ T zero() { return 0.f; }
  static __device__ __forceinline__ T scale(T a, float s) { return a * s; }
  static __device__ __forceinline__ T load(const float* p) { return *p; }
};

// Merge one row: its part p sits at o_part[(base + p * stride) * D] and
// lse_part[base + p * stride]; the result goes to o_row[0 .. D) and *lse_row
// (if not null).  Called by all 64 lanes of one wave.
template <int D>
__device__ __forceinline__ void merge_row(const float* __restrict__ o_part,
                                          const float* __restrict__ lse_part, int64_t base,
                                          int64_t stride, int32_t n_parts, float* __restrict__ o_row,
                                          float* __restrict__ lse_row) {
  using C = Cols<D>;
  using T = typename C::T;
  constexpr int PER = D / 64;   // columns per lane
  const int lane = threadIdx.x & 63;
  auto part_row = [&](int p) { return base + (int64_t)p * stride; };
  float mx = -INFINITY;
  for (int p = lane; p < n_parts; p += 64) mx = fmaxf(mx, lse_part[part_row(p)]);
  mx = wave_max(mx);
  T acc = C::zero();
  float sum = 0.f;
  if (mx > -INFINITY) {
    for (int p0 = 0; p0 < n_parts; p0 += 64) {
      const int pl = p0 + lane;
      const float lp = pl < n_parts ? lse_part[part_row(pl)] : -INFINITY;
      const float wl = lp > -INFINITY ? expf(lp - mx) : 0.f;
      sum += wl;
      const int cnt = min(64, n_parts - p0);
      int j = 0;
      for (; j + 8 <= cnt; j += 8) {
        T x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = C::load(o_part + part_row(p0 + j + u) * D + lane * PER);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = __shfl(wl, j + u);
          T y = x[u];
          if (!(w > 0.f)) y = C::zero();
          C::fma(w, y, acc);
        }
      }
      for (; j < cnt; ++j) {
        const float w = __shfl(wl, j);
        T y = C::load(o_part + part_row(p0 + j) * D + lane * PER);
        if (!(w > 0.f)) y = C::zero();
        C::fma(w, y, acc);
      }
    }
    sum = wave_sum(sum);
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  reinterpret_cast<T*>(o_row)[lane] = C::scale(acc, inv);
  if (lse_row && lane == 0) *lse_row = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

}  // namespace pulsar
