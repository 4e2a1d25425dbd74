// Exact log-sum-exp merge of partial attention results.
//
// "Dropping the Anchor ..." Section 2.2: an online-softmax merge of the
// gathered per-shard results gives exact attention over all retained shards.
// The Star Attention review states the corrected update: part h contributes
// exp(s_h - s_global) * A_h, where A_h is the part's normalised output and s_h
// its log-sum-exp.  Hence, per query row and head,
//   lse = ln sum_p exp(lse_p),   o = sum_p exp(lse_p - lse) * o_p.
// Parts with lse = -inf (no keys) contribute nothing.
//
// One wave per (sequence, token, head) row; each lane owns D/64 output
// columns; the part statistics are read as a broadcast by every lane.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(int64_t n_rows, int32_t n_parts,
                                                        int32_t rows_per_seq,
                                                        const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        float* __restrict__ o,
                                                        float* __restrict__ lse) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int64_t seq = row / rows_per_seq;
  const int64_t r = row - seq * rows_per_seq;
  const int64_t base = seq * n_parts * (int64_t)rows_per_seq;  // row index of part 0
  float mx = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mx = fmaxf(mx, lse_part[base + (int64_t)p * rows_per_seq + r]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float sum = 0.f;
  if (mx > -INFINITY) {
    for (int p = 0; p < n_parts; ++p) {
      const int64_t pr = base + (int64_t)p * rows_per_seq + r;
      const float lp = lse_part[pr];
      if (lp == -INFINITY) continue;
      const float w = expf(lp - mx);
      sum += w;
      const float* src = o_part + pr * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, src[lane + 64 * e], acc[e]);
    }
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[row * D + lane + 64 * e] = acc[e] * inv;
  if (lse && lane == 0) lse[row] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

int launch_merge(int32_t batch, int32_t n_parts, int32_t q_len, int32_t n_q_heads,
                 int32_t head_dim, const float* o_part, const float* lse_part, float* o,
                 float* lse, hipStream_t stream) {
  const int32_t rows_per_seq = q_len * n_q_heads;
  const int64_t n_rows = (int64_t)batch * rows_per_seq;
  const int64_t grid = (n_rows + 3) / 4;
  if (head_dim == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, n_rows, n_parts,
                       rows_per_seq, o_part, lse_part, o, lse);
  else
    hipLaunchKernelGGL(lse_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, n_rows, n_parts,
                       rows_per_seq, o_part, lse_part, o, lse);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
