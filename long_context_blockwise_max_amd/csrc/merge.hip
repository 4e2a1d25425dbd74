// Exact log-sum-exp merge of partial attention results: one wave per
// (sequence, token, head) row, each running merge_row (merge_row.hpp, where the
// formula and its sources are stated).
#include "launch.hpp"
#include "merge_row.hpp"

namespace pulsar {

template <int D>
__global__ void __launch_bounds__(256) lse_merge_kernel(int64_t n_rows, int32_t n_parts,
                                                        int32_t rows_per_seq,
                                                        const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        float* __restrict__ o,
                                                        float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int64_t seq = row / rows_per_seq;
  const int64_t r = row - seq * rows_per_seq;
  const int64_t base = seq * n_parts * (int64_t)rows_per_seq + r;  // row of part 0
  merge_row<D>(o_part, lse_part, base, rows_per_seq, n_parts, o + row * D,
                      lse ? lse + row : nullptr);
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
