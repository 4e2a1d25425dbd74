// Max-IDF summary selection on gfx950.
//
// "Dropping the Anchor ..." Section 2.1 / Figure 2: each block is a document,
// df(t) counts the blocks that contain t, a 32-token chunk is scored by its
// rarest token (max idf = log(N / min df)), and the k best chunks per block are
// kept in original order.  Because log(N / x) is strictly decreasing in x, the
// kernels rank chunks by the integer min df: lower is better, the earlier
// chunk wins among equals.  No floating point is involved.
//
// Three launches:
//   select_clear    zero df[V] and the status word
//   select_df       one workgroup per block: an LDS bitmap over the vocabulary
//                   marks the block's distinct tokens; the lane that flips a
//                   bit from 0 to 1 adds 1 to df[t] in global memory
//   select_topk     one workgroup per block: chunk min-df into LDS, an LDS
//                   histogram over the score range finds the cut-off score, and
//                   wave ballots + mbcnt rank ties in chunk order and compact
//                   the kept chunks in ascending order
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

__global__ void __launch_bounds__(256) select_clear(int32_t* __restrict__ df, int32_t vocab,
                                                    int32_t* __restrict__ status) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) status[0] = 0;
  for (; i < vocab; i += (int64_t)gridDim.x * blockDim.x) df[i] = 0;
}

__global__ void __launch_bounds__(1024) select_df(const int32_t* __restrict__ tok, int32_t block_size,
                                                  int32_t vocab, int32_t* __restrict__ df,
                                                  int32_t* __restrict__ status) {
  extern __shared__ uint32_t bits[];  // ceil(vocab / 32) words
  const int nwords = (vocab + 31) >> 5;
  for (int w = threadIdx.x; w < nwords; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  const int32_t* t = tok + (int64_t)blockIdx.x * block_size;
  bool bad = false;
  for (int p = threadIdx.x; p < block_size; p += blockDim.x) {
    int32_t id = t[p];
    if (id < 0 || id >= vocab) {
      bad = true;
      continue;
    }
    uint32_t m = 1u << (id & 31);
    uint32_t old = atomicOr(&bits[id >> 5], m);
    if (!(old & m)) atomicAdd(&df[id], 1);
  }
  if (bad) atomicOr(status, 1);
}

// exclusive prefix of `pred` over the workgroup's threads in thread order;
// returns this thread's prefix and writes the workgroup total to *total.
__device__ __forceinline__ int wg_exclusive_count(bool pred, int* wave_tot, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint64_t mask = __ballot(pred);
  int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
  if (lane == 0) wave_tot[wave] = __popcll(mask);
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    int c = wave_tot[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

__global__ void __launch_bounds__(kSelThreads) select_topk(
    const int32_t* __restrict__ tok, const int32_t* __restrict__ df, int32_t n_blocks,
    int32_t block_size, int32_t chunk_size, int32_t kept, int32_t vocab,
    int32_t* __restrict__ sel, int32_t* __restrict__ chunk_min_df) {
  extern __shared__ int32_t lds[];
  const int n_chunks = block_size / chunk_size;
  int32_t* score = lds;                    // [n_chunks]
  int32_t* hist = lds + n_chunks;          // [n_blocks + 2]
  __shared__ int wave_tot[kSelWaves];
  __shared__ int cut[2];                   // cut-off score, ties still needed
  const int j = blockIdx.x;
  const int32_t* t = tok + (int64_t)j * block_size;
  const int big = n_blocks + 1;            // a chunk with no valid token ranks last

  for (int h = threadIdx.x; h < n_blocks + 2; h += blockDim.x) hist[h] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) {
    int mn = big;
    const int32_t* ct = t + c * chunk_size;
    for (int e = 0; e < chunk_size; ++e) {
      int32_t id = ct[e];
      if (id >= 0 && id < vocab) mn = min(mn, df[id]);
    }
    score[c] = mn;
    atomicAdd(&hist[mn], 1);
    if (chunk_min_df) chunk_min_df[(int64_t)j * n_chunks + c] = mn;
  }
  __syncthreads();
  if (kept <= 0) return;
  if (threadIdx.x == 0) {
    int cum = 0, th = big;
    for (int s = 0; s <= big; ++s) {
      if (cum + hist[s] >= kept) {
        th = s;
        break;
      }
      cum += hist[s];
    }
    cut[0] = th;
    cut[1] = kept - cum;
  }
  __syncthreads();
  const int th = cut[0], need = cut[1];
  int eq_base = 0, out_base = 0;
  for (int base = 0; base < n_chunks; base += kSelThreads) {
    const int c = base + threadIdx.x;
    const int sc = (c < n_chunks) ? score[c] : big + 1;
    int eq_tot, out_tot;
    int eq_rank = eq_base + wg_exclusive_count(sc == th, wave_tot, &eq_tot);
    bool take = (sc < th) || (sc == th && eq_rank < need);
    int slot = out_base + wg_exclusive_count(take, wave_tot, &out_tot);
    if (take) sel[(int64_t)j * kept + slot] = c;
    eq_base += eq_tot;
    out_base += out_tot;
  }
}

int launch_select(const int32_t* tok, int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                  int32_t kept, int32_t vocab, int32_t* sel, int32_t* chunk_min_df, int32_t* df,
                  int32_t* status, hipStream_t stream) {
  int clear_blocks = (int)std::min<int64_t>(1024, ((int64_t)vocab + 255) / 256);
  hipLaunchKernelGGL(select_clear, dim3(clear_blocks), dim3(256), 0, stream, df, vocab, status);
  size_t bitmap_bytes = (size_t)((vocab + 31) / 32) * 4;
  if (bitmap_bytes > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&select_df),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bitmap_bytes) != hipSuccess)
    return -3;
  hipLaunchKernelGGL(select_df, dim3(n_blocks), dim3(1024), bitmap_bytes, stream, tok,
                     block_size, vocab, df, status);
  int n_chunks = block_size / chunk_size;
  size_t lds = (size_t)(n_chunks + n_blocks + 2) * 4;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&select_topk),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return -3;
  hipLaunchKernelGGL(select_topk, dim3(n_blocks), dim3(kSelThreads), lds, stream, tok, df,
                     n_blocks, block_size, chunk_size, kept, vocab, sel, chunk_min_df);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
