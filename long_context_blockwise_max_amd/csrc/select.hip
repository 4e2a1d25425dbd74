// Max-IDF summary selection on gfx950.
//
// "Dropping the Anchor ..." Section 2.1 / Figure 2: each block is a document,
// df(t) counts the blocks that contain t, a 32-token chunk is scored by its
// rarest token (max idf = log(N / min df)), and the k best chunks per block are
// kept in original order.  Because log(N / x) is strictly decreasing in x, the
// kernels rank chunks by the integer min df: lower is better, the earlier
// chunk wins among equals.  No floating point is involved.
//
// Four launches:
//   select_bits     one workgroup per block: an LDS bitmap over the vocabulary
//                   marks the block's distinct valid tokens and is written out
//                   whole (nothing to clear beforehand)
//   select_df_sum   one lane per id: df[t] = the number of block bitmaps holding t
//   select_score    one lane per token over the whole context: the token's df,
//                   then a min over the lanes of its chunk (the chunk's score),
//                   so the df gathers run in parallel on every CU
//   select_topk     one workgroup per block: the block's scores into LDS, an
//                   LDS histogram over the score range finds the cut-off score,
//                   and wave ballots + mbcnt rank ties in chunk order and
//                   compact the kept chunks in ascending order
// (The mean-IDF method below counts df with the same two kernels.)
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

__global__ void __launch_bounds__(64) select_clear(int32_t* __restrict__ status) {
  if (threadIdx.x == 0) status[0] = 0;
}

constexpr int kDfThreads = 1024;
constexpr int kDfBatch = 16;   // tokens a thread loads before its bitmap updates

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

// One workgroup per block: the block's distinct valid ids as a bitmap,
// bits[j * words + t / 32] bit t % 32.  Block 0 also clears the status word.
__global__ void __launch_bounds__(kDfThreads) select_bits(const int32_t* __restrict__ tok,
                                                          int32_t block_size, int32_t vocab,
                                                          uint32_t* __restrict__ bits_out,
                                                          int32_t* __restrict__ status) {
  extern __shared__ uint32_t bits[];  // ceil(vocab / 32) words
  const int nwords = (vocab + 31) >> 5;
  for (int w = threadIdx.x; w < nwords; w += blockDim.x) bits[w] = 0u;
  if (threadIdx.x == 0 && blockIdx.x == 0) status[0] = 0;
  __syncthreads();
  const int32_t* t = tok + (int64_t)blockIdx.x * block_size;
  for (int p0 = 0; p0 < block_size; p0 += kDfThreads * kDfBatch) {
    int32_t ids[kDfBatch];
#pragma unroll
    for (int e = 0; e < kDfBatch; ++e) {
      const int p = p0 + e * kDfThreads + (int)threadIdx.x;
      ids[e] = p < block_size ? t[p] : -1;
    }
#pragma unroll
    for (int e = 0; e < kDfBatch; ++e) {
      if (ids[e] < 0 || ids[e] >= vocab) continue;
      // frequent ids find their bit already set: a plain read spares the atomic
      // (two lanes that both read it clear both set it, which is harmless)
      const uint32_t m = 1u << (ids[e] & 31);
      if (!(bits[ids[e] >> 5] & m)) atomicOr(&bits[ids[e] >> 5], m);
    }
  }
  __syncthreads();
  uint32_t* out = bits_out + (int64_t)blockIdx.x * nwords;
  for (int w = threadIdx.x; w < nwords; w += blockDim.x) out[w] = bits[w];
}

// number of blocks whose bitmap holds id, 8 bitmaps a round with every read of
// the round issued before the first count (a round past the last block re-reads
// block 0's word and counts nothing for it)
__device__ __forceinline__ int df_of(const uint32_t* __restrict__ bits, int nwords, int n_blocks,
                                     int32_t id) {
  const uint32_t* b = bits + (id >> 5);
  const int sh = id & 31;
  int c = 0;
  for (int j0 = 0; j0 < n_blocks; j0 += 8) {
    uint32_t w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = b[(int64_t)(j0 + u < n_blocks ? j0 + u : 0) * nwords];
#pragma unroll
    for (int u = 0; u < 8; ++u) c += j0 + u < n_blocks ? (w[u] >> sh) & 1 : 0;
  }
  return c;
}

// df[t] = number of block bitmaps holding t, for every id t < vocab (lanes of a
// wave read the same bitmap words)
__global__ void __launch_bounds__(256) select_df_sum(const uint32_t* __restrict__ bits,
                                                     int32_t n_blocks, int32_t vocab,
                                                     int32_t* __restrict__ df) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < vocab) df[t] = df_of(bits, (vocab + 31) >> 5, n_blocks, (int32_t)t);
}

// Chunk scores (min df over the chunk; n_blocks + 1 for a chunk with no valid
// token, so it ranks last) of the whole context, score[j * n_chunks + c].
// CS = chunk size when it divides the wave (8, 16, 32 or 64): one lane per
// token, a min over each group of CS lanes.  CS = 0: any chunk size, one thread
// per chunk.
template <int CS>
__global__ void __launch_bounds__(256) select_score(const int32_t* __restrict__ tok,
                                                    const int32_t* __restrict__ df, int64_t L,
                                                    int32_t chunk_size, int32_t n_blocks,
                                                    int32_t vocab, int32_t* __restrict__ score,
                                                    int32_t* __restrict__ status) {
  const int big = n_blocks + 1;
  if constexpr (CS > 0) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // token
    int v = big;
    if (p < L) {
      const int32_t id = tok[p];
      if (id >= 0 && id < vocab) v = df[id];
      else atomicOr(status, 1);   // an id outside [0, V): skipped, flagged
    }
#pragma unroll
    for (int off = CS / 2; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
    if (p < L && (p % CS) == 0) score[p / CS] = v;
  } else {
    const int64_t n = L / chunk_size;
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= n) return;
    const int32_t* ct = tok + c * chunk_size;
    int v = big;
    for (int e0 = 0; e0 < chunk_size; e0 += 8) {
      int32_t ids[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ids[e] = ct[e0 + e];   // chunk_size is a multiple of 8
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (ids[e] >= 0 && ids[e] < vocab) v = min(v, df[ids[e]]);
        else atomicOr(status, 1);
      }
    }
    score[c] = v;
  }
}

__global__ void __launch_bounds__(kSelThreads) select_topk(
    const int32_t* __restrict__ chunk_score, int32_t n_blocks, int32_t n_chunks, int32_t kept,
    int32_t* __restrict__ sel) {
  extern __shared__ int32_t lds[];
  int32_t* score = lds;                    // [n_chunks]
  int32_t* hist = lds + n_chunks;          // [n_blocks + 2]
  __shared__ int wave_tot[kSelWaves];
  __shared__ int cut[2];                   // cut-off score, ties still needed
  const int j = blockIdx.x;
  const int big = n_blocks + 1;            // a chunk with no valid token ranks last

  for (int h = threadIdx.x; h < n_blocks + 2; h += blockDim.x) hist[h] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < n_chunks; c += blockDim.x) {
    const int mn = chunk_score[(int64_t)j * n_chunks + c];
    score[c] = mn;
    atomicAdd(&hist[mn], 1);
  }
  __syncthreads();
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
                  int32_t kept, int32_t vocab, int32_t* sel, int32_t* chunk_score, int32_t* df,
                  uint32_t* bits, int32_t* status, hipStream_t stream) {
  const size_t bitmap_bytes = (size_t)((vocab + 31) / 32) * 4;
  if (bitmap_bytes > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(&select_bits),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bitmap_bytes) != hipSuccess)
    return -3;
  hipLaunchKernelGGL(select_bits, dim3(n_blocks), dim3(kDfThreads), bitmap_bytes, stream, tok,
                     block_size, vocab, bits, status);
  hipLaunchKernelGGL(select_df_sum, dim3((unsigned)(((int64_t)vocab + 255) / 256)), dim3(256), 0,
                     stream, bits, n_blocks, vocab, df);
  const int64_t L = (int64_t)n_blocks * block_size;
  const int n_chunks = block_size / chunk_size;
  if (64 % chunk_size == 0) {
    const dim3 grid((unsigned)((L + 255) / 256));
    switch (chunk_size) {
      case 8: hipLaunchKernelGGL(select_score<8>, grid, dim3(256), 0, stream, tok, df, L, chunk_size, n_blocks, vocab, chunk_score, status); break;
      case 16: hipLaunchKernelGGL(select_score<16>, grid, dim3(256), 0, stream, tok, df, L, chunk_size, n_blocks, vocab, chunk_score, status); break;
      case 32: hipLaunchKernelGGL(select_score<32>, grid, dim3(256), 0, stream, tok, df, L, chunk_size, n_blocks, vocab, chunk_score, status); break;
      default: hipLaunchKernelGGL(select_score<64>, grid, dim3(256), 0, stream, tok, df, L, chunk_size, n_blocks, vocab, chunk_score, status); break;
    }
  } else {
    const int64_t n = L / chunk_size;
    hipLaunchKernelGGL(select_score<0>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       tok, df, L, chunk_size, n_blocks, vocab, chunk_score, status);
  }
  if (kept > 0) {
    size_t lds = (size_t)(n_chunks + n_blocks + 2) * 4;
    if (lds > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&select_topk),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
      return -3;
    hipLaunchKernelGGL(select_topk, dim3(n_blocks), dim3(kSelThreads), lds, stream, chunk_score,
                       n_blocks, n_chunks, kept, sel);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ------------------------------------------------------- other chunk scores
// The alternatives the Dutch technical summary's ablation compares against
// ("Dropping the Anchor ..." Section 2.1 contrasts the maximum with the mean):
//   mean IDF   mean over the chunk's tokens of ln(N / df) (an id outside the
//              vocabulary counts as df = N, idf 0)
//   entropy    Shannon entropy of the chunk's token histogram
//   uniform    k chunks per block uniformly at random: each chunk's key is the
//              SplitMix64 output with counter j * n_chunks + c + 1 from the seed
//              (Steele, Lea and Flood, 2014), the k smallest keys are kept
//   even       chunks floor(m * n_chunks / k), m = 0 .. k-1
// Mean IDF is ln N - (1/C) ln prod_pos df(t_pos) and the entropy
// ln C - (1/C) ln prod_pos c(t_pos), c(t_pos) = count of that token in its
// chunk, so both fall as an integer product over the chunk's positions rises.
// Each chunk's product is formed exactly in 256 bits (the launcher checks that
// it fits), and a chunk is kept when fewer than k chunks of its block have a
// smaller product, or an equal product and a lower index: the same ties as
// Max-IDF, decided exactly.  Three launches, spread over all chunk pairs:
//   select_keys     one thread per chunk: its key into the workspace, its rank
//                   counter zeroed
//   select_rank     one wave per (block, 64 chunks, 64 other chunks): the other
//                   chunks' keys through LDS, each lane counts the ones that beat
//                   its chunk and adds the count to the chunk's rank
//   select_compact  one workgroup per block: chunks with rank < k, in order

constexpr int kKeyLimbs = 8;   // 256-bit keys, little-endian 32-bit limbs
constexpr int kRankTile = 64;  // chunks per side of a select_rank tile

__device__ __forceinline__ void key_mul(uint32_t (&k)[kKeyLimbs], uint32_t f) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < kKeyLimbs; ++i) {
    const uint64_t x = (uint64_t)k[i] * f + carry;
    k[i] = (uint32_t)x;
    carry = x >> 32;
  }
}

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <int METHOD>   // 1 mean IDF, 2 entropy, 3 uniform
__global__ void __launch_bounds__(256) select_keys(
    const int32_t* __restrict__ tok, const int32_t* __restrict__ df, int32_t n_blocks,
    int32_t block_size, int32_t chunk_size, int32_t vocab, uint64_t seed,
    uint32_t* __restrict__ keys, int32_t* __restrict__ ranks, int32_t* __restrict__ status) {
  const int n_chunks = block_size / chunk_size;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_blocks * n_chunks) return;
  uint32_t k[kKeyLimbs] = {1u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if constexpr (METHOD == 3) {
    const uint64_t z = splitmix64(seed, (uint64_t)idx + 1);   // counter j * n_chunks + c + 1
    k[0] = (uint32_t)z;
    k[1] = (uint32_t)(z >> 32);
  } else if (METHOD == 2 && chunk_size == 32) {
    // the method's 32-token chunks: the ids in registers, counted pairwise there
    const int j = (int)(idx / n_chunks), c = (int)(idx % n_chunks);
    const int32_t* ct = tok + (int64_t)j * block_size + (int64_t)c * 32;
    int32_t ids[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 x = reinterpret_cast<const u32x4*>(ct)[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) ids[4 * q + e] = (int32_t)x[e];
    }
    bool bad = false;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      bad |= !(ids[e] >= 0 && ids[e] < vocab);
      uint32_t f = 0;
#pragma unroll
      for (int e2 = 0; e2 < 32; ++e2) f += ids[e2] == ids[e];
      key_mul(k, f);
    }
    if (bad) atomicOr(status, 1);
  } else if (METHOD == 1) {
    // 8 tokens at a time: their ids, then their df values, each group of loads in
    // flight together (chunk_size is a multiple of 8); the product in token order
    const int j = (int)(idx / n_chunks), c = (int)(idx % n_chunks);
    const int32_t* ct = tok + (int64_t)j * block_size + (int64_t)c * chunk_size;
    bool bad = false;
    for (int e0 = 0; e0 < chunk_size; e0 += 8) {
      const u32x4 x0 = reinterpret_cast<const u32x4*>(ct + e0)[0];
      const u32x4 x1 = reinterpret_cast<const u32x4*>(ct + e0)[1];
      int32_t ids[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ids[e] = (int32_t)x0[e];
        ids[4 + e] = (int32_t)x1[e];
      }
      uint32_t f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool in_range = ids[e] >= 0 && ids[e] < vocab;
        bad |= !in_range;
        f[e] = (uint32_t)df[in_range ? ids[e] : 0];
        if (!in_range) f[e] = (uint32_t)n_blocks;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) key_mul(k, f[e]);
    }
    if (bad) atomicOr(status, 1);
  } else {
    const int j = (int)(idx / n_chunks), c = (int)(idx % n_chunks);
    const int32_t* ct = tok + (int64_t)j * block_size + (int64_t)c * chunk_size;
    bool bad = false;
    for (int e = 0; e < chunk_size; ++e) {
      const int32_t id = ct[e];
      bad |= !(id >= 0 && id < vocab);
      uint32_t f = 0;
      for (int e2 = 0; e2 < chunk_size; ++e2) f += ct[e2] == id;
      key_mul(k, f);
    }
    if (bad) atomicOr(status, 1);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(keys + idx * kKeyLimbs);
  dst[0] = u32x4{k[0], k[1], k[2], k[3]};
  dst[1] = u32x4{k[4], k[5], k[6], k[7]};
  ranks[idx] = 0;
}

// -1, 0, 1 as key a (registers) is smaller than, equal to or larger than key b
// -1, 0 or 1 as key a is below, equal to or above key b (16-byte aligned).  All
// limbs are read at once and compared without branches, so that the reads of
// successive comparisons are not serialised behind each other's outcomes.
__device__ __forceinline__ int key_cmp(const uint32_t (&a)[kKeyLimbs], const uint32_t* b) {
  static_assert(kKeyLimbs == 8, "two 16-byte reads per key");
  const u32x4 b0 = reinterpret_cast<const u32x4*>(b)[0];
  const u32x4 b1 = reinterpret_cast<const u32x4*>(b)[1];
  const uint32_t y[kKeyLimbs] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  int r = 0;
#pragma unroll
  for (int i = kKeyLimbs - 1; i >= 0; --i) {
    const int c = (int)(a[i] > y[i]) - (int)(a[i] < y[i]);
    r = r != 0 ? r : c;
  }
  return r;
}

__global__ void __launch_bounds__(kRankTile) select_rank(const uint32_t* __restrict__ keys,
                                                         int32_t n_chunks, int32_t tiles,
                                                         int32_t* __restrict__ ranks) {
  __shared__ __attribute__((aligned(16))) uint32_t other[kRankTile * kKeyLimbs];
  const int per_block = tiles * tiles;
  const int j = blockIdx.x / per_block;
  const int r = blockIdx.x % per_block;
  const int c = (r / tiles) * kRankTile + threadIdx.x;       // this lane's chunk
  const int c2_0 = (r % tiles) * kRankTile;                 // the other chunks
  const uint32_t* kb = keys + (int64_t)j * n_chunks * kKeyLimbs;
  const int n_other = min(kRankTile, n_chunks - c2_0);
  if ((int)threadIdx.x < n_other) {
    const u32x4* src = reinterpret_cast<const u32x4*>(kb + (int64_t)(c2_0 + threadIdx.x) * kKeyLimbs);
    u32x4* dst = reinterpret_cast<u32x4*>(other + threadIdx.x * kKeyLimbs);
    dst[0] = src[0];
    dst[1] = src[1];
  }
  __syncthreads();
  if (c >= n_chunks) return;
  uint32_t k[kKeyLimbs];
  const u32x4* mine = reinterpret_cast<const u32x4*>(kb + (int64_t)c * kKeyLimbs);
  const u32x4 lo = mine[0], hi = mine[1];
  k[0] = lo[0]; k[1] = lo[1]; k[2] = lo[2]; k[3] = lo[3];
  k[4] = hi[0]; k[5] = hi[1]; k[6] = hi[2]; k[7] = hi[3];
  int better = 0;
  for (int u = 0; u < n_other; ++u) {
    const int cmp = key_cmp(k, other + u * kKeyLimbs);
    better += (cmp > 0) || (cmp == 0 && c2_0 + u < c);
  }
  if (better) atomicAdd(&ranks[(int64_t)j * n_chunks + c], better);
}

__global__ void __launch_bounds__(kSelThreads) select_compact(const int32_t* __restrict__ ranks,
                                                              int32_t n_chunks, int32_t kept,
                                                              int32_t* __restrict__ sel) {
  __shared__ int wave_tot[kSelWaves];
  const int j = blockIdx.x;
  int out_base = 0;
  for (int base = 0; base < n_chunks; base += kSelThreads) {
    const int c = base + threadIdx.x;
    const bool take = c < n_chunks && ranks[(int64_t)j * n_chunks + c] < kept;
    int out_tot;
    const int slot = out_base + wg_exclusive_count(take, wave_tot, &out_tot);
    if (take) sel[(int64_t)j * kept + slot] = c;
    out_base += out_tot;
  }
}

__global__ void __launch_bounds__(256) select_even(int32_t n_blocks, int32_t n_chunks,
                                                   int32_t kept, int32_t* __restrict__ sel) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_blocks * kept) return;
  const int m = (int)(i % kept);
  sel[i] = (int32_t)((int64_t)m * n_chunks / kept);
}

int launch_select_method(int32_t method, uint64_t seed, const int32_t* tok, int32_t n_blocks,
                         int32_t block_size, int32_t chunk_size, int32_t kept, int32_t vocab,
                         int32_t* sel, int32_t* df, uint32_t* bits, uint32_t* keys,
                         int32_t* ranks, int32_t* status, hipStream_t stream) {
  const int n_chunks = block_size / chunk_size;
  if (method == 1 && kept > 0) {
    // df as Max-IDF counts it: the block bitmaps (whose first workgroup clears the
    // status word), then the sum over them per id
    const size_t bitmap_bytes = (size_t)((vocab + 31) / 32) * 4;
    if (bitmap_bytes > 65536 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(&select_bits),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bitmap_bytes) != hipSuccess)
      return -3;
    hipLaunchKernelGGL(select_bits, dim3(n_blocks), dim3(kDfThreads), bitmap_bytes, stream, tok,
                       block_size, vocab, bits, status);
    hipLaunchKernelGGL(select_df_sum, dim3((unsigned)(((int64_t)vocab + 255) / 256)), dim3(256), 0,
                       stream, bits, n_blocks, vocab, df);
  } else {
    hipLaunchKernelGGL(select_clear, dim3(1), dim3(64), 0, stream, status);   // status starts at 0
  }
  if (kept <= 0) return hipGetLastError() == hipSuccess ? 0 : -3;
  if (method == 4) {
    const int64_t n = (int64_t)n_blocks * kept;
    hipLaunchKernelGGL(select_even, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       n_blocks, n_chunks, kept, sel);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  const int64_t total = (int64_t)n_blocks * n_chunks;
  const dim3 kgrid((unsigned)((total + 255) / 256));
  if (method == 1)
    hipLaunchKernelGGL(select_keys<1>, kgrid, dim3(256), 0, stream, tok, df, n_blocks, block_size,
                       chunk_size, vocab, seed, keys, ranks, status);
  else if (method == 2)
    hipLaunchKernelGGL(select_keys<2>, kgrid, dim3(256), 0, stream, tok, df, n_blocks, block_size,
                       chunk_size, vocab, seed, keys, ranks, status);
  else
    hipLaunchKernelGGL(select_keys<3>, kgrid, dim3(256), 0, stream, tok, df, n_blocks, block_size,
                       chunk_size, vocab, seed, keys, ranks, status);
  const int tiles = (n_chunks + kRankTile - 1) / kRankTile;
  hipLaunchKernelGGL(select_rank, dim3((unsigned)((int64_t)n_blocks * tiles * tiles)),
                     dim3(kRankTile), 0, stream, keys, n_chunks, tiles, ranks);
  hipLaunchKernelGGL(select_compact, dim3(n_blocks), dim3(kSelThreads), 0, stream, ranks, n_chunks,
                     kept, sel);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
