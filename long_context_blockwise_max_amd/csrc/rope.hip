// Rotary embedding and retained-cache fill (HBM-bound elementwise passes).
//
// Every token keeps its original position ID ("Dropping the Anchor ..."
// Section 2.1; the Star Attention review notes the anchor keeps its original
// indices).  Rotation is the rotate-half form: the pair (x_i, x_{i+d/2}) is
// turned by theta = pos * base^(-2i/d).  theta, cos and sin are float64 and
// rounded to float32 once; at positions near 5e5 a float32 product
// pos * inv_freq would already be off by up to ~0.03 rad.  The rotated values
// are rounded to bf16: they are the attention kernels' MFMA operands.
//
//   rope_fill    Phase-1 prep: q_rot = bf16(RoPE(q)); k_cache = bf16(RoPE(k))
//                re-laid out from [L][Hkv][d] to the per-block, per-head
//                [N][Hkv][b][d] (the keys each block keeps)
//   v_cache_fill the values each block keeps, d-major: [N][Hkv][d][b]
//   phase2_prep  Phase-2 prep in one launch: rotated query rows and rotated
//                self keys (positions pos0 + t), and the d-major copy of the
//                self values
//   self_append  generation: a new token's rotated keys into the self key
//                cache and its values into the d-major self value cache
//
// (The Phase-2 decode form rotates its query rows inside the attention launch,
// with the same angle and rotation functions.)
//
// In rope_fill one thread per (token, 8-wide pair chunk c) derives cos/sin for
// the 8 frequencies 8c .. 8c+7 once and applies them to elements [8c, 8c+8) and
// [d/2 + 8c, d/2 + 8c + 8) of every head of the token.
#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

template <int D>
__device__ __forceinline__ void chunk_angles(int64_t pos, int c, double base, int scaling,
                                             float (&cs)[8], float (&sn)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) rope_cos_sin(pos, 8 * c + e, D / 2, base, scaling, &cs[e], &sn[e]);
}

template <int D>
__device__ __forceinline__ void rotate_chunk(const uint16_t* src, uint16_t* dst, int c,
                                             const float (&cs)[8], const float (&sn)[8]) {
  constexpr int HALF = D / 2;
  const u32x4 x1 = *(const u32x4*)(src + 8 * c);
  const u32x4 x2 = *(const u32x4*)(src + HALF + 8 * c);
  u32x4 y1, y2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a0 = bf16_to_f32(x1[e] & 0xffffu), a1 = bf16_to_f32(x1[e] >> 16);
    const float b0 = bf16_to_f32(x2[e] & 0xffffu), b1 = bf16_to_f32(x2[e] >> 16);
    float u0, v0, u1, v1;
    rope_pair(a0, b0, cs[2 * e], sn[2 * e], u0, v0);
    rope_pair(a1, b1, cs[2 * e + 1], sn[2 * e + 1], u1, v1);
    y1[e] = pack_bf16x2(u0, u1);
    y2[e] = pack_bf16x2(v0, v1);
  }
  *(u32x4*)(dst + 8 * c) = y1;
  *(u32x4*)(dst + HALF + 8 * c) = y2;
}

template <int D>
__global__ void __launch_bounds__(256) rope_fill(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k, int64_t L,
                                                 int32_t block_size, int32_t n_q, int32_t n_kv,
                                                 double base, int32_t scaling,
                                                 uint16_t* __restrict__ q_rot,
                                                 uint16_t* __restrict__ kc) {
  constexpr int HALF = D / 2;
  constexpr int CPH = HALF / 8;  // pair chunks per head row
  const int64_t n = L * CPH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % CPH);
    const int64_t pos = idx / CPH;
    float cs[8], sn[8];
    chunk_angles<D>(pos, c, base, scaling, cs, sn);
    for (int h = 0; h < n_q; ++h) {
      const int64_t r = (pos * n_q + h) * D;
      rotate_chunk<D>(q + r, q_rot + r, c, cs, sn);
    }
    const int64_t blk = pos / block_size;
    const int64_t w = pos - blk * block_size;
    for (int h = 0; h < n_kv; ++h) {
      const int64_t src = (pos * n_kv + h) * D;
      const int64_t dst = ((blk * n_kv + h) * block_size + w) * D;
      rotate_chunk<D>(k + src, kc + dst, c, cs, sn);
    }
  }
}

// d-major V: v [T][Hkv][D] -> vt, element (t, h, d) at vt_index(t, h) + d * ld.
// One workgroup transposes 64 tokens x D of one head through LDS; every thread
// then writes 16-byte runs of 8 consecutive tokens of one d-row.  The 8 tokens
// of a run never straddle a block (tokens are grouped from a multiple of 64
// and the block length is a multiple of 8).
template <int D, class Dst>
__device__ __forceinline__ void transpose_tile(const uint16_t* __restrict__ v, int64_t n_tok,
                                               int32_t n_kv, int h, int64_t t0, Dst dst) {
  __shared__ uint16_t tile[64][D + 8];
  constexpr int CPR = D / 8;
  for (int idx = threadIdx.x; idx < 64 * CPR; idx += blockDim.x) {
    const int r = idx / CPR, c = idx % CPR;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (t0 + r < n_tok) x = *(const u32x4*)(v + ((t0 + r) * n_kv + h) * D + 8 * c);
    *(u32x4*)(&tile[r][8 * c]) = x;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < D * 8; idx += blockDim.x) {
    const int d = idx / 8, run = idx % 8;
    const int64_t t = t0 + 8 * run;
    if (t >= n_tok) continue;
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = (uint32_t)tile[8 * run + 2 * e][d] | ((uint32_t)tile[8 * run + 2 * e + 1][d] << 16);
    *(u32x4*)(dst(t, h, d)) = y;
  }
}

// retained V cache: [N][Hkv][D][b]
template <int D>
__global__ void __launch_bounds__(256) v_cache_fill(const uint16_t* __restrict__ v, int64_t L,
                                                    int32_t block_size, int32_t n_kv,
                                                    uint16_t* __restrict__ vc) {
  transpose_tile<D>(v, L, n_kv, blockIdx.y, (int64_t)blockIdx.x * 64, [&](int64_t t, int h, int d) {
    const int64_t blk = t / block_size, w = t - blk * block_size;
    return vc + ((blk * n_kv + h) * D + d) * block_size + w;
  });
}

// Phase-2 prep.  Workgroups [0, n_tok) take one query-host token each: the
// first D/2 threads derive cos/sin of the token's position into LDS, then the
// workgroup rotates its Hq query heads and (with a self shard) its Hkv key
// heads, one 8-wide pair chunk per thread.  The remaining workgroups transpose
// 64 self-value tokens of one (sequence, head) into the d-major copy
// [B][Hkv][D][lq_pad], zero past Lq.
template <int D>
__global__ void __launch_bounds__(256) phase2_prep(const uint16_t* __restrict__ qq,
                                                   const uint16_t* __restrict__ ks,
                                                   const uint16_t* __restrict__ vs, int32_t lq,
                                                   int32_t n_tok, int32_t hq, int32_t hkv,
                                                   int64_t pos0, double base, int32_t scaling,
                                                   int32_t lq_pad,
                                                   uint16_t* __restrict__ q_rot,
                                                   uint16_t* __restrict__ k_rot,
                                                   uint16_t* __restrict__ vt) {
  constexpr int HALF = D / 2;
  constexpr int CPH = HALF / 8;
  if ((int)blockIdx.x < n_tok) {
    __shared__ float cs_l[HALF], sn_l[HALF];
    const int t = blockIdx.x;
    const int64_t pos = pos0 + t % lq;
    if ((int)threadIdx.x < HALF)
      rope_cos_sin(pos, threadIdx.x, HALF, base, scaling, &cs_l[threadIdx.x], &sn_l[threadIdx.x]);
    __syncthreads();
    const int n_heads = hq + (ks ? hkv : 0);
    for (int idx = threadIdx.x; idx < n_heads * CPH; idx += blockDim.x) {
      const int h = idx / CPH, c = idx % CPH;
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[e] = cs_l[8 * c + e];
        sn[e] = sn_l[8 * c + e];
      }
      if (h < hq) {
        const int64_t r = ((int64_t)t * hq + h) * D;
        rotate_chunk<D>(qq + r, q_rot + r, c, cs, sn);
      } else {
        const int64_t r = ((int64_t)t * hkv + (h - hq)) * D;
        rotate_chunk<D>(ks + r, k_rot + r, c, cs, sn);
      }
    }
    return;
  }
  // self values: workgroup -> (sequence, head, 64-token group)
  const int n_grp = (lq + 63) / 64;
  int w = blockIdx.x - n_tok;
  const int grp = w % n_grp;
  w /= n_grp;
  const int h = w % hkv;
  const int bb = w / hkv;
  const uint16_t* src = vs + (int64_t)bb * lq * hkv * D;
  uint16_t* base_t = vt + (int64_t)bb * hkv * D * lq_pad;
  transpose_tile<D>(src, lq, hkv, h, (int64_t)grp * 64, [&](int64_t tt, int hh, int d) {
    return base_t + ((int64_t)hh * D + d) * lq_pad + tt;
  });
  if (grp == 0)
    for (int idx = threadIdx.x; idx < D * (lq_pad - lq); idx += blockDim.x) {
      const int d = idx / (lq_pad - lq), tt = lq + idx % (lq_pad - lq);
      base_t[((int64_t)h * D + d) * lq_pad + tt] = 0;
    }
}

// Self-cache append (generation): one workgroup per (sequence, new token).  The
// first D/2 threads derive cos/sin of the token's position into LDS; the
// workgroup rotates the token's Hkv key heads into the key cache and writes its
// values into their d-major columns.  The workgroup of the last new token also
// zeroes the value columns from the new length up to the next multiple of 8,
// which the attention kernels read (masked) in runs of 8 keys.
template <int D>
__global__ void __launch_bounds__(256) self_append(const uint16_t* __restrict__ k_new,
                                                   const uint16_t* __restrict__ v_new,
                                                   int32_t n_new, int32_t n_self, int32_t cap,
                                                   int32_t hkv, int64_t pos0, double base,
                                                   int32_t scaling, uint16_t* __restrict__ kc,
                                                   uint16_t* __restrict__ vc) {
  constexpr int HALF = D / 2;
  constexpr int CPH = HALF / 8;
  __shared__ float cs_l[HALF], sn_l[HALF];
  const int j = blockIdx.x % n_new;
  const int bb = blockIdx.x / n_new;
  const int slot = n_self + j;
  if ((int)threadIdx.x < HALF)
    rope_cos_sin(pos0 + slot, threadIdx.x, HALF, base, scaling, &cs_l[threadIdx.x], &sn_l[threadIdx.x]);
  __syncthreads();
  const uint16_t* ksrc = k_new + ((int64_t)bb * n_new + j) * hkv * D;
  uint16_t* kdst = kc + ((int64_t)bb * cap + slot) * hkv * D;
  for (int idx = threadIdx.x; idx < hkv * CPH; idx += blockDim.x) {
    const int h = idx / CPH, c = idx % CPH;
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cs[e] = cs_l[8 * c + e];
      sn[e] = sn_l[8 * c + e];
    }
    rotate_chunk<D>(ksrc + (int64_t)h * D, kdst + (int64_t)h * D, c, cs, sn);
  }
  const uint16_t* vsrc = v_new + ((int64_t)bb * n_new + j) * hkv * D;
  uint16_t* vbase = vc + (int64_t)bb * hkv * D * cap;
  for (int idx = threadIdx.x; idx < hkv * D; idx += blockDim.x)
    vbase[(int64_t)idx * cap + slot] = vsrc[idx];
  if (j == n_new - 1) {
    const int n_tot = n_self + n_new;
    const int pad = ((n_tot + 7) & ~7) - n_tot;
    for (int idx = threadIdx.x; idx < hkv * D * pad; idx += blockDim.x)
      vbase[(int64_t)(idx / pad) * cap + n_tot + idx % pad] = 0;
  }
}

static int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

int launch_rope_fill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t L,
                     int32_t block_size, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     double rope_base, int32_t scaling, uint16_t* q_rot, uint16_t* k_cache,
                     uint16_t* v_cache, hipStream_t stream) {
  const int64_t n = L * (head_dim / 16);
  const dim3 tgrid((unsigned)((L + 63) / 64), (unsigned)n_kv_heads);
  if (head_dim == 128) {
    hipLaunchKernelGGL(rope_fill<128>, dim3(grid_for(n, 256)), dim3(256), 0, stream, q, k, L,
                       block_size, n_q_heads, n_kv_heads, rope_base, scaling, q_rot, k_cache);
    hipLaunchKernelGGL(v_cache_fill<128>, tgrid, dim3(256), 0, stream, v, L, block_size,
                       n_kv_heads, v_cache);
  } else {
    hipLaunchKernelGGL(rope_fill<64>, dim3(grid_for(n, 256)), dim3(256), 0, stream, q, k, L,
                       block_size, n_q_heads, n_kv_heads, rope_base, scaling, q_rot, k_cache);
    hipLaunchKernelGGL(v_cache_fill<64>, tgrid, dim3(256), 0, stream, v, L, block_size,
                       n_kv_heads, v_cache);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_phase2_prep(const uint16_t* qq, const uint16_t* k_self, const uint16_t* v_self,
                       int32_t batch, int32_t q_len, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t head_dim, int64_t pos0, double rope_base, int32_t scaling,
                       int32_t lq_pad, uint16_t* q_rot, uint16_t* k_rot, uint16_t* v_t,
                       hipStream_t stream) {
  const int32_t n_tok = batch * q_len;
  const int32_t n_vt = k_self ? ((q_len + 63) / 64) * n_kv_heads * batch : 0;
  const dim3 grid((unsigned)(n_tok + n_vt));
  if (head_dim == 128)
    hipLaunchKernelGGL(phase2_prep<128>, grid, dim3(256), 0, stream, qq, k_self, v_self, q_len,
                       n_tok, n_q_heads, n_kv_heads, pos0, rope_base, scaling, lq_pad, q_rot, k_rot,
                       v_t);
  else
    hipLaunchKernelGGL(phase2_prep<64>, grid, dim3(256), 0, stream, qq, k_self, v_self, q_len,
                       n_tok, n_q_heads, n_kv_heads, pos0, rope_base, scaling, lq_pad, q_rot, k_rot,
                       v_t);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_self_append(const uint16_t* k_new, const uint16_t* v_new, int32_t batch,
                       int32_t n_new, int32_t n_self, int32_t cap, int32_t n_kv_heads,
                       int32_t head_dim, int64_t pos0, double rope_base, int32_t scaling,
                       uint16_t* k_cache, uint16_t* v_cache, hipStream_t stream) {
  const dim3 grid((unsigned)(batch * n_new));
  if (head_dim == 128)
    hipLaunchKernelGGL(self_append<128>, grid, dim3(256), 0, stream, k_new, v_new, n_new, n_self,
                       cap, n_kv_heads, pos0, rope_base, scaling, k_cache, v_cache);
  else
    hipLaunchKernelGGL(self_append<64>, grid, dim3(256), 0, stream, k_new, v_new, n_new, n_self,
                       cap, n_kv_heads, pos0, rope_base, scaling, k_cache, v_cache);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
