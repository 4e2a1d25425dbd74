// Rotary table and retained-cache fill (HBM-bound elementwise passes).
//
// Every token keeps its original position ID ("Dropping the Anchor ..."
// Section 2.1; the Star Attention review notes the anchor keeps its original
// indices).  Rotation is the rotate-half form: the pair (x_i, x_{i+d/2}) is
// turned by theta = pos * base^(-2i/d).  theta, cos and sin are float64 and
// rounded to float32 once; at positions near 5e5 a float32 product
// pos * inv_freq would already be off by up to ~0.03 rad.
//
//   rope_table   cos/sin [L][d/2] float2, read by the Phase-1 query loader
//   rope_fill    k_cache = bf16(RoPE(k)), v_cache = v, re-laid out from
//                [L][Hkv][d] to the per-block, per-head [N][Hkv][b][d]
//                (the KV each block keeps after Phase 1)
#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

__global__ void __launch_bounds__(256) rope_table(float2* __restrict__ cs, int64_t L, int half,
                                                  double base) {
  const int64_t n = L * half;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t pos = idx / half;
    int i = (int)(idx - pos * half);
    float c, s;
    rope_cos_sin(pos, i, half, base, &c, &s);
    cs[idx] = make_float2(c, s);
  }
}

// One thread per (position, kv head, 8-wide pair chunk): loads elements
// [8c, 8c+8) and [d/2 + 8c, d/2 + 8c + 8) of a key row and of a value row.
template <int D>
__global__ void __launch_bounds__(256) rope_fill(const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v,
                                                 const float2* __restrict__ cs, int64_t L,
                                                 int32_t block_size, int32_t n_kv,
                                                 uint16_t* __restrict__ kc,
                                                 uint16_t* __restrict__ vc) {
  constexpr int HALF = D / 2;
  constexpr int CPH = HALF / 8;  // pair chunks per head row
  const int64_t n = L * n_kv * CPH;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(idx % CPH);
    const int64_t rest = idx / CPH;
    const int hd = (int)(rest % n_kv);
    const int64_t pos = rest / n_kv;
    const int64_t src = (pos * n_kv + hd) * D;
    const int64_t blk = pos / block_size;
    const int64_t w = pos - blk * block_size;
    const int64_t dst = ((blk * n_kv + hd) * block_size + w) * D;
    const u32x4 x1 = *(const u32x4*)(k + src + 8 * c);
    const u32x4 x2 = *(const u32x4*)(k + src + HALF + 8 * c);
    const float2* csr = cs + pos * HALF + 8 * c;
    u32x4 y1, y2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 cs0 = csr[2 * e], cs1 = csr[2 * e + 1];
      const float a0 = bf16_to_f32(x1[e] & 0xffffu), a1 = bf16_to_f32(x1[e] >> 16);
      const float b0 = bf16_to_f32(x2[e] & 0xffffu), b1 = bf16_to_f32(x2[e] >> 16);
      y1[e] = pack_bf16x2(a0 * cs0.x - b0 * cs0.y, a1 * cs1.x - b1 * cs1.y);
      y2[e] = pack_bf16x2(b0 * cs0.x + a0 * cs0.y, b1 * cs1.x + a1 * cs1.y);
    }
    *(u32x4*)(kc + dst + 8 * c) = y1;
    *(u32x4*)(kc + dst + HALF + 8 * c) = y2;
    *(u32x4*)(vc + dst + 8 * c) = *(const u32x4*)(v + src + 8 * c);
    *(u32x4*)(vc + dst + HALF + 8 * c) = *(const u32x4*)(v + src + HALF + 8 * c);
  }
}

static int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

int launch_rope_fill(const uint16_t* k, const uint16_t* v, int64_t L, int32_t block_size,
                     int32_t n_kv_heads, int32_t head_dim, double rope_base, float* rope_cs,
                     uint16_t* k_cache, uint16_t* v_cache, hipStream_t stream) {
  const int half = head_dim / 2;
  float2* cs = reinterpret_cast<float2*>(rope_cs);
  hipLaunchKernelGGL(rope_table, dim3(grid_for(L * half, 256)), dim3(256), 0, stream, cs, L, half,
                     rope_base);
  const int64_t n = L * n_kv_heads * (half / 8);
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_fill<128>, dim3(grid_for(n, 256)), dim3(256), 0, stream, k, v, cs, L,
                       block_size, n_kv_heads, k_cache, v_cache);
  else
    hipLaunchKernelGGL(rope_fill<64>, dim3(grid_for(n, 256)), dim3(256), 0, stream, k, v, cs, L,
                       block_size, n_kv_heads, k_cache, v_cache);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
