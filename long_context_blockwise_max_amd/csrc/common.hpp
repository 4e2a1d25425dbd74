// Shared device-side definitions for the gfx950 kernels of the Pulsar hot path.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define PULSAR_LDS __attribute__((address_space(3)))

namespace pulsar {

constexpr int kWave = 64;

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// two floats -> packed bf16x2 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Rotary angle pair for position `pos` and frequency index i (of half = d/2):
// theta = pos * base^(-i/half) in float64, cos/sin in float64, rounded to float32.
// Llama-3.1 frequency scaling (the "llama3" rope type published with Llama 3.1:
// factor 8, low-frequency factor 1, high-frequency factor 4, original context
// 8192): frequencies whose wavelength 2 pi / f is under 8192 / 4 positions are
// kept, those over 8192 / 1 are divided by 8, and in between the two are blended
// linearly in 8192 / wavelength.
__device__ __forceinline__ double llama3_scale(double inv) {
  constexpr double kFactor = 8.0, kLow = 1.0, kHigh = 4.0, kOrig = 8192.0;
  const double wavelen = 6.283185307179586 / inv;
  if (wavelen < kOrig / kHigh) return inv;
  if (wavelen > kOrig / kLow) return inv / kFactor;
  const double smooth = (kOrig / wavelen - kLow) / (kHigh - kLow);
  return (1.0 - smooth) * inv / kFactor + smooth * inv;
}

// scaling: 0 none, 1 Llama-3.1
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int i, int half, double base,
                                             int scaling, float* c, float* s) {
  double inv = pow(base, -(double)i / (double)half);
  if (scaling == 1) inv = llama3_scale(inv);
  double th = (double)pos * inv;
  double sd, cd;
  sincos(th, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// The pair (a, b) turned by the angle with cosine c and sine s, one fused
// multiply-add per output.  Every rotation of a query or key goes through this
// function, so all of them round identically.
__device__ __forceinline__ void rope_pair(float a, float b, float c, float s, float& y1, float& y2) {
  y1 = fmaf(a, c, -(b * s));
  y2 = fmaf(b, c, a * s);
}

// The value of a lane in the other half of the wave (lane ^ 32), via
// v_permlane32_swap: lanes 0-31 receive it in the second result, lanes 32-63
// in the first.
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

}  // namespace pulsar
