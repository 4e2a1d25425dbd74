// Flash-style attention kernels for Phase 1 (context encoding) and Phase 2
// (query attention over retained shards) on gfx950.
//
// Both phases run one MFMA tile routine.  A workgroup is 4 waves (one per
// SIMD).  All 4 waves share each 64-key K/V tile staged in LDS; each wave owns
// NQ x 32 query rows and keeps, per row, a running max, a running sum and an
// fp32 output accumulator (online softmax, Milakov & Gimelshein, as named in
// the Star Attention review).
//
// The contraction is done transposed so that every lane keeps one query row
// throughout:
//   S^T (keys x queries)    = K  . Q^T   v_mfma_f32_32x32x16_bf16, A = K rows
//                                         from LDS, B = Q^T held in registers
//   O^T (d x queries)      += V^T . P^T  A = V^T read from the row-major V tile
//                                         with ds_read_b64_tr_b16, B = P^T
// In the 32x32 accumulator layout, lane l holds column l % 32 (its query) and
// 16 rows; the K rows are loaded in a permuted order (bits 2 and 3 of the row
// index swapped) so that the 8 accumulator registers a lane hands to each PV
// step are 8 consecutive keys, which is exactly what one transposed V read
// pair delivers.  Row max and row sum need one exchange with lane l ^ 32
// (v_permlane32_swap); the rescale of O touches only the lane's own registers.
//
// Softmax runs in base 2: t = (q.k) * log2(e) / sqrt(d), p = exp2(t - m).  P is
// rounded to bf16 for the PV MFMA; the running sum uses the fp32 p.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

constexpr int KT = 64;     // keys per LDS tile
constexpr int PADE = 8;    // bf16 elements of padding per LDS row
constexpr int NTHR = 256;  // 4 waves per workgroup

template <int D>
struct TileShape {
  static constexpr int LD = D + PADE;       // LDS row stride (elements)
  static constexpr int CPR = D / 8;         // 16-byte chunks per row
  static constexpr int RPP = NTHR / CPR;    // rows per load pass
  static constexpr int PASSES = KT / RPP;   // load passes per tile
};

// S^T row m holds key perm(m): bits 2 and 3 of m swapped.
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// key (within the 64-key tile) held by accumulator register r of key subtile kt
__device__ __forceinline__ int reg_key(int kt, int r, int half) {
  return kt * 32 + 16 * (r >> 3) + 8 * half + (r & 7);
}

template <int D, int NQ>
struct FlashState {
  f32x16 o[D / 32][NQ];
  float m[NQ];
  float l[NQ];
};

template <int D, int NQ>
__device__ __forceinline__ void flash_init(FlashState<D, NQ>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[dt][qt][r] = 0.f;
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    st.m[qt] = -1e30f;  // finite, so a fully masked tile leaves the state unchanged
    st.l[qt] = 0.f;
  }
}

// One 64-key tile.  `valid(key, qt)` says whether tile key `key` is visible to
// this lane's query row of subtile qt; it is consulted only when `masked`.
template <int D, int NQ, class Valid>
__device__ __forceinline__ void flash_tile(const uint16_t* Ks, const uint16_t* Vs,
                                           const bf16x8 (&q)[NQ][D / 16], FlashState<D, NQ>& st,
                                           float scale_log2, bool masked, Valid valid) {
  constexpr int LD = TileShape<D>::LD;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int lr = lane & 31;

  f32x16 s[2][NQ];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][qt][r] = 0.f;

#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const uint16_t* krow = Ks + (kt * 32 + key_perm(lr)) * LD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 a = *(const bf16x8*)(krow + 16 * ks);
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt)
        s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[qt][ks], s[kt][qt], 0, 0, 0);
    }
  }

  bf16x8 p[NQ][2][2];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    if (masked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!valid(reg_key(kt, r, half), qt)) s[kt][qt][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(st.m[qt], mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(st.m[qt] - m_new);
    st.m[qt] = m_new;
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][r], scale_log2, -m_new));
        s[kt][qt][r] = e;
        sum += e;
      }
    st.l[qt] = st.l[qt] * alpha + sum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[dt][qt][r] *= alpha;
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack_bf16x2(s[kt][qt][8 * hh + 2 * e], s[kt][qt][8 * hh + 2 * e + 1]);
        p[qt][kt][hh] = __builtin_bit_cast(bf16x8, w);
      }
  }

  const int q4 = lane >> 4;
  const int li = lane & 15;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int d0 = dt * 32 + 16 * (q4 & 1);
        const int key0 = kt * 32 + 16 * hh + 8 * (q4 >> 1);
        const uint16_t* src = Vs + (key0 + (li >> 2)) * LD + d0 + 4 * (li & 3);
        const i16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((PULSAR_LDS i16x4*)(src));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((PULSAR_LDS i16x4*)(src + 4 * LD));
        u32x4 w;
        w[0] = (uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
        w[1] = (uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
        w[2] = (uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
        w[3] = (uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
        const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt)
          st.o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[qt][kt][hh], st.o[dt][qt], 0, 0, 0);
      }
  }
}

// Rotate a query row held as B fragments (lane holds d = 16 ks + 8 half + e) in
// place.  cs(i) returns (cos, sin) for frequency index i.
template <int D, class CosSin>
__device__ __forceinline__ void rotate_q(bf16x8 (&qf)[D / 16], CosSin cs) {
  const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    u32x4 a = __builtin_bit_cast(u32x4, qf[ks]);
    u32x4 b = __builtin_bit_cast(u32x4, qf[ks + D / 32]);
    u32x4 ya, yb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i0 = 16 * ks + 8 * half + 2 * e;
      const float2 c0 = cs(i0), c1 = cs(i0 + 1);
      const float a0 = bf16_to_f32(a[e] & 0xffffu), a1 = bf16_to_f32(a[e] >> 16);
      const float b0 = bf16_to_f32(b[e] & 0xffffu), b1 = bf16_to_f32(b[e] >> 16);
      ya[e] = pack_bf16x2(a0 * c0.x - b0 * c0.y, a1 * c1.x - b1 * c1.y);
      yb[e] = pack_bf16x2(b0 * c0.x + a0 * c0.y, b1 * c1.x + a1 * c1.y);
    }
    qf[ks] = __builtin_bit_cast(bf16x8, ya);
    qf[ks + D / 32] = __builtin_bit_cast(bf16x8, yb);
  }
}

// Cooperative tile staging: thread t owns 16-byte chunk t % CPR of rows
// t / CPR + p * RPP.  off[p] < 0 marks a row past the key list: it is zero-filled.
template <int D>
__device__ __forceinline__ void load_tile(const uint16_t* kbase, const uint16_t* vbase,
                                          const int64_t (&off)[TileShape<D>::PASSES],
                                          u32x4 (&kr)[TileShape<D>::PASSES],
                                          u32x4 (&vr)[TileShape<D>::PASSES]) {
  const int c = threadIdx.x % TileShape<D>::CPR;
#pragma unroll
  for (int p = 0; p < TileShape<D>::PASSES; ++p) {
    if (off[p] >= 0) {
      kr[p] = *(const u32x4*)(kbase + off[p] + 8 * c);
      vr[p] = *(const u32x4*)(vbase + off[p] + 8 * c);
    } else {
      kr[p] = u32x4{0u, 0u, 0u, 0u};
      vr[p] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(uint16_t* Ks, uint16_t* Vs,
                                           const u32x4 (&kr)[TileShape<D>::PASSES],
                                           const u32x4 (&vr)[TileShape<D>::PASSES]) {
  constexpr int CPR = TileShape<D>::CPR, RPP = TileShape<D>::RPP, LD = TileShape<D>::LD;
  const int c = threadIdx.x % CPR;
  const int r0 = threadIdx.x / CPR;
#pragma unroll
  for (int p = 0; p < TileShape<D>::PASSES; ++p) {
    *(u32x4*)(Ks + (r0 + p * RPP) * LD + 8 * c) = kr[p];
    *(u32x4*)(Vs + (r0 + p * RPP) * LD + 8 * c) = vr[p];
  }
}

// Write O / l (and, for Phase 2, the log-sum-exp) of one query subtile.
template <int D, int NQ>
__device__ __forceinline__ void flash_finish(const FlashState<D, NQ>& st, int qt, float* orow,
                                             float* lse_out) {
  const int half = (threadIdx.x & 63) >> 5;
  const float l_tot = st.l[qt] + swap_halves(st.l[qt]);
  if (orow) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = st.o[dt][qt][4 * rq + e] * inv;
        *(f32x4*)(orow + dt * 32 + 8 * rq + 4 * half) = v;
      }
    if (lse_out && half == 0)
      *lse_out = l_tot > 0.f ? (st.m[qt] + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

// ------------------------------------------------------------------ Phase 1
struct P1Args {
  const uint16_t* q;       // [L][Hq][D]
  const uint16_t* kc;      // [N][Hkv][b][D]
  const uint16_t* vc;
  const int32_t* sel;      // [N][kept]
  const float2* cs;        // [L][D/2]
  const int32_t* order;    // [N * n_rt] (block, row tile) pairs, longest first
  float* o;                // [L][Hq][D]
  int32_t n_blocks, b, chunk, kept, sink, hq, hkv, group, hpw, n_hs, n_rt, rpw;
  float scale_log2;
};

__device__ __forceinline__ int64_t p1_prefix_pos(const P1Args& a, int e) {
  if (e < a.sink) return e;
  const int e2 = e - a.sink;
  const int span = a.chunk * a.kept;
  const int j = e2 / span;
  const int rem = e2 - j * span;
  const int ci = rem / a.chunk;
  // chunk indices outside [0, n_chunks) are clamped so a bad `sel` cannot read out of bounds
  const int c = min(max(a.sel[j * a.kept + ci], 0), a.b / a.chunk - 1);
  return (int64_t)j * a.b + (int64_t)c * a.chunk + (rem - ci * a.chunk);
}

template <int D>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
phase1_kernel(P1Args a) {
  constexpr int NQ = 2;
  constexpr int LD = TileShape<D>::LD;
  constexpr int PASSES = TileShape<D>::PASSES;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * LD];

  const int hc_count = a.hkv * a.n_hs;
  const int pair = a.order[blockIdx.x / hc_count];
  const int hc = blockIdx.x % hc_count;
  const int g = hc % a.hkv;
  const int hs = hc / a.hkv;
  const int i = pair / a.n_rt;
  const int rt = pair % a.n_rt;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int lr = lane & 31;
  const int h = g * a.group + hs * a.hpw + (wave % a.hpw);
  const int r0 = rt * a.rpw + (wave / a.hpw) * 64;   // first own row of this wave

  const int P = (i == 0) ? 0 : a.sink + a.chunk * a.kept * i;
  const int n_pre = (P + KT - 1) / KT;
  const int own_end = min((rt + 1) * a.rpw, a.b);
  const int n_own = (own_end + KT - 1) / KT;
  const int T = n_pre + n_own;

  // query fragments, rotated at their original positions
  bf16x8 qf[NQ][D / 16];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = r0 + qt * 32 + lr;
    const int64_t pos = (int64_t)i * a.b + r;
    if (r < a.b) {
      const uint16_t* qrow = a.q + (pos * a.hq + h) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[qt][ks] = *(const bf16x8*)(qrow + 16 * ks);
      const float2* csr = a.cs + pos * (D / 2);
      rotate_q<D>(qf[qt], [&](int f) { return csr[f]; });
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[qt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  FlashState<D, NQ> st;
  flash_init(st);

  const int crow0 = threadIdx.x / TileShape<D>::CPR;
  auto row_offsets = [&](int t, int64_t (&off)[PASSES]) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = crow0 + p * TileShape<D>::RPP;
      int64_t pos = -1;
      if (t < n_pre) {
        const int e = t * KT + row;
        if (e < P) pos = p1_prefix_pos(a, e);
      } else {
        const int kk = (t - n_pre) * KT + row;
        if (kk < own_end) pos = (int64_t)i * a.b + kk;
      }
      if (pos >= 0) {
        const int64_t blk = pos / a.b;
        off[p] = ((blk * a.hkv + g) * a.b + (pos - blk * a.b)) * D;
      } else {
        off[p] = -1;
      }
    }
  };

  u32x4 kr[PASSES], vr[PASSES];
  int64_t off[PASSES];
  row_offsets(0, off);
  load_tile<D>(a.kc, a.vc, off, kr, vr);
  const float sl2 = a.scale_log2;
  for (int t = 0; t < T; ++t) {
    __syncthreads();
    store_tile<D>(Ks, Vs, kr, vr);
    if (t + 1 < T) {
      row_offsets(t + 1, off);
      load_tile<D>(a.kc, a.vc, off, kr, vr);
    }
    __syncthreads();
    if (t < n_pre) {
      const int e0 = t * KT;
      const bool masked = e0 + KT > P;
      flash_tile<D, NQ>(Ks, Vs, qf, st, sl2, masked,
                        [&](int key, int) { return e0 + key < P; });
    } else {
      const int k0 = (t - n_pre) * KT;
      if (k0 > r0 + 63) continue;  // the whole tile lies above this wave's diagonal
      const bool masked = (k0 + KT - 1 > r0) || (k0 + KT > own_end);
      flash_tile<D, NQ>(Ks, Vs, qf, st, sl2, masked, [&](int key, int qt) {
        const int kk = k0 + key;
        return kk <= r0 + qt * 32 + lr && kk < own_end;
      });
    }
  }

#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = r0 + qt * 32 + lr;
    float* orow = nullptr;
    if (r < a.b) orow = a.o + (((int64_t)i * a.b + r) * a.hq + h) * D;
    flash_finish<D, NQ>(st, qt, orow, nullptr);
  }
}

// Work order: (block, row tile) pairs by descending number of key tiles, ties by
// pair id.  One thread per pair computes its rank directly: the tile count of
// (i, rt) is pre(i) + own(rt) with both parts non-decreasing, so the number of
// pairs of block i' above a given count has a closed form.
__device__ __forceinline__ int p1_pre_tiles(int i, int sink, int chunk, int kept) {
  const int P = (i == 0) ? 0 : sink + chunk * kept * i;
  return (P + KT - 1) / KT;
}
__device__ __forceinline__ int p1_own_tiles(int rt, int rpw, int b) {
  return (min((rt + 1) * rpw, b) + KT - 1) / KT;
}
// number of row tiles rt' with own(rt') <= x
__device__ __forceinline__ int p1_count_le(int x, int rpw, int b, int n_rt) {
  if (x < 0) return 0;
  int lo = 0, hi = n_rt;  // own() is non-decreasing: binary search the first rt with own > x
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p1_own_tiles(mid, rpw, b) <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(256) phase1_order(int32_t n_blocks, int32_t b, int32_t chunk,
                                                    int32_t kept, int32_t sink, int32_t rpw,
                                                    int32_t n_rt, int32_t* __restrict__ order) {
  const int n_pairs = n_blocks * n_rt;
  for (int pid = blockIdx.x * blockDim.x + threadIdx.x; pid < n_pairs;
       pid += gridDim.x * blockDim.x) {
    const int i = pid / n_rt, rt = pid % n_rt;
    const int v = p1_pre_tiles(i, sink, chunk, kept) + p1_own_tiles(rt, rpw, b);
    int rank = 0;
    for (int i2 = 0; i2 < n_blocks; ++i2) {
      const int pre = p1_pre_tiles(i2, sink, chunk, kept);
      const int above = n_rt - p1_count_le(v - pre, rpw, b, n_rt);       // own > v - pre
      rank += above;
      const int eq_all = p1_count_le(v - pre, rpw, b, n_rt) - p1_count_le(v - pre - 1, rpw, b, n_rt);
      if (i2 < i) {
        rank += eq_all;
      } else if (i2 == i) {
        // ties within block i with a smaller row tile index
        rank += min(rt, p1_count_le(v - pre, rpw, b, n_rt)) -
                min(rt, p1_count_le(v - pre - 1, rpw, b, n_rt));
      }
    }
    order[rank] = pid;
  }
}

Phase1Geometry phase1_geometry(int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                               int32_t kept, int32_t sink_size, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim) {
  Phase1Geometry g{};
  g.n_blocks = n_blocks;
  g.block_size = block_size;
  g.chunk_size = chunk_size;
  g.kept = kept;
  g.sink_size = sink_size;
  g.n_q_heads = n_q_heads;
  g.n_kv_heads = n_kv_heads;
  g.head_dim = head_dim;
  const int group = n_q_heads / n_kv_heads;
  g.heads_per_wg = group >= 4 ? 4 : group;           // waves per workgroup split as heads x row groups
  g.n_head_sub = group / g.heads_per_wg;
  g.rows_per_wg = 64 * (4 / g.heads_per_wg);
  g.n_row_tiles = (block_size + g.rows_per_wg - 1) / g.rows_per_wg;
  return g;
}

int launch_phase1(const Phase1Geometry& g, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* sel, const float* rope_cs,
                  int32_t* order, float* o, hipStream_t stream) {
  const int n_pairs = g.n_blocks * g.n_row_tiles;
  hipLaunchKernelGGL(phase1_order, dim3((n_pairs + 255) / 256), dim3(256), 0, stream, g.n_blocks,
                     g.block_size, g.chunk_size, g.kept, g.sink_size, g.rows_per_wg,
                     g.n_row_tiles, order);
  P1Args a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.sel = sel;
  a.cs = reinterpret_cast<const float2*>(rope_cs);
  a.order = order;
  a.o = o;
  a.n_blocks = g.n_blocks;
  a.b = g.block_size;
  a.chunk = g.chunk_size;
  a.kept = g.kept;
  a.sink = g.sink_size;
  a.hq = g.n_q_heads;
  a.hkv = g.n_kv_heads;
  a.group = g.n_q_heads / g.n_kv_heads;
  a.hpw = g.heads_per_wg;
  a.n_hs = g.n_head_sub;
  a.n_rt = g.n_row_tiles;
  a.rpw = g.rows_per_wg;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.head_dim));
  const int grid = n_pairs * g.n_kv_heads * g.n_head_sub;
  if (g.head_dim == 128)
    hipLaunchKernelGGL(phase1_kernel<128>, dim3(grid), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL(phase1_kernel<64>, dim3(grid), dim3(NTHR), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ------------------------------------------------------------------ Phase 2
struct P2Args {
  const uint16_t* qq;   // [B][Lq][Hq][D]
  const uint16_t* kc;   // [B][S][Hkv][n][D]
  const uint16_t* vc;
  const uint16_t* ks;   // [B][Lq][Hkv][D] or null
  const uint16_t* vs;
  float* o_part;        // [B][n_parts][Lq][Hq][D]
  float* lse_part;      // [B][n_parts][Lq][Hq]
  int64_t q_pos0;
  double base;
  int32_t batch, n_shards, n, lq, hq, hkv, group, splits, n_parts, n_rg;
  float scale_log2;
};

template <int D, int NQ>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
phase2_kernel(P2Args a) {
  constexpr int LD = TileShape<D>::LD;
  constexpr int PASSES = TileShape<D>::PASSES;
  constexpr int CPR = TileShape<D>::CPR;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * LD];

  int w = blockIdx.x;
  const int p = w % a.n_parts;
  w /= a.n_parts;
  const int rg = w % a.n_rg;
  w /= a.n_rg;
  const int g = w % a.hkv;
  const int bb = w / a.hkv;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31;
  const int n_rows = a.group * a.lq;
  const int row_base = rg * (4 * NQ * 32) + wave * (NQ * 32);

  const bool self_part = p >= a.n_shards * a.splits;
  int shard = 0, k0 = 0, k1 = 0;
  if (!self_part) {
    shard = p / a.splits;
    const int sp = p % a.splits;
    const int nt = (a.n + KT - 1) / KT;
    k0 = (int)(((int64_t)sp * nt) / a.splits) * KT;
    k1 = min((int)(((int64_t)(sp + 1) * nt) / a.splits) * KT, a.n);
  } else {
    k0 = 0;
    k1 = a.lq;
  }
  const int T = (k1 - k0 + KT - 1) / KT;

  // query fragments: row fr = head-in-group * Lq + token
  bf16x8 qf[NQ][D / 16];
  bool wave_active = row_base < n_rows;
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int fr = row_base + qt * 32 + lr;
    if (fr < n_rows) {
      const int hh = fr / a.lq, t = fr % a.lq;
      const int h = g * a.group + hh;
      const uint16_t* qrow = a.qq + (((int64_t)bb * a.lq + t) * a.hq + h) * D + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[qt][ks] = *(const bf16x8*)(qrow + 16 * ks);
      const int64_t pos = a.q_pos0 + t;
      const double base = a.base;
      rotate_q<D>(qf[qt], [&](int f) {
        float c, s;
        rope_cos_sin(pos, f, D / 2, base, &c, &s);
        return make_float2(c, s);
      });
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        qf[qt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  FlashState<D, NQ> st;
  flash_init(st);

  const int c = threadIdx.x % CPR;
  const int crow0 = threadIdx.x / CPR;
  const uint16_t* kbase = a.kc + ((((int64_t)bb * a.n_shards + shard) * a.hkv + g) * a.n) * D;
  const uint16_t* vbase = a.vc + ((((int64_t)bb * a.n_shards + shard) * a.hkv + g) * a.n) * D;
  u32x4 kr[PASSES], vr[PASSES];
  auto fetch = [&](int t) {
    if (!self_part) {
      int64_t off[PASSES];
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        const int kk = k0 + t * KT + crow0 + pp * TileShape<D>::RPP;
        off[pp] = kk < k1 ? (int64_t)kk * D : -1;
      }
      load_tile<D>(kbase, vbase, off, kr, vr);
    } else {
      // self keys are pre-RoPE: rotate while staging (partner chunk is +-D/16 chunks away)
#pragma unroll
      for (int pp = 0; pp < PASSES; ++pp) {
        const int kk = t * KT + crow0 + pp * TileShape<D>::RPP;
        if (kk < a.lq) {
          const int64_t roff = (((int64_t)bb * a.lq + kk) * a.hkv + g) * D;
          const bool first = c < CPR / 2;
          const int cp = first ? c + CPR / 2 : c - CPR / 2;
          const u32x4 x = *(const u32x4*)(a.ks + roff + 8 * c);
          const u32x4 y = *(const u32x4*)(a.ks + roff + 8 * cp);
          const int64_t pos = a.q_pos0 + kk;
          u32x4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int f0 = 8 * (first ? c : cp) + 2 * e;
            float c0, s0, c1, s1;
            rope_cos_sin(pos, f0, D / 2, a.base, &c0, &s0);
            rope_cos_sin(pos, f0 + 1, D / 2, a.base, &c1, &s1);
            const float x0 = bf16_to_f32(x[e] & 0xffffu), x1 = bf16_to_f32(x[e] >> 16);
            const float y0 = bf16_to_f32(y[e] & 0xffffu), y1 = bf16_to_f32(y[e] >> 16);
            // first half: x*cos - partner*sin; second half: x*cos + partner*sin
            const float sg = first ? -1.f : 1.f;
            out[e] = pack_bf16x2(x0 * c0 + sg * y0 * s0, x1 * c1 + sg * y1 * s1);
          }
          kr[pp] = out;
          vr[pp] = *(const u32x4*)(a.vs + roff + 8 * c);
        } else {
          kr[pp] = u32x4{0u, 0u, 0u, 0u};
          vr[pp] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  fetch(0);
  const float sl2 = a.scale_log2;
  for (int t = 0; t < T; ++t) {
    __syncthreads();
    store_tile<D>(Ks, Vs, kr, vr);
    if (t + 1 < T) fetch(t + 1);
    __syncthreads();
    if (!wave_active) continue;
    const int kb = k0 + t * KT;
    if (!self_part) {
      const bool masked = kb + KT > k1;
      flash_tile<D, NQ>(Ks, Vs, qf, st, sl2, masked, [&](int key, int) { return kb + key < k1; });
    } else {
      flash_tile<D, NQ>(Ks, Vs, qf, st, sl2, true, [&](int key, int qt) {
        const int fr = row_base + qt * 32 + lr;
        const int tok = fr % a.lq;
        const int kk = kb + key;
        return kk <= tok && kk < a.lq;
      });
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int fr = row_base + qt * 32 + lr;
    float* orow = nullptr;
    float* lrow = nullptr;
    if (fr < n_rows) {
      const int hh = fr / a.lq, t = fr % a.lq;
      const int h = g * a.group + hh;
      const int64_t rix = (((int64_t)bb * a.n_parts + p) * a.lq + t) * a.hq + h;
      orow = a.o_part + rix * D;
      lrow = a.lse_part + rix;
    }
    flash_finish<D, NQ>(st, qt, orow, lrow);
  }
}

Phase2Geometry phase2_geometry(int32_t batch, int32_t n_shards, int32_t shard_len,
                               int32_t q_len, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t has_self) {
  Phase2Geometry g{};
  g.batch = batch;
  g.n_shards = n_shards;
  g.shard_len = shard_len;
  g.q_len = q_len;
  g.n_q_heads = n_q_heads;
  g.n_kv_heads = n_kv_heads;
  g.head_dim = head_dim;
  g.has_self = has_self ? 1 : 0;
  const int rows = (n_q_heads / n_kv_heads) * q_len;
  g.nq = rows > 128 ? 2 : 1;
  const int rows_per_wg = 4 * g.nq * 32;
  g.n_row_groups = (rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t combos = (int64_t)batch * n_kv_heads * n_shards * g.n_row_groups;
  const int64_t target = g.nq == 2 ? 256 : 512;   // workgroups to fill 256 CUs
  int64_t splits = (target + combos - 1) / combos;
  const int64_t nt = (shard_len + KT - 1) / KT;
  if (splits > nt) splits = nt;
  if (splits < 1) splits = 1;
  g.splits = (int32_t)splits;
  g.n_parts = n_shards * g.splits + g.has_self;
  return g;
}

int launch_phase2(const Phase2Geometry& g, const uint16_t* qq, int64_t q_pos0,
                  const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_self,
                  const uint16_t* v_self, double rope_base, float* o_part, float* lse_part,
                  hipStream_t stream) {
  P2Args a;
  a.qq = qq;
  a.kc = k_cache;
  a.vc = v_cache;
  a.ks = k_self;
  a.vs = v_self;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.q_pos0 = q_pos0;
  a.base = rope_base;
  a.batch = g.batch;
  a.n_shards = g.n_shards;
  a.n = g.shard_len;
  a.lq = g.q_len;
  a.hq = g.n_q_heads;
  a.hkv = g.n_kv_heads;
  a.group = g.n_q_heads / g.n_kv_heads;
  a.splits = g.splits;
  a.n_parts = g.n_parts;
  a.n_rg = g.n_row_groups;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.head_dim));
  const int64_t grid = (int64_t)g.batch * g.n_kv_heads * g.n_row_groups * g.n_parts;
  if (g.head_dim == 128) {
    if (g.nq == 2)
      hipLaunchKernelGGL((phase2_kernel<128, 2>), dim3(grid), dim3(NTHR), 0, stream, a);
    else
      hipLaunchKernelGGL((phase2_kernel<128, 1>), dim3(grid), dim3(NTHR), 0, stream, a);
  } else {
    if (g.nq == 2)
      hipLaunchKernelGGL((phase2_kernel<64, 2>), dim3(grid), dim3(NTHR), 0, stream, a);
    else
      hipLaunchKernelGGL((phase2_kernel<64, 1>), dim3(grid), dim3(NTHR), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
