// Flash-style attention kernels for Phase 1 (context encoding) and Phase 2
// (query attention over retained shards) on gfx950.
//
// Both phases run one MFMA tile routine.  A workgroup is 8 waves, two per SIMD
// (Phase 1: 12 waves, three per SIMD, where the GQA group divides them), so
// that one wave's softmax (VALU) can overlap another wave's matrix work.  All
// waves share each KT-key K / V tile staged in LDS; each wave owns 32 query rows
// and keeps, per row, a running reference maximum, a running sum and an fp32
// output accumulator (online softmax, Milakov & Gimelshein, as the Star
// Attention review names it).
//
// The contraction is done transposed so that every lane keeps one query row:
//   S^T (keys x queries)  = K   . Q^T   v_mfma_f32_32x32x16_bf16: A = K rows from
//                                       LDS, B = Q^T held in registers (or, with
//                                       12 waves, read from LDS)
//   O^T (d x queries)    += V^T . P^T   A = rows of the d-major V tile, B = P^T
// In the 32x32 accumulator layout lane l holds column l % 32 (its query) and
// 16 rows.  The K rows are fed in a permuted order (bits 2 and 3 of the row
// index swapped) so that the 8 accumulator registers a lane hands to a PV step
// are 8 consecutive keys -- one 16-byte chunk of a d-major V row.  The row max
// and row sum need one exchange with lane l ^ 32 (v_permlane32_swap); the
// rescale of O touches only the lane's own registers.
//
// Tiles are staged with direct global->LDS loads (buffer_load_dwordx4 ... lds in
// Phase 1 and for Phase-2 shard tiles, global_load_lds_dwordx4 for the Phase-2
// self tiles), one barrier per tile: two slots,
// one tile ahead, for Phase 1 and the Phase-2 query; four slots, three tiles
// ahead, for the Phase-2 decode form, which streams from HBM with little work
// per tile.  The 16-byte chunks of every LDS row are XOR-swizzled so that
// fragment reads are bank-conflict free.
//
// Softmax runs in base 2: t = (q.k) * log2(e) / sqrt(d), p = exp2(t - m), with
// the reference maximum m raised lazily (see kRescaleSlack).  P is rounded to
// bf16 for the PV MFMA; the running sum uses the fp32 p.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace pulsar {

constexpr int KT = 64;            // keys per LDS tile (one barrier per tile)
constexpr int NSUB = KT / 32;     // 32-key subtiles per tile
constexpr int NW = 8;             // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int P1_WQ = 12;         // Phase-1 waves per workgroup when the GQA group allows (query rows in LDS)

// K tile: KT key rows x D (row = 2D bytes)
template <int D>
struct KTile {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int ROWB = 2 * D;
  static constexpr int BYTES = KT * ROWB;
  static constexpr int RPI = 1024 / ROWB;     // rows one 64-lane DMA fills
  static constexpr int NI = KT / RPI / NW;    // DMAs per wave per tile
  __device__ static __forceinline__ int sw(int r) {
    return D == 128 ? ((4 * (r & 3)) ^ ((r >> 2) & 3)) : ((r >> 1) & 7);
  }
  // byte offset of elements [e, e + 8) of row r (e a multiple of 8)
  __device__ static __forceinline__ int off(int r, int e) {
    return r * ROWB + (((e >> 3) ^ sw(r)) << 4);
  }
};

// V tile, d-major: D rows (one per d) x KT keys (a row holds KT / 8 chunks of 8 keys)
template <int D>
struct VTile {
  static constexpr int CPR = KT / 8;
  static constexpr int ROWB = 2 * KT;
  static constexpr int BYTES = D * ROWB;
  static constexpr int RPI = 1024 / ROWB;     // d-rows per DMA
  static constexpr int NI = D / RPI / NW;
  __device__ static __forceinline__ int sw(int r) {
    return CPR == 16 ? ((4 * (r & 3)) ^ ((r >> 2) & 3)) : ((r >> 1) & 7);
  }
  // byte offset of key chunk c (keys 8c .. 8c+7) of d-row r
  __device__ static __forceinline__ int off(int r, int c) { return r * ROWB + ((c ^ sw(r)) << 4); }
};

template <int D>
struct Stage {
  static constexpr int BYTES = KTile<D>::BYTES + VTile<D>::BYTES;
};

// S^T row m holds key perm(m): bits 2 and 3 of m swapped.
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// key (within a 32-key subtile) held by accumulator register r
__device__ __forceinline__ int reg_key(int r, int half) {
  return 16 * (r >> 3) + 8 * half + (r & 7);
}

template <int D, int NQ>
struct FlashState {
  f32x16 o[D / 32][NQ];
  float m[NQ];   // reference maximum (log2 units), raised lazily
  float l[NQ];   // this lane's partial row sum (the other half-wave holds the rest)
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
    st.m[qt] = -1e30f;  // finite, so fully masked keys never produce inf - inf
    st.l[qt] = 0.f;
  }
}

// The reference maximum m only moves when a score exceeds it by more than the
// slack (log2 units); until then p = exp2(t - m) <= 2^8, which fp32 sums and
// bf16 P hold without loss, and O / l at the end is the same ratio either way.
constexpr float kRescaleSlack = 8.f;
constexpr float kRescaleBound = 256.f;   // 2^kRescaleSlack

// p = exp2(s * sl2 - m) for the 16 scores of one accumulator, rounded to bf16
// into the two PV operands; sum = the fp32 sum of the p.  (Summing the rounded
// pairs with v_dot2_f32_bf16, eight instructions instead of sixteen adds, gives
// correct sums but a 3 % slower loop: the dot products into one accumulator
// form a longer dependent chain.)
template <int NQ>
__device__ __forceinline__ void softmax_p(const f32x16& s, float sl2, float m, bf16x8 (&p)[2],
                                          float& sum) {
  const float neg_m = -m;
  float acc = 0.f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[8 * hh + 2 * e], sl2, neg_m));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[8 * hh + 2 * e + 1], sl2, neg_m));
      w[e] = pack_bf16x2(e0, e1);
      acc += e0 + e1;
    }
    p[hh] = __builtin_bit_cast(bf16x8, w);
  }
  sum = acc;
}

// One 32-key subtile `kt` (0 .. NSUB-1) of a staged tile, in three steps (the
// Phase-1 loop issues the next tile's loads between them):
//   sub_qk       s = K . Q^T for the query tile's 32 rows
//   sub_softmax  mask, p = exp2(s * sl2 - m) rounded to bf16, running sum and max
//   sub_pv       O^T += V^T . P^T
template <int D>
__device__ __forceinline__ void sub_qk(const char* stage, int kt, const bf16x8 (&q)[D / 16],
                                       f32x16& s) {
  using KTl = KTile<D>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int krow = kt * 32 + key_perm(lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = *(const bf16x8*)(stage + KTl::off(krow, 16 * ks + 8 * half));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[ks], s, 0, 0, 0);
  }
}

// sub_qk with the query rows staged in LDS (laid out like K tile rows); the
// first QR fragments come from registers.
template <int D, int QR>
__device__ __forceinline__ void sub_qk_lds(const char* stage, int kt, const char* qlds,
                                           const bf16x8 (&q)[D / 16], f32x16& s) {
  using KTl = KTile<D>;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int krow = kt * 32 + key_perm(lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = *(const bf16x8*)(stage + KTl::off(krow, 16 * ks + 8 * half));
    const bf16x8 b = ks < QR ? q[ks] : *(const bf16x8*)(qlds + KTl::off(lane & 31, 16 * ks + 8 * half));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, s, 0, 0, 0);
  }
}

// Keys 0 .. lim-1 of the subtile are visible to this lane's query row (lim >= 32:
// all of them); the mask is applied only when some lane of the wave needs it.
// Fast path: p against the current reference maximum m, no max reduction.  Every
// p stays <= 2^kRescaleSlack unless a score rose more than the slack above m,
// and then this lane's subtile sum exceeds 2^kRescaleSlack too (or is inf /
// nan), which sends the wave to the slow path: exact maximum, rescale of O and
// l, p recomputed.  The first subtile always takes it (m starts at -1e30).
template <int D>
__device__ __forceinline__ void sub_softmax(f32x16& s, FlashState<D, 1>& st, float sl2, int lim,
                                            bf16x8 (&p)[2]) {
  const int half = (threadIdx.x & 63) >> 5;
  if (__builtin_expect(__ballot(lim < 32) != 0, 0)) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (reg_key(r, half) >= lim) s[r] = -INFINITY;
  }
  float sum;
  softmax_p<1>(s, sl2, st.m[0], p, sum);
  if (__builtin_expect(__ballot(!(sum <= kRescaleBound)) != 0, 0)) {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(st.m[0], mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(st.m[0] - m_new);
    st.m[0] = m_new;
    st.l[0] *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[dt][0][r] *= alpha;
    softmax_p<1>(s, sl2, st.m[0], p, sum);
  }
  st.l[0] += sum;
}

template <int D>
__device__ __forceinline__ void sub_pv(const char* stage, int kt, const bf16x8 (&p)[2],
                                       FlashState<D, 1>& st) {
  using VTl = VTile<D>;
  const char* Vt = stage + KTile<D>::BYTES;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int lr = lane & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const bf16x8 a = *(const bf16x8*)(Vt + VTl::off(dt * 32 + lr, kt * 4 + 2 * hh + half));
      st.o[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[hh], st.o[dt][0], 0, 0, 0);
    }
  }
}

// Raw byte-addressed buffer resource over `bytes` bytes at `base`: loads at
// offsets past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16 bytes per lane at base + soff + voff into LDS (buffer_load_dwordx4 ... lds).
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                          char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PULSAR_LDS void*)lds, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void dma16(const uint16_t* src, char* lds) {
  __builtin_amdgcn_global_load_lds((const void*)src, (PULSAR_LDS void*)lds, 16, 0, 0);
}

// Wait until this wave's direct-to-LDS loads have landed, then barrier: after it
// the staged tile is visible to every wave.  The compiler does not count these
// loads as outstanding at a barrier, so the vmcnt wait is explicit.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// gfx9 s_waitcnt immediate: vmcnt = n, lgkmcnt = 0, expcnt not waited on.
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

// Barrier after which every load this wave issued before its newest N vector
// memory loads has landed, and this wave's LDS reads are done.  The wait is the
// builtin, so the compiler's own wait bookkeeping knows about it; the s_barrier
// carries no fence (the fence of __syncthreads() waits for every outstanding
// load, tiles still in flight included); the empty asm statements keep the
// compiler from moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void tile_barrier_n() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(N));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Stage one K tile and one d-major V tile into LDS with direct global->LDS
// 16-byte loads.  DMA number `blk` of a tile fills 1 KB of consecutive LDS rows;
// lane j fetches the chunk that the swizzle puts at position j, so the layout
// falls out of the source addresses alone.  Each lane stages NI key rows and NI
// value chunks per tile; which ones is fixed by its lane and wave:
template <int D>
__device__ __forceinline__ int staged_k_row(int i) {   // key row (0..63) of K DMA i
  using KTl = KTile<D>;
  return ((threadIdx.x >> 6) * KTl::NI + i) * KTl::RPI + (threadIdx.x & 63) / KTl::CPR;
}
template <int D>
__device__ __forceinline__ int staged_v_d(int i) {     // d-row of V DMA i
  using VTl = VTile<D>;
  return ((threadIdx.x >> 6) * VTl::NI + i) * VTl::RPI + (threadIdx.x & 63) / VTl::CPR;
}
template <int D>
__device__ __forceinline__ int staged_v_chunk(int i) { // 8-key chunk (0..7) of V DMA i
  using VTl = VTile<D>;
  return ((threadIdx.x & 63) % VTl::CPR) ^ VTl::sw(staged_v_d<D>(i));
}

// Source element offsets of this lane's staged rows: k[i] of key row
// staged_k_row(i), v[i] of the first of the 8 keys of chunk staged_v_chunk(i)
// at d = 0 (the source's d-rows are v_ld elements apart).  Keys past the list
// must still point at readable memory; the caller masks them.
template <int D>
struct TileSrc {
  int64_t k[KTile<D>::NI];
  int64_t v[VTile<D>::NI];
};

template <int D>
__device__ __forceinline__ void stage_tile(char* stage, const uint16_t* kbase,
                                           const uint16_t* vbase, int64_t v_ld,
                                           const TileSrc<D>& src) {
  using KTl = KTile<D>;
  using VTl = VTile<D>;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < KTl::NI; ++i) {
    const int blk = wave * KTl::NI + i;
    const int row = staged_k_row<D>(i);
    const int c = (lane % KTl::CPR) ^ KTl::sw(row);
    dma16(kbase + src.k[i] + 8 * c, stage + blk * 1024);
  }
#pragma unroll
  for (int i = 0; i < VTl::NI; ++i) {
    const int blk = wave * VTl::NI + i;
    dma16(vbase + src.v[i] + (int64_t)staged_v_d<D>(i) * v_ld,
          stage + KTl::BYTES + blk * 1024);
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

// Query fragments of one 32-row subtile: lane holds row `row` (or zeros when
// row is null), elements 16 ks + 8 half .. +7, already rotated.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* row, bf16x8 (&qf)[D / 16]) {
  const int half = (threadIdx.x & 63) >> 5;
  if (row) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *(const bf16x8*)(row + 16 * ks + 8 * half);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
}

// ------------------------------------------------------------------ Phase 1
// Prefix index lists ("Dropping the Anchor ..." Section 2: block i > 0 prepends
// [sink || summary of block 0 || ... || summary of block i-1]; the Dutch
// technical summary writes the host input as [S_sink || Sigma_0 || ... ||
// Sigma_{i-1} || B_i]).  For prefix entry e of block i, at position pos in
// block blk = pos / b, column w = pos % b:
//   krow[e] = blk * Hkv * b + w        (K cache row, KV head 0; head g adds g * b)
//   vcol[e] = blk * Hkv * D * b + w    (d-major V cache column, head 0, d = 0;
//                                       head g adds g * D * b, d adds d * b)
// Block i's entries start at sum_{i' < i} P_i' = (i - 1) S + K (i - 1) i / 2
// for i >= 1, with P_i = S + K i and K = chunk * kept.
__host__ __device__ __forceinline__ int64_t p1_list_start(int i, int sink, int span) {
  return i == 0 ? 0 : (int64_t)(i - 1) * sink + (int64_t)span * (i - 1) * i / 2;
}

__global__ void __launch_bounds__(256) phase1_prefix_list(const int32_t* __restrict__ sel,
                                                          int32_t b, int32_t chunk, int32_t kept,
                                                          int32_t sink, int32_t hkv, int32_t d,
                                                          int32_t* __restrict__ krow,
                                                          int32_t* __restrict__ vcol) {
  const int i = blockIdx.y + 1;
  const int span = chunk * kept;
  const int P = sink + span * i;
  const int64_t start = p1_list_start(i, sink, span);
  const int n_chunks = b / chunk;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < P; e += gridDim.x * blockDim.x) {
    int blk, w;
    if (e < sink) {
      blk = e / b;
      w = e - blk * b;
    } else {
      const int e2 = e - sink;
      const int j = e2 / span;
      const int rem = e2 - j * span;
      const int ci = rem / chunk;
      // chunk indices outside [0, n_chunks) are clamped so a bad `sel` cannot read out of bounds
      const int c = min(max(sel[j * kept + ci], 0), n_chunks - 1);
      blk = j;
      w = c * chunk + (rem - ci * chunk);
    }
    krow[start + e] = blk * hkv * b + w;
    vcol[start + e] = blk * hkv * d * b + w;
  }
}

struct P1Args {
  const uint16_t* q;       // [L][Hq][D], rotated
  const uint16_t* kc;      // [N][Hkv][b][D]
  const uint16_t* vc;      // [N][Hkv][D][b]
  const int32_t* krow;     // prefix index lists
  const int32_t* vcol;
  const int32_t* order;    // [N * n_rt] (block, row tile) pairs, longest first
  float* o;                // [L][Hq][D] (prefix rows: [P][Hq][D])
  int32_t n_blocks, b, chunk, kept, sink, hq, hkv, group, hpw, n_hs, n_rt, rpw;
  float scale_log2;
};

// PR = false: the block rows of every block (the encode step).
// PR = true: the prefix rows.  The last block's prefix list
// [sink || summaries of blocks 0 .. N-2] is itself a sequence: its entry e is a
// query at its original position and attends to entries 0 .. e (every host's
// prefix is a leading part of this list, so one pass serves all hosts).  Tiles
// come through the list, the mask is causal in list order, row tiles run longest
// first, and a.n_rt counts the list's row tiles.

template <int D, bool PR, int NWV>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * NWV, 64 * NWV),
                               amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
phase1_kernel(P1Args a) {
  constexpr int NQ = 1;
  // With 12 waves (3 per SIMD) the registers no longer hold all of the query
  // rows: they sit in LDS behind the two slots (8 KB per wave at d = 128, 160 KB
  // in all), and only the first QRN fragments are also kept in registers: 6 of 8
  // fit the 168-register budget at d = 128 (its few spills fall outside the
  // loop), all 4 at d = 64.
  constexpr bool QL = NWV > NW;
  constexpr int QRN = D == 128 ? 6 : D / 16;
  constexpr int QBYTES = 32 * KTile<D>::ROWB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * Stage<D>::BYTES + (QL ? NWV * QBYTES : 0)];

  const int hc_count = a.hkv * a.n_hs;
  const int hc = blockIdx.x % hc_count;
  const int g = hc % a.hkv;
  const int hs = hc / a.hkv;
  int i, rt;
  if constexpr (PR) {
    i = a.n_blocks - 1;
    rt = a.n_rt - 1 - (int)(blockIdx.x / hc_count);   // longest row tiles first
  } else {
    const int pair = a.order[blockIdx.x / hc_count];
    i = pair / a.n_rt;
    rt = pair % a.n_rt;
  }
  const int wave = threadIdx.x >> 6;
  const int lr = threadIdx.x & 31;
  const int h = g * a.group + hs * a.hpw + (wave % a.hpw);
  const int r0 = rt * a.rpw + (wave / a.hpw) * 32;   // first own row of this wave

  const int span = a.chunk * a.kept;
  const int P = (i == 0) ? 0 : a.sink + span * i;
  const int n_rows = PR ? P : a.b;                  // query rows of the sequence
  const int n_pre = PR ? 0 : (P + KT - 1) / KT;     // list tiles seen in full
  const int own_end = min((rt + 1) * a.rpw, n_rows);
  const int n_own = (own_end + KT - 1) / KT;
  const int n_tiles = n_pre + n_own;
  const int64_t lst = p1_list_start(i, a.sink, span);
  const int32_t* krow = a.krow + lst;
  const int32_t* vcol = a.vcol + lst;
  const int64_t kb_ = (int64_t)g * a.b;                       // K rows of head g
  const int64_t vb_ = (int64_t)g * D * a.b;                   // V columns of head g
  const int64_t own_k = ((int64_t)i * a.hkv) * a.b + kb_;     // K row of own key 0
  const int64_t own_v = ((int64_t)i * a.hkv) * D * a.b + vb_; // V column of own key 0
  const uint16_t* kbase = a.kc;
  const uint16_t* vbase = a.vc;

  bf16x8 qf[NQ][D / 16];
  char* qlds = smem + 2 * Stage<D>::BYTES + (QL ? wave * QBYTES : 0);   // used when QL
  if constexpr (QL) {
    // Each lane of DMA x stages one 16-byte chunk of row x * RPI + lane / CPR;
    // rows past the sequence read row r0 (finite; their outputs are not written).
    using KTl = KTile<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int x = 0; x < 32 / KTl::RPI; ++x) {
      const int row = x * KTl::RPI + lane / KTl::CPR;
      int r = r0 + row;
      if (r >= n_rows) r = r0 < n_rows ? r0 : 0;
      int64_t pos = (int64_t)i * a.b + r;
      if constexpr (PR) {
        const int64_t kr = krow[r];
        const int64_t hb = (int64_t)a.hkv * a.b;
        pos = (kr / hb) * a.b + kr % hb;
      }
      const int c = (lane % KTl::CPR) ^ KTl::sw(row);
      dma16(a.q + (pos * a.hq + h) * D + 8 * c, qlds + x * 1024);
    }
    if constexpr (QRN > 0) {   // the register-held fragments (load_q's others go unused)
      const int r = r0 + lr;
      int64_t pos = (int64_t)i * a.b + r;
      if constexpr (PR) {
        const int64_t kr = r < n_rows ? krow[r] : 0;
        const int64_t hb = (int64_t)a.hkv * a.b;
        pos = (kr / hb) * a.b + kr % hb;
      }
      load_q<D>(r < n_rows ? a.q + (pos * a.hq + h) * D : nullptr, qf[0]);
    }
  } else {
    const int r = r0 + lr;
    int64_t pos = (int64_t)i * a.b + r;
    if constexpr (PR) {
      // position of list entry r: its K row is blk * Hkv * b + w, position blk * b + w
      const int64_t kr = r < n_rows ? krow[r] : 0;
      const int64_t hb = (int64_t)a.hkv * a.b;
      pos = (kr / hb) * a.b + kr % hb;
    }
    load_q<D>(r < n_rows ? a.q + (pos * a.hq + h) * D : nullptr, qf[0]);
  }

  FlashState<D, NQ> st;
  flash_init(st);

  // Staging, through buffer resources over the caches (byte offsets fit in 32
  // bits: L Hkv d < 2^31).  Every 8-entry run of a prefix list is 8 consecutive
  // cache rows (sink, chunk and block sizes are multiples of 8), and the K rows a
  // wave stages per tile are one such run: a K tile needs one list entry per
  // wave (a scalar load), and a lane's source offset is a constant of the lane
  // plus a per-wave base.  A V lane stages the 8-key run `v_run` of its d-row,
  // whose list entry it loads one tile ahead.  List entries past the list read
  // as 0 (the buffer resource ends with the list), which is a readable key, and
  // own-block runs past the block's b keys (a ragged last tile) read key 0.
  using KTl = KTile<D>;
  using VTl = VTile<D>;
  constexpr int KNI = KTl::NI, VNI = VTl::NI;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t kbytes = (uint32_t)a.n_blocks * a.hkv * a.b * D * 2;   // < 2^32 (L Hkv d < 2^31)
  const __amdgpu_buffer_rsrc_t krs = raw_rsrc(kbase, kbytes);
  const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(vbase, kbytes);
  const int n_list = PR ? n_rows : P;                  // entries of this block's list
  const __amdgpu_buffer_rsrc_t vls = raw_rsrc(vcol, (uint32_t)n_list * 4);
  const __attribute__((address_space(4))) int32_t* krow_s =
      (const __attribute__((address_space(4))) int32_t*)krow;
  uint32_t k_voff[KNI], v_voff[VNI], vl_voff[VNI];
#pragma unroll
  for (int x = 0; x < KNI; ++x) {
    const int row = (wv * KNI + x) * KTl::RPI + lane / KTl::CPR;   // tile row (0..63)
    const int c = (lane % KTl::CPR) ^ KTl::sw(row);
    k_voff[x] = (uint32_t)((row - 8 * wv) * D + 8 * c) * 2;
  }
  int v_run[VNI];
#pragma unroll
  for (int y = 0; y < VNI; ++y) {
    const int dv = (wv * VNI + y) * VTl::RPI + lane / VTl::CPR;   // d-row (0..D-1)
    v_run[y] = (lane % VTl::CPR) ^ VTl::sw(dv);                   // 8-key run of the tile
    v_voff[y] = (uint32_t)dv * (uint32_t)a.b * 2;
    vl_voff[y] = (uint32_t)(8 * v_run[y]) * 4;
  }
  int32_t k_ent = 0;        // list entry of this wave's K run of the next tile to stage
  int32_t rv[VNI];          // list entries of this lane's V runs of that tile
  const bool stager = !QL || wv < NW;   // the first 8 waves stage the tiles (one K run each)
  auto fetch_raw = [&](int t) __attribute__((always_inline)) {
    if (stager && (PR || t < n_pre)) {
      const int e = t * KT + 8 * wv;
      k_ent = krow_s[e < n_list ? e : 0];
#pragma unroll
      for (int y = 0; y < VNI; ++y)
        rv[y] = __builtin_amdgcn_raw_buffer_load_b32(vls, vl_voff[y] + (uint32_t)t * (KT * 4), 0, 0);
    }
  };
  // part 0: K only, 1: V only, 2: both
  auto stage = [&](int t, char* dst, int part) __attribute__((always_inline)) {
    if (!stager) return;
    const bool pre = PR || t < n_pre;
    uint32_t ks, vs;
    bool v_const = true;
    if (pre) {
      ks = (uint32_t)(kb_ + k_ent) * (D * 2);
      vs = (uint32_t)vb_ * 2;
      v_const = false;
    } else {
      int kk = (t - n_pre) * KT + 8 * wv;
      kk = kk < a.b ? kk : 0;
      ks = (uint32_t)(own_k + kk) * (D * 2);
      v_const = (t - n_pre + 1) * KT <= a.b;
      vs = (uint32_t)(own_v + (v_const ? (t - n_pre) * KT : 0)) * 2;
    }
    if (part != 1) {
#pragma unroll
      for (int x = 0; x < KNI; ++x) dma16_buf(krs, k_voff[x], ks, dst + (wv * KNI + x) * 1024);
    }
    if (part == 0) return;
#pragma unroll
    for (int y = 0; y < VNI; ++y) {
      uint32_t vo;
      if (pre) {
        vo = v_voff[y] + (uint32_t)rv[y] * 2;
      } else if (v_const) {
        vo = v_voff[y] + (uint32_t)(8 * v_run[y]) * 2;
      } else {
        const int col = (t - n_pre) * KT + 8 * v_run[y];   // ragged last tile
        vo = v_voff[y] + (uint32_t)(col < a.b ? col : 0) * 2;
      }
      dma16_buf(vrs, vo, vs, dst + KTl::BYTES + (wv * VNI + y) * 1024);
    }
  };

  fetch_raw(0);
  stage(0, smem, 2);
  if (n_tiles > 1) fetch_raw(1);
  const float sl2 = a.scale_log2;
  for (int t = 0; t < n_tiles; ++t) {
    tile_barrier();  // tile t has landed for every wave; tile t-1 is no longer read
    const char* stg = smem + (t & 1) * Stage<D>::BYTES;
    char* nxt = smem + ((t + 1) & 1) * Stage<D>::BYTES;
    const bool more = t + 1 < n_tiles;
    const bool pre = t < n_pre;
    // The loads of tile t+1 are issued in two parts, each behind the K.Q^T
    // products of a subtile, so that a wave waiting to issue them has matrix
    // work in flight.
#pragma unroll
    for (int kt = 0; kt < NSUB; ++kt) {
      // prefix: every listed key is visible; own block: keys up to the row (causal)
      const int k1 = (pre ? t : t - n_pre) * KT + kt * 32;
      const int lim = pre ? P - k1 : min(r0 + lr - k1 + 1, own_end - k1);
      const bool act = __ballot(lim > 0) != 0;   // else past the list, or above the diagonal
      f32x16 s;
      if (act) {
        if constexpr (QL) sub_qk_lds<D, QRN>(stg, kt, qlds, qf[0], s);
        else sub_qk<D>(stg, kt, qf[0], s);
      }
      if (more) stage(t + 1, nxt, kt);
      if (kt == NSUB - 1 && t + 2 < n_tiles) fetch_raw(t + 2);
      if (act) {
        bf16x8 p[2];
        sub_softmax<D>(s, st, sl2, lim, p);
        sub_pv<D>(stg, kt, p, st);
      }
    }
  }

  const int r = r0 + lr;
  const int64_t orow = PR ? (int64_t)r : (int64_t)i * a.b + r;
  flash_finish<D, NQ>(st, 0, r < n_rows ? a.o + (orow * a.hq + h) * D : nullptr, nullptr);
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
      const int le = p1_count_le(v - pre, rpw, b, n_rt);
      const int lt = p1_count_le(v - pre - 1, rpw, b, n_rt);
      rank += n_rt - le;                     // pairs of block i2 with more tiles
      if (i2 < i) rank += le - lt;           // equal tiles, smaller pair id
      else if (i2 == i) rank += min(rt, le) - min(rt, lt);
    }
    order[rank] = pid;
  }
}

// phase1_kernel with the geometry's wave count
template <int D, bool PR>
void launch_p1(const Phase1Geometry& g, int grid, hipStream_t stream, const P1Args& a) {
  if (g.rows_per_wg / 32 * g.heads_per_wg == P1_WQ)
    hipLaunchKernelGGL((phase1_kernel<D, PR, P1_WQ>), dim3(grid), dim3(64 * P1_WQ), 0, stream, a);
  else
    hipLaunchKernelGGL((phase1_kernel<D, PR, NW>), dim3(grid), dim3(NTHR), 0, stream, a);
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
  // 12 waves (3 per SIMD) where the heads x 32-row groups divide them (GQA group
  // 1, 2, 3, 4, 6 or 12), else 8
  const int waves = (group <= P1_WQ && P1_WQ % group == 0) ? P1_WQ : NW;
  g.heads_per_wg = group >= waves ? waves : group;   // the waves split as heads x 32-row groups
  g.n_head_sub = group / g.heads_per_wg;
  g.rows_per_wg = 32 * (waves / g.heads_per_wg);
  g.n_row_tiles = (block_size + g.rows_per_wg - 1) / g.rows_per_wg;
  return g;
}

int64_t phase1_prefix_total(const Phase1Geometry& g) {
  if (g.n_blocks < 2) return 0;
  return p1_list_start(g.n_blocks, g.sink_size, g.chunk_size * g.kept);
}

int launch_phase1_lists(const Phase1Geometry& g, const int32_t* sel, int32_t* prefix_rows,
                        int32_t* order, hipStream_t stream) {
  const int n_pairs = g.n_blocks * g.n_row_tiles;
  hipLaunchKernelGGL(phase1_order, dim3((n_pairs + 255) / 256), dim3(256), 0, stream, g.n_blocks,
                     g.block_size, g.chunk_size, g.kept, g.sink_size, g.rows_per_wg,
                     g.n_row_tiles, order);
  const int64_t total = phase1_prefix_total(g);
  if (g.n_blocks > 1 && total > 0) {
    const int p_max = g.sink_size + g.chunk_size * g.kept * (g.n_blocks - 1);
    const int gx = (int)std::min<int64_t>(1024, ((int64_t)p_max + 255) / 256);
    hipLaunchKernelGGL(phase1_prefix_list, dim3(gx, g.n_blocks - 1), dim3(256), 0, stream, sel,
                       g.block_size, g.chunk_size, g.kept, g.sink_size, g.n_kv_heads, g.head_dim,
                       prefix_rows, prefix_rows + total);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_phase1_attend(const Phase1Geometry& g, const uint16_t* q_rot, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* prefix_rows,
                         const int32_t* order, float* o, hipStream_t stream) {
  const int n_pairs = g.n_blocks * g.n_row_tiles;
  const int64_t total = phase1_prefix_total(g);
  const int32_t* krow = prefix_rows;
  const int32_t* vcol = prefix_rows + total;
  P1Args a;
  a.q = q_rot;
  a.kc = k_cache;
  a.vc = v_cache;
  a.krow = krow;
  a.vcol = vcol;
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
  if (g.head_dim == 128) launch_p1<128, false>(g, grid, stream, a);
  else launch_p1<64, false>(g, grid, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int64_t phase1_prefix_rows_len(const Phase1Geometry& g) {
  return g.n_blocks < 2 ? 0 : (int64_t)g.sink_size + (int64_t)g.chunk_size * g.kept * (g.n_blocks - 1);
}

int launch_phase1_prefix_rows(const Phase1Geometry& g, const uint16_t* q_rot,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* prefix_rows, float* o_prefix, hipStream_t stream) {
  const int64_t n = phase1_prefix_rows_len(g);
  if (n == 0) return 0;
  const int64_t total = phase1_prefix_total(g);
  P1Args a;
  a.q = q_rot;
  a.kc = k_cache;
  a.vc = v_cache;
  a.krow = prefix_rows;
  a.vcol = prefix_rows + total;
  a.order = nullptr;
  a.o = o_prefix;
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
  a.rpw = g.rows_per_wg;
  a.n_rt = (int32_t)((n + g.rows_per_wg - 1) / g.rows_per_wg);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.head_dim));
  const int grid = a.n_rt * g.n_kv_heads * g.n_head_sub;
  if (g.head_dim == 128) launch_p1<128, true>(g, grid, stream, a);
  else launch_p1<64, true>(g, grid, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ------------------------------------------------------------------ Phase 2
struct P2Args {
  const uint16_t* q;    // [B][Lq][Hq][D], rotated
  const uint16_t* kc;   // [B][S][Hkv][n][D]
  const uint16_t* vc;   // [B][S][Hkv][D][n]
  const uint16_t* ks;   // self keys, rotated: token j of sequence b at ks + b * ks_seq + j * Hkv * D
  const uint16_t* vs;   // self values, d-major: (b, head, d) row at vs + b * vs_seq + (head * D + d) * vs_ld
  float* o_part;        // [B][n_parts][Lq][Hq][D]
  float* lse_part;      // [B][n_parts][Lq][Hq]
  int64_t ks_seq, vs_seq;
  int32_t batch, n_shards, n, lq, hq, hkv, group, splits, n_parts, n_rg;
  int32_t n_self;       // self tokens; the Lq queries are the last Lq of them
  int32_t vs_ld;        // >= n_self rounded up to 8
  float scale_log2;
  // Decode form only: when q_raw is set, q is not used and the kernel rotates
  // the pre-RoPE query rows itself (token t at position q_pos0 + t).
  const uint16_t* q_raw;
  int64_t q_pos0;
  double rope_base;
  int32_t rope_scaling;
  // Generation step (decode form with q_raw only): k_new / v_new
  // [B][lq][Hkv][D] pre-RoPE; the query tokens are the last lq self tokens and
  // the launch appends them first (rotated keys into ks_w, values into the
  // d-major vs_w).
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* ks_w;
  uint16_t* vs_w;
};

// cos / sin table of the in-kernel query rotation: at most 32 tokens x D/2 pairs
template <int D>
struct QTab {
  static constexpr int MAX_TOK = 32;
  static constexpr int BYTES = MAX_TOK * (D / 2) * 8;
};

// Generation step, append: self tokens tok_lo .. tok_hi - 1 (new tokens; token
// tk is new token tk - (n_self - lq), at the query position of that index) of
// sequence bb, KV head g, into the self caches: keys turned with the query
// rotation table, values into their d-major columns; when tok_hi is the last
// self token, the value columns after it up to the next multiple of 8 are
// zeroed (the attention reads values in runs of 8 keys).  Called by the whole
// workgroup, outside the attention loop (not inlined, so that its registers do
// not add to the loop's).
template <int D>
__device__ __forceinline__ void append_self_tokens(const uint16_t* k_new, const uint16_t* v_new,
                                                uint16_t* ks_w, uint16_t* vs_w, int64_t ks_seq,
                                                int64_t vs_seq, int vs_ld, int n_self, int lq,
                                                int hkv, const float2* tab, int bb, int g,
                                                int tok_lo, int tok_hi) {
  const int n_old = n_self - lq;
  uint16_t* kdst = ks_w + (int64_t)bb * ks_seq + (int64_t)g * D;
  uint16_t* vdst = vs_w + (int64_t)bb * vs_seq + (int64_t)g * D * vs_ld;
  const int n_tok = tok_hi - tok_lo;
  for (int e = threadIdx.x; e < n_tok * (D / 2); e += NTHR) {
    const int tk = tok_lo + e / (D / 2), i = e % (D / 2), t = tk - n_old;
    const uint16_t* src = k_new + (((int64_t)bb * lq + t) * hkv + g) * D;
    const float2 cs = tab[t * (D / 2) + i];
    float y1, y2;
    rope_pair(bf16_to_f32(src[i]), bf16_to_f32(src[i + D / 2]), cs.x, cs.y, y1, y2);
    uint16_t* kr = kdst + (int64_t)tk * hkv * D;
    kr[i] = __builtin_bit_cast(uint16_t, (__bf16)y1);
    kr[i + D / 2] = __builtin_bit_cast(uint16_t, (__bf16)y2);
  }
  for (int e = threadIdx.x; e < n_tok * D; e += NTHR) {
    const int tk = tok_lo + e / D, d = e % D, t = tk - n_old;
    vdst[(int64_t)d * vs_ld + tk] = v_new[(((int64_t)bb * lq + t) * hkv + g) * D + d];
  }
  if (tok_hi == n_self) {
    const int pad = ((n_self + 7) & ~7) - n_self;
    for (int e = threadIdx.x; e < D * pad; e += NTHR)
      vdst[(int64_t)(e / pad) * vs_ld + n_self + e % pad] = 0;
  }
}

// KSPLIT: the decode form (all query rows of the workgroup in one 32-row wave),
// chosen by the launcher; two waves then split the subtiles of every tile.
template <int D, bool KSPLIT, bool FUSED = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(NTHR, NTHR), amdgpu_waves_per_eu(2, 2)))
phase2_kernel(P2Args a) {
  static_assert(!FUSED || KSPLIT, "the generation step's append runs in the decode form");
  constexpr int NQ = 1;
  // Tile slots.  The decode form streams its part from HBM with little work per
  // tile, so its loads run three tiles ahead (four slots, 128 KB at d = 128);
  // otherwise one tile ahead (two slots).
  constexpr int NSLOT = KSPLIT ? 4 : 2;
  constexpr int AHEAD = NSLOT - 1;
  // one LDS object: the slots, then (decode form) the query rotation table
  constexpr int TAB = KSPLIT ? QTab<D>::BYTES : 0;
  __shared__ __attribute__((aligned(1024))) char smem[NSLOT * Stage<D>::BYTES + TAB];

  int w = blockIdx.x;
  const int p = w % a.n_parts;
  w /= a.n_parts;
  const int rg = w % a.n_rg;
  w /= a.n_rg;
  const int g = w % a.hkv;
  const int bb = w / a.hkv;
  const int wave = threadIdx.x >> 6;
  const int lr = threadIdx.x & 31;
  const int n_rows = a.group * a.lq;
  // Decode shapes (every query row of the workgroup fits one 32-row wave): two
  // waves share the rows and take one of the two subtiles of every tile each,
  // so the matrix work per tile is split; their partial states are combined
  // exactly at the end.
  constexpr bool key_split = KSPLIT;
  const int row_base = key_split ? 0 : rg * (NW * 32) + wave * 32;

  // Key tiles of this (sequence, KV head): every retained shard's tiles in shard
  // order, then the self tiles.  The parts take equal contiguous ranges of them,
  // so the self keys add at most one tile to a part instead of a part of their own.
  const int nt = (a.n + KT - 1) / KT;
  const int64_t shard_tiles = (int64_t)a.n_shards * nt;
  const int64_t all_tiles = shard_tiles + (a.n_self + KT - 1) / KT;
  const int64_t t0 = (int64_t)p * all_tiles / a.n_parts;
  const int n_tiles = (int)((int64_t)(p + 1) * all_tiles / a.n_parts - t0);
  // Source of a tile: keys lo .. hi - 1 of one shard, or of the self shard, which
  // is attended causally.
  struct Src {
    const uint16_t* k;
    const uint16_t* v;
    int64_t k_ld, v_ld;
    int lo, hi;
    bool causal;
  };
  // Tile cursor: tile lt of shard `shard`, shard n_shards being the self shard.
  // Staging and compute each walk the part's tiles with one, so no tile index is
  // divided inside the loop.
  struct Cur {
    int shard, lt;
  };
  Cur first;
  if (t0 < shard_tiles) {
    first.shard = (int)(t0 / nt);
    first.lt = (int)(t0 - (int64_t)first.shard * nt);
  } else {
    first.shard = a.n_shards;
    first.lt = (int)(t0 - shard_tiles);
  }
  auto advance = [&](Cur& c) __attribute__((always_inline)) {
    if (++c.lt == nt && c.shard < a.n_shards) {
      c.lt = 0;
      ++c.shard;
    }
  };
  auto src_of = [&](const Cur& c) __attribute__((always_inline)) {
    Src r;
    r.lo = c.lt * KT;
    if (c.shard < a.n_shards) {
      const int64_t base = (((int64_t)bb * a.n_shards + c.shard) * a.hkv + g) * a.n * D;
      r.k = a.kc + base;
      r.v = a.vc + base;
      r.k_ld = D;
      r.v_ld = a.n;
      r.hi = a.n;
      r.causal = false;
    } else {
      r.k = a.ks + (int64_t)bb * a.ks_seq + (int64_t)g * D;
      r.v = a.vs + (int64_t)bb * a.vs_seq + (int64_t)g * D * a.vs_ld;
      r.k_ld = (int64_t)a.hkv * D;
      r.v_ld = a.vs_ld;
      r.hi = a.n_self;
      r.causal = true;
    }
    return r;
  };

  // query fragments: row fr = head-in-group * Lq + token
  bf16x8 qf[NQ][D / 16];
  const bool wave_active = key_split ? wave < NSUB : row_base < n_rows;
  const int fr = row_base + lr;
  const bool rotate_q = KSPLIT && a.q_raw != nullptr;
  const uint16_t* qrow = nullptr;
  if (fr < n_rows) {
    const int hh = fr / a.lq, t = fr % a.lq;
    qrow = (rotate_q ? a.q_raw : a.q) + (((int64_t)bb * a.lq + t) * a.hq + g * a.group + hh) * D;
  }
  load_q<D>(qrow, qf[0]);   // pre-RoPE when rotate_q: turned once the table is ready
  const int tok = fr % a.lq;

  FlashState<D, NQ> st;
  flash_init(st);

  // Shard tiles are staged through buffer resources over the (sequence, shard,
  // KV head) slabs: a lane's source offset within a tile is a constant of the
  // lane (computed here once) and the tile adds a scalar offset, so staging a
  // tile costs no per-lane address arithmetic.  Keys past the shard read zero
  // (past the K slab) or the next value row (inside the V slab), both finite
  // and masked below.  Self tiles (at most a couple per part) take the per-lane
  // path further down, whose keys past the self tokens read the tile's first key.
  uint32_t k_vo[KTile<D>::NI], v_vo[VTile<D>::NI];
  {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int x = 0; x < KTile<D>::NI; ++x) {
      const int row = staged_k_row<D>(x);
      const int c = (lane % KTile<D>::CPR) ^ KTile<D>::sw(row);
      k_vo[x] = (uint32_t)((row * D + 8 * c) * 2);
    }
#pragma unroll
    for (int y = 0; y < VTile<D>::NI; ++y)
      v_vo[y] = (uint32_t)((staged_v_d<D>(y) * (uint32_t)a.n + 8 * staged_v_chunk<D>(y)) * 2);
  }
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto stage_part_tile = [&](char* dst, const Cur& c) __attribute__((always_inline)) {
    if (c.shard < a.n_shards) {
      const int64_t base = (((int64_t)bb * a.n_shards + c.shard) * a.hkv + g) * a.n * D;
      const uint32_t bytes = (uint32_t)a.n * D * 2;
      const __amdgpu_buffer_rsrc_t krs = raw_rsrc(a.kc + base, bytes);
      const __amdgpu_buffer_rsrc_t vrs = raw_rsrc(a.vc + base, bytes);
      const uint32_t lo = (uint32_t)c.lt * KT;
#pragma unroll
      for (int x = 0; x < KTile<D>::NI; ++x)
        dma16_buf(krs, k_vo[x], lo * D * 2, dst + (wv * KTile<D>::NI + x) * 1024);
#pragma unroll
      for (int y = 0; y < VTile<D>::NI; ++y)
        dma16_buf(vrs, v_vo[y], lo * 2, dst + KTile<D>::BYTES + (wv * VTile<D>::NI + y) * 1024);
      return;
    }
    const Src r = src_of(c);
    TileSrc<D> sr;
#pragma unroll
    for (int x = 0; x < KTile<D>::NI; ++x) {
      const int kk = r.lo + staged_k_row<D>(x);
      sr.k[x] = (int64_t)(kk < r.hi ? kk : r.lo) * r.k_ld;
    }
#pragma unroll
    for (int x = 0; x < VTile<D>::NI; ++x) {
      const int kk = r.lo + 8 * staged_v_chunk<D>(x);
      sr.v[x] = kk < r.hi ? kk : r.lo;
    }
    stage_tile<D>(dst, r.k, r.v, r.v_ld, sr);
  };
  // Every iteration issues the same ND loads per wave (tiles past the part are
  // staged into a free slot and never read), so at each barrier exactly the
  // loads of the AHEAD - 1 newest tiles may still be in flight.
  constexpr int ND = KTile<D>::NI + VTile<D>::NI;
  auto slot = [&](int t) __attribute__((always_inline)) { return smem + (t % NSLOT) * Stage<D>::BYTES; };
  // Decode form with a pre-RoPE query: cos / sin of every (token, pair) into the
  // table before the first tiles are staged (an LDS store issued while the tile
  // loads are in flight would first wait for all of them).
  float2* tab = reinterpret_cast<float2*>(smem + NSLOT * Stage<D>::BYTES);
  if (rotate_q) {
    for (int e = threadIdx.x; e < a.lq * (D / 2); e += NTHR) {
      float c, sn;
      rope_cos_sin(a.q_pos0 + e / (D / 2), e % (D / 2), D / 2, a.rope_base, a.rope_scaling, &c, &sn);
      tab[e] = make_float2(c, sn);
    }
  }
  if constexpr (FUSED) {
    // Append the query tokens (self tokens n_self - lq .. n_self - 1) that lie in
    // this part's self tiles, for KV head g, before this workgroup stages any
    // tile, so that its own loads see them; no other workgroup reads those tiles.
    const int64_t s_lo = (t0 > shard_tiles ? t0 : shard_tiles) - shard_tiles;
    const int64_t s_hi = (t0 + n_tiles < all_tiles ? t0 + n_tiles : all_tiles) - shard_tiles;
    const int n_old = a.n_self - a.lq;
    const int tok_lo = (int)(s_lo * KT > n_old ? s_lo * KT : n_old);
    const int tok_hi = (int)(s_hi * KT < a.n_self ? s_hi * KT : a.n_self);
    if (tok_lo < tok_hi) {
      __syncthreads();   // the table is written
      append_self_tokens<D>(a.k_new, a.v_new, a.ks_w, a.vs_w, a.ks_seq, a.vs_seq, a.vs_ld, a.n_self,
                            a.lq, a.hkv, tab, bb, g, tok_lo, tok_hi);
      __syncthreads();   // the stores have completed before any tile load is issued
    }
  }
  // tiles past the part: the staging cursor stays on the last tile (staged into a
  // free slot, never read)
  Cur sc = first;
#pragma unroll
  for (int u = 0; u < AHEAD; ++u) {
    stage_part_tile(slot(u), sc);
    if (u < n_tiles - 1) advance(sc);
  }
  if (rotate_q) {
    // Each lane turns the pairs (i, i + D/2) it holds: i = 16 ks + 8 half + j for
    // ks < D/32, the partner in fragment ks + D/32.
    tile_barrier_n<AHEAD * ND>();   // the table is written; the tiles may still be in flight
    if (qrow) {
      const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float2 cs = tab[tok * (D / 2) + 16 * ks + 8 * half + j];
          float y1, y2;
          rope_pair((float)qf[0][ks][j], (float)qf[0][ks + D / 32][j], cs.x, cs.y, y1, y2);
          qf[0][ks][j] = (__bf16)y1;
          qf[0][ks + D / 32][j] = (__bf16)y2;
        }
    }
  }
  const float sl2 = a.scale_log2;
  Cur cc = first;
  for (int t = 0; t < n_tiles; ++t) {
    tile_barrier_n<(AHEAD - 1) * ND>();   // tile t has landed; every wave is past its reads of tile t-1
    stage_part_tile(slot(t + AHEAD), sc);   // into the slot of tile t-1
    if (t + AHEAD < n_tiles - 1) advance(sc);
    if (!wave_active) continue;
    const char* stg = slot(t);
    const Src r = src_of(cc);
    advance(cc);
#pragma unroll
    for (int kt = 0; kt < NSUB; ++kt) {
      if (key_split && kt != wave) continue;
      // shard keys are all visible; self keys up to the query token itself
      // (query token tok is self token n_self - Lq + tok)
      const int kb = r.lo + kt * 32;
      const int lim = r.causal ? min(a.n_self - a.lq + tok - kb + 1, r.hi - kb) : r.hi - kb;
      if (!__ballot(lim > 0)) break;
      f32x16 s;
      bf16x8 p[2];
      sub_qk<D>(stg, kt, qf[0], s);
      sub_softmax<D>(s, st, sl2, lim, p);
      sub_pv<D>(stg, kt, p, st);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load may land after the workgroup ends

  if (key_split) {
    // Wave 1 hands its state to wave 0 through LDS (every wave is past its last
    // read of the slots); wave 0 merges: m = max(m0, m1), O and l rescaled by
    // exp2(m_i - m) and added.  Both waves hold the same rows in the same lanes.
    constexpr int NO = D / 32 * 16;   // accumulator floats per lane
    float* xf = reinterpret_cast<float*>(smem);
    const int lane = threadIdx.x & 63;
    __syncthreads();
    if (wave == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xf[(dt * 16 + r) * 64 + lane] = st.o[dt][0][r];
      xf[NO * 64 + lane] = st.m[0];
      xf[(NO + 1) * 64 + lane] = st.l[0];
    }
    __syncthreads();
    if (wave != 0) return;
    const float m1 = xf[NO * 64 + lane];
    const float m = fmaxf(st.m[0], m1);
    const float a0 = __builtin_amdgcn_exp2f(st.m[0] - m);
    const float a1 = __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        st.o[dt][0][r] = st.o[dt][0][r] * a0 + xf[(dt * 16 + r) * 64 + lane] * a1;
    st.l[0] = st.l[0] * a0 + xf[(NO + 1) * 64 + lane] * a1;
    st.m[0] = m;
  }

  if (!wave_active) return;
  float* orow = nullptr;
  float* lrow = nullptr;
  if (fr < n_rows) {
    const int hh = fr / a.lq;
    const int h = g * a.group + hh;
    const int64_t rix = (((int64_t)bb * a.n_parts + p) * a.lq + tok) * a.hq + h;
    orow = a.o_part + rix * D;
    lrow = a.lse_part + rix;
  }
  flash_finish<D, NQ>(st, 0, orow, lrow);
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
  g.nq = 1;
  const int rows_per_wg = NW * 32;
  g.n_row_groups = (rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t combos = (int64_t)batch * n_kv_heads * n_shards * g.n_row_groups;
  const int64_t target = 256;   // one workgroup per CU
  int64_t splits = combos > 0 ? (target + combos - 1) / combos : 1;
  const int64_t nt = (shard_len + KT - 1) / KT;
  if (splits > nt) splits = nt;
  if (splits < 1) splits = 1;
  g.splits = (int32_t)splits;
  // the self tiles join the shards' tiles; with no shard one part holds them
  g.n_parts = n_shards > 0 ? n_shards * g.splits : 1;
  g.self_pad = (q_len + KT - 1) / KT * KT;
  return g;
}

bool phase2_decode_form(const Phase2Geometry& g) {
  return g.n_row_groups == 1 && (g.n_q_heads / g.n_kv_heads) * g.q_len <= 32;
}

int launch_phase2(const Phase2Geometry& g, const uint16_t* q_rot, const uint16_t* k_cache,
                  const uint16_t* v_cache, const SelfShard& self, float* o_part,
                  float* lse_part, hipStream_t stream, const RawQuery* raw,
                  const FusedStep* step) {
  P2Args a;
  a.k_new = step ? step->k_new : nullptr;
  a.v_new = step ? step->v_new : nullptr;
  a.ks_w = step ? step->k_self : nullptr;
  a.vs_w = step ? step->v_self : nullptr;
  a.q = q_rot;
  a.q_raw = raw ? raw->q : nullptr;
  a.q_pos0 = raw ? raw->pos0 : 0;
  a.rope_base = raw ? raw->base : 0.0;
  a.rope_scaling = raw ? raw->scaling : 0;
  a.kc = k_cache;
  a.vc = v_cache;
  a.ks = self.k;
  a.vs = self.v;
  a.ks_seq = self.k_seq;
  a.vs_seq = self.v_seq;
  a.n_self = self.n;
  a.vs_ld = self.v_ld;
  a.o_part = o_part;
  a.lse_part = lse_part;
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
  const bool ksplit = phase2_decode_form(g);
  if (raw && (!ksplit || g.q_len > QTab<128>::MAX_TOK)) return -1;
  if (step && !raw) return -1;
  if (g.head_dim == 128) {
    if (step) hipLaunchKernelGGL((phase2_kernel<128, true, true>), dim3(grid), dim3(NTHR), 0, stream, a);
    else if (ksplit) hipLaunchKernelGGL((phase2_kernel<128, true>), dim3(grid), dim3(NTHR), 0, stream, a);
    else hipLaunchKernelGGL((phase2_kernel<128, false>), dim3(grid), dim3(NTHR), 0, stream, a);
  } else {
    if (step) hipLaunchKernelGGL((phase2_kernel<64, true, true>), dim3(grid), dim3(NTHR), 0, stream, a);
    else if (ksplit) hipLaunchKernelGGL((phase2_kernel<64, true>), dim3(grid), dim3(NTHR), 0, stream, a);
    else hipLaunchKernelGGL((phase2_kernel<64, false>), dim3(grid), dim3(NTHR), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace pulsar
