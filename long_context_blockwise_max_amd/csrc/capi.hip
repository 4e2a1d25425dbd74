// C ABI of the Pulsar hot path: host-side validation, workspace carving and
// launches on the caller's stream.  Declarations and contracts: include/pulsar.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/pulsar.h"
#include "launch.hpp"

using namespace pulsar;

namespace {

constexpr int64_t kMaxVocab = 1 << 20;
constexpr int64_t kMaxContext = int64_t(1) << 30;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t kept_chunks(const pulsar_geom* g) {
  const int32_t n_chunks = g->block_size / g->chunk_size;
  return g->budget_chunks < n_chunks ? g->budget_chunks : n_chunks;
}

int check_geom(const pulsar_geom* g) {
  if (!g) return PULSAR_EINVAL;
  if (g->n_blocks < 1 || g->block_size < 1 || g->chunk_size < 1 || g->budget_chunks < 0 ||
      g->sink_size < 0 || g->vocab_size < 1)
    return PULSAR_EINVAL;
  if (g->block_size % g->chunk_size != 0) return PULSAR_EINVAL;
  // the d-major value tiles move keys in runs of 8: runs must not straddle a chunk or the sink
  if (g->chunk_size % 8 != 0 || g->sink_size % 8 != 0) return PULSAR_EUNSUPPORTED;
  const int64_t L = (int64_t)g->n_blocks * g->block_size;
  if (L > kMaxContext) return PULSAR_EUNSUPPORTED;
  if (g->vocab_size > kMaxVocab) return PULSAR_EUNSUPPORTED;
  if (g->sink_size > L) return PULSAR_EINVAL;
  const int64_t n_chunks = g->block_size / g->chunk_size;
  if (n_chunks + g->n_blocks + 2 > 40000) return PULSAR_EUNSUPPORTED;  // LDS of the top-k kernel
  const int64_t p_last = (int64_t)g->sink_size +
                         (int64_t)g->chunk_size * kept_chunks(g) * (g->n_blocks - 1);
  if (p_last > (int64_t(1) << 30)) return PULSAR_EUNSUPPORTED;
  return PULSAR_OK;
}

int check_attn(const pulsar_attn* a) {
  if (!a) return PULSAR_EINVAL;
  if (a->n_q_heads < 1 || a->n_kv_heads < 1) return PULSAR_EINVAL;
  if (a->rope_scaling != 0 && a->rope_scaling != 1) return PULSAR_EINVAL;
  if (a->n_q_heads % a->n_kv_heads != 0) return PULSAR_EINVAL;
  if (!(a->rope_base > 1.0) || !isfinite(a->rope_base)) return PULSAR_EINVAL;
  if (a->head_dim != 64 && a->head_dim != 128) return PULSAR_EUNSUPPORTED;
  const int group = a->n_q_heads / a->n_kv_heads;
  if (!(group == 1 || group == 2 || group == 4 || group % 8 == 0)) return PULSAR_EUNSUPPORTED;
  return PULSAR_OK;
}

// cache element offsets are formed in 32-bit list entries: L * Hkv * d must fit
int check_pair(const pulsar_geom* g, const pulsar_attn* a) {
  const int64_t L = (int64_t)g->n_blocks * g->block_size;
  if (L * a->n_kv_heads * a->head_dim > INT32_MAX) return PULSAR_EUNSUPPORTED;
  return PULSAR_OK;
}

// select + phase 1 workspace: status word | df | chunk keys | chunk ranks |
// block bitmaps | rotated q | prefix lists | work order (keys and ranks serve
// the selection methods other than Max-IDF; Max-IDF keeps its chunk scores in
// the ranks area when the caller does not ask for them)
struct Layout {
  size_t status, df, keys, ranks, bits, q_rot, lists, order, total;
};

Layout layout(const pulsar_geom* g, const pulsar_attn* a) {
  Layout l{};
  size_t off = 0;
  l.status = off;
  off += kAlign;
  l.df = off;
  off = align_up(off + (size_t)g->vocab_size * 4);
  const size_t chunks = (size_t)g->n_blocks * (g->block_size / g->chunk_size);
  l.keys = off;
  off = align_up(off + chunks * 32);
  l.ranks = off;
  off = align_up(off + chunks * 4);
  l.bits = off;
  off = align_up(off + (size_t)g->n_blocks * ((g->vocab_size + 31) / 32) * 4);
  const int64_t L = (int64_t)g->n_blocks * g->block_size;
  l.q_rot = l.lists = l.order = off;
  if (a) {
    Phase1Geometry pg = phase1_geometry(g->n_blocks, g->block_size, g->chunk_size,
                                        kept_chunks(g), g->sink_size, a->n_q_heads,
                                        a->n_kv_heads, a->head_dim);
    l.q_rot = off;
    off = align_up(off + (size_t)L * a->n_q_heads * a->head_dim * 2);
    l.lists = off;
    off = align_up(off + (size_t)phase1_prefix_total(pg) * 2 * 4);
    l.order = off;
    off = align_up(off + (size_t)pg.n_blocks * pg.n_row_tiles * 4);
  }
  l.total = off;
  return l;
}

// phase 2 workspace: rotated query | rotated self keys | d-major self values
struct Layout2 {
  size_t q_rot, k_rot, v_t, total;
};

Layout2 layout2(const Phase2Geometry& pg) {
  Layout2 l{};
  size_t off = 0;
  const size_t tok = (size_t)pg.batch * pg.q_len;
  l.q_rot = off;
  off = align_up(off + tok * pg.n_q_heads * pg.head_dim * 2);
  l.k_rot = l.v_t = off;
  if (pg.has_self) {
    off = align_up(off + tok * pg.n_kv_heads * pg.head_dim * 2);
    l.v_t = off;
    off = align_up(off + (size_t)pg.batch * pg.n_kv_heads * pg.head_dim * pg.self_pad * 2);
  }
  l.total = off;
  return l;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// one workgroup per (sequence, KV head, row group, part); a launch takes at most
// 2^31 - 1 workgroups
bool phase2_grid_ok(const Phase2Geometry& pg) {
  if ((int64_t)pg.batch * pg.n_kv_heads * pg.n_row_groups * pg.n_parts > INT32_MAX) return false;
  // the preparation launch: one workgroup per query token, plus one per 64 self
  // tokens of each sequence and KV head for the value transpose
  const int64_t tok = (int64_t)pg.batch * pg.q_len;
  const int64_t vt = pg.has_self ? (int64_t)((pg.q_len + 63) / 64) * pg.n_kv_heads * pg.batch : 0;
  return tok + vt <= INT32_MAX;
}

}  // namespace

extern "C" {

size_t pulsar_workspace_bytes(const pulsar_geom* g, const pulsar_attn* a) {
  if (check_geom(g) != PULSAR_OK) return 0;
  if (a && (check_attn(a) != PULSAR_OK || check_pair(g, a) != PULSAR_OK)) return 0;
  return layout(g, a).total;
}

int32_t pulsar_kept_chunks(const pulsar_geom* g) {
  if (check_geom(g) != PULSAR_OK) return -1;
  return kept_chunks(g);
}

int pulsar_select(const pulsar_geom* g, const int32_t* tok, int32_t* sel, int32_t* chunk_min_df,
                  int32_t* df, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_geom(g);
  if (rc) return rc;
  const int32_t kept = kept_chunks(g);
  if (!aligned16(tok)) return PULSAR_EINVAL;
  if (kept > 0 && !aligned16(sel)) return PULSAR_EINVAL;
  if (chunk_min_df && !aligned16(chunk_min_df)) return PULSAR_EINVAL;
  if (df && !aligned16(df)) return PULSAR_EINVAL;
  const Layout l = layout(g, nullptr);
  if (!ws || ws_bytes < l.total) return PULSAR_EWORKSPACE;
  if (!aligned16(ws)) return PULSAR_EINVAL;
  char* w = static_cast<char*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(w + l.status);
  // chunk scores land in chunk_min_df when the caller wants them, else in the
  // workspace's per-chunk rank area (used only by the other selection methods)
  int32_t* scores = chunk_min_df ? chunk_min_df : reinterpret_cast<int32_t*>(w + l.ranks);
  int32_t* dfp = df ? df : reinterpret_cast<int32_t*>(w + l.df);
  return launch_select(tok, g->n_blocks, g->block_size, g->chunk_size, kept, g->vocab_size, sel,
                       scores, dfp, reinterpret_cast<uint32_t*>(w + l.bits), status,
                       as_stream(stream)) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

int pulsar_select_method(const pulsar_geom* g, int32_t method, uint64_t seed, const int32_t* tok,
                         int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  if (method == PULSAR_SELECT_MAX_IDF) return pulsar_select(g, tok, sel, nullptr, nullptr, ws, ws_bytes, stream);
  int rc = check_geom(g);
  if (rc) return rc;
  if (method < PULSAR_SELECT_MEAN_IDF || method > PULSAR_SELECT_EVEN) return PULSAR_EINVAL;
  const int32_t kept = kept_chunks(g);
  const bool reads_tokens = method == PULSAR_SELECT_MEAN_IDF || method == PULSAR_SELECT_ENTROPY;
  if (reads_tokens && !aligned16(tok)) return PULSAR_EINVAL;
  if (kept > 0 && !aligned16(sel)) return PULSAR_EINVAL;
  // the exact order keys are products over a chunk's positions held in 256 bits
  if (method == PULSAR_SELECT_MEAN_IDF && g->chunk_size * log2((double)g->n_blocks) >= 255.5)
    return PULSAR_EUNSUPPORTED;
  if (method == PULSAR_SELECT_ENTROPY && g->chunk_size * log2((double)g->chunk_size) >= 255.5)
    return PULSAR_EUNSUPPORTED;
  const Layout l = layout(g, nullptr);
  if (!ws || ws_bytes < l.total) return PULSAR_EWORKSPACE;
  if (!aligned16(ws)) return PULSAR_EINVAL;
  char* w = static_cast<char*>(ws);
  int32_t* status = reinterpret_cast<int32_t*>(w + l.status);
  int32_t* dfp = reinterpret_cast<int32_t*>(w + l.df);
  uint32_t* keys = reinterpret_cast<uint32_t*>(w + l.keys);
  int32_t* ranks = reinterpret_cast<int32_t*>(w + l.ranks);
  uint32_t* bits = reinterpret_cast<uint32_t*>(w + l.bits);
  return launch_select_method(method, seed, tok, g->n_blocks, g->block_size, g->chunk_size, kept,
                              g->vocab_size, sel, dfp, bits, keys, ranks, status,
                              as_stream(stream)) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

}  // extern "C"

namespace {

// shared checks of the three Phase-1 calls; fills the workspace pointers
struct P1Ws {
  uint16_t* q_rot;
  int32_t* lists;
  int32_t* order;
  Phase1Geometry pg;
};

int phase1_common(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* k_cache,
                  const uint16_t* v_cache, void* ws, size_t ws_bytes, P1Ws* out) {
  int rc = check_geom(g);
  if (rc) return rc;
  rc = check_attn(a);
  if (rc) return rc;
  rc = check_pair(g, a);
  if (rc) return rc;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PULSAR_EINVAL;
  const Layout l = layout(g, a);
  if (!ws || ws_bytes < l.total) return PULSAR_EWORKSPACE;
  if (!aligned16(ws)) return PULSAR_EINVAL;
  char* w = static_cast<char*>(ws);
  out->q_rot = reinterpret_cast<uint16_t*>(w + l.q_rot);
  out->lists = reinterpret_cast<int32_t*>(w + l.lists);
  out->order = reinterpret_cast<int32_t*>(w + l.order);
  out->pg = phase1_geometry(g->n_blocks, g->block_size, g->chunk_size, kept_chunks(g),
                            g->sink_size, a->n_q_heads, a->n_kv_heads, a->head_dim);
  return PULSAR_OK;
}

int phase1_prepare_checked(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* q,
                           const uint16_t* k, const uint16_t* v, const int32_t* sel,
                           uint16_t* k_cache, uint16_t* v_cache, const P1Ws& w, hipStream_t s) {
  const int64_t L = (int64_t)g->n_blocks * g->block_size;
  if (launch_rope_fill(q, k, v, L, g->block_size, a->n_q_heads, a->n_kv_heads, a->head_dim,
                       a->rope_base, a->rope_scaling, w.q_rot, k_cache, v_cache, s))
    return PULSAR_EHIP;
  if (launch_phase1_lists(w.pg, sel, w.lists, w.order, s)) return PULSAR_EHIP;
  return PULSAR_OK;
}

int prepare_pointers_ok(const pulsar_geom* g, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int32_t* sel) {
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return PULSAR_EINVAL;
  if (g->n_blocks > 1 && kept_chunks(g) > 0 && !aligned16(sel)) return PULSAR_EINVAL;
  return PULSAR_OK;
}

// Checks shared by the two Phase-2 query calls (everything but the workspace);
// fills the launch geometry.
int phase2_query_checked(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                         int32_t shard_len, const uint16_t* qq, int32_t q_len, int64_t q_pos0,
                         const uint16_t* k_cache, const uint16_t* v_cache,
                         const uint16_t* k_self, const uint16_t* v_self, const float* o_part,
                         const float* lse_part, int32_t n_parts, Phase2Geometry* out) {
  const int has_self = k_self != nullptr || v_self != nullptr;
  const int32_t want = pulsar_phase2_num_parts(a, batch, n_shards, shard_len, q_len, has_self);
  if (want <= 0) return want < 0 ? want : PULSAR_EINVAL;
  if (n_parts != want) return PULSAR_EINVAL;
  if (has_self && (!aligned16(k_self) || !aligned16(v_self))) return PULSAR_EINVAL;
  if (!aligned16(qq) || !aligned16(o_part) || !lse_part) return PULSAR_EINVAL;
  if (n_shards > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) return PULSAR_EINVAL;
  if (n_shards > 0 && shard_len % 8 != 0) return PULSAR_EUNSUPPORTED;  // d-major value runs of 8
  if (q_pos0 < 0) return PULSAR_EINVAL;
  if ((int64_t)batch * n_shards * shard_len * a->n_kv_heads > INT32_MAX) return PULSAR_EUNSUPPORTED;
  if ((int64_t)shard_len * a->head_dim * 2 > UINT32_MAX) return PULSAR_EUNSUPPORTED;  // slab bytes
  if ((int64_t)batch * q_len > INT32_MAX / 2) return PULSAR_EUNSUPPORTED;
  *out = phase2_geometry(batch, n_shards, n_shards > 0 ? shard_len : 1, q_len, a->n_q_heads,
                         a->n_kv_heads, a->head_dim, has_self);
  if (!phase2_grid_ok(*out)) return PULSAR_EUNSUPPORTED;
  return PULSAR_OK;
}

// Preparation and attention launches of a checked Phase-2 query over the
// workspace at w (layout2(pg).total bytes).
int phase2_query_launch(const pulsar_attn* a, const Phase2Geometry& pg, const uint16_t* qq,
                        int64_t q_pos0, const uint16_t* k_cache, const uint16_t* v_cache,
                        const uint16_t* k_self, const uint16_t* v_self, float* o_part,
                        float* lse_part, char* w, hipStream_t s) {
  const bool has_self = pg.has_self != 0;
  const Layout2 l = layout2(pg);
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(w + l.q_rot);
  uint16_t* k_rot = has_self ? reinterpret_cast<uint16_t*>(w + l.k_rot) : nullptr;
  uint16_t* v_t = has_self ? reinterpret_cast<uint16_t*>(w + l.v_t) : nullptr;
  if (launch_phase2_prep(qq, has_self ? k_self : nullptr, v_self, pg.batch, pg.q_len,
                         a->n_q_heads, a->n_kv_heads, a->head_dim, q_pos0, a->rope_base,
                         a->rope_scaling, pg.self_pad, q_rot, k_rot, v_t, s))
    return PULSAR_EHIP;
  SelfShard self{};
  if (has_self) {
    self.k = k_rot;
    self.v = v_t;
    self.k_seq = (int64_t)pg.q_len * a->n_kv_heads * a->head_dim;
    self.v_seq = (int64_t)a->n_kv_heads * a->head_dim * pg.self_pad;
    self.n = pg.q_len;
    self.v_ld = pg.self_pad;
  }
  return launch_phase2(pg, q_rot, k_cache, v_cache, self, o_part, lse_part, s) == 0 ? PULSAR_OK
                                                                                       : PULSAR_EHIP;
}

// Scratch of pulsar_phase2_query_noalloc: the workspace of the Phase-2 query
// (rotated query, rotated self keys, d-major self values) in one fixed device
// array, so that the call allocates nothing.  Each device holds its own copy at
// its own address; in host code `scratch` names a host-side stand-in, so kernels
// are only ever given the device address hipGetSymbolAddress returns, looked up
// once per device (with that device current) and kept.  Every call on a device
// shares that device's array: calls that overlap on one device race.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_dev[kMaxDevices];

int noalloc_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PULSAR_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PULSAR_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PULSAR_EHIP;
    g_scratch_dev[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_dev[dev];
  return PULSAR_OK;
}

}  // namespace

extern "C" {

int pulsar_phase1_prepare(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const int32_t* sel,
                          uint16_t* k_cache, uint16_t* v_cache, void* ws, size_t ws_bytes,
                          void* stream) {
  P1Ws w;
  int rc = phase1_common(g, a, k_cache, v_cache, ws, ws_bytes, &w);
  if (rc) return rc;
  rc = prepare_pointers_ok(g, q, k, v, sel);
  if (rc) return rc;
  return phase1_prepare_checked(g, a, q, k, v, sel, k_cache, v_cache, w, as_stream(stream));
}

int pulsar_phase1_attend(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* k_cache,
                         const uint16_t* v_cache, float* o, void* ws, size_t ws_bytes,
                         void* stream) {
  P1Ws w;
  int rc = phase1_common(g, a, k_cache, v_cache, ws, ws_bytes, &w);
  if (rc) return rc;
  if (!aligned16(o)) return PULSAR_EINVAL;
  return launch_phase1_attend(w.pg, w.q_rot, k_cache, v_cache, w.lists, w.order, o,
                              as_stream(stream))
             ? PULSAR_EHIP
             : PULSAR_OK;
}

int pulsar_phase1_encode(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const int32_t* sel, float* o,
                         uint16_t* k_cache, uint16_t* v_cache, void* ws, size_t ws_bytes,
                         void* stream) {
  P1Ws w;
  int rc = phase1_common(g, a, k_cache, v_cache, ws, ws_bytes, &w);
  if (rc) return rc;
  rc = prepare_pointers_ok(g, q, k, v, sel);
  if (rc) return rc;
  if (!aligned16(o)) return PULSAR_EINVAL;
  const hipStream_t s = as_stream(stream);
  rc = phase1_prepare_checked(g, a, q, k, v, sel, k_cache, v_cache, w, s);
  if (rc) return rc;
  return launch_phase1_attend(w.pg, w.q_rot, k_cache, v_cache, w.lists, w.order, o, s)
             ? PULSAR_EHIP
             : PULSAR_OK;
}

int64_t pulsar_prefix_rows_len(const pulsar_geom* g) {
  if (check_geom(g) != PULSAR_OK) return -1;
  Phase1Geometry pg = phase1_geometry(g->n_blocks, g->block_size, g->chunk_size, kept_chunks(g),
                                      g->sink_size, 1, 1, 64);
  return phase1_prefix_rows_len(pg);
}

int pulsar_phase1_prefix_rows(const pulsar_geom* g, const pulsar_attn* a,
                              const uint16_t* k_cache, const uint16_t* v_cache, float* o_prefix,
                              void* ws, size_t ws_bytes, void* stream) {
  P1Ws w;
  int rc = phase1_common(g, a, k_cache, v_cache, ws, ws_bytes, &w);
  if (rc) return rc;
  if (phase1_prefix_rows_len(w.pg) == 0) return PULSAR_OK;
  if (!aligned16(o_prefix)) return PULSAR_EINVAL;
  return launch_phase1_prefix_rows(w.pg, w.q_rot, k_cache, v_cache, w.lists, o_prefix,
                                   as_stream(stream))
             ? PULSAR_EHIP
             : PULSAR_OK;
}

int32_t pulsar_phase2_num_parts(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                                int32_t shard_len, int32_t q_len, int32_t has_self) {
  if (check_attn(a) != PULSAR_OK) return PULSAR_EINVAL;
  if (batch < 1 || n_shards < 0 || q_len < 1) return PULSAR_EINVAL;
  if (n_shards > 0 && shard_len < 1) return PULSAR_EINVAL;
  if (n_shards == 0 && !has_self) return PULSAR_EINVAL;
  Phase2Geometry pg = phase2_geometry(batch, n_shards, n_shards > 0 ? shard_len : 1, q_len,
                                      a->n_q_heads, a->n_kv_heads, a->head_dim, has_self);
  return pg.n_parts;
}

size_t pulsar_phase2_workspace_bytes(const pulsar_attn* a, int32_t batch, int32_t q_len,
                                     int32_t has_self) {
  if (check_attn(a) != PULSAR_OK || batch < 1 || q_len < 1) return 0;
  Phase2Geometry pg = phase2_geometry(batch, 1, 1, q_len, a->n_q_heads, a->n_kv_heads,
                                      a->head_dim, has_self);
  return layout2(pg).total;
}

int pulsar_phase2_query(const pulsar_attn* a, int32_t batch, int32_t n_shards, int32_t shard_len,
                        const uint16_t* qq, int32_t q_len, int64_t q_pos0,
                        const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_self,
                        const uint16_t* v_self, float* o_part, float* lse_part, int32_t n_parts,
                        void* ws, size_t ws_bytes, void* stream) {
  Phase2Geometry pg;
  int rc = phase2_query_checked(a, batch, n_shards, shard_len, qq, q_len, q_pos0, k_cache,
                                v_cache, k_self, v_self, o_part, lse_part, n_parts, &pg);
  if (rc) return rc;
  if (!ws || ws_bytes < layout2(pg).total) return PULSAR_EWORKSPACE;
  if (!aligned16(ws)) return PULSAR_EINVAL;
  return phase2_query_launch(a, pg, qq, q_pos0, k_cache, v_cache, k_self, v_self, o_part,
                             lse_part, static_cast<char*>(ws), as_stream(stream));
}

int pulsar_phase2_query_noalloc(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                                int32_t shard_len, const uint16_t* qq, int32_t q_len,
                                int64_t q_pos0, const uint16_t* k_cache, const uint16_t* v_cache,
                                const uint16_t* k_self, const uint16_t* v_self, float* o_part,
                                float* lse_part, int32_t n_parts, void* stream) {
  Phase2Geometry pg;
  int rc = phase2_query_checked(a, batch, n_shards, shard_len, qq, q_len, q_pos0, k_cache,
                                v_cache, k_self, v_self, o_part, lse_part, n_parts, &pg);
  if (rc) return rc;
  if (layout2(pg).total > kNoAllocScratchBytes) return PULSAR_EUNSUPPORTED;
  char* w = nullptr;
  rc = noalloc_scratch(&w);
  if (rc) return rc;
  return phase2_query_launch(a, pg, qq, q_pos0, k_cache, v_cache, k_self, v_self, o_part,
                             lse_part, w, as_stream(stream));
}

size_t pulsar_phase2_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int pulsar_self_append(const pulsar_attn* a, int32_t batch, int32_t cap, int32_t n_self,
                       int32_t n_new, int64_t self_pos0, const uint16_t* k_new,
                       const uint16_t* v_new, uint16_t* k_self_cache, uint16_t* v_self_cache,
                       void* stream) {
  if (check_attn(a) != PULSAR_OK) return check_attn(a);
  if (batch < 1 || n_new < 1 || n_self < 0 || cap < 8 || self_pos0 < 0) return PULSAR_EINVAL;
  if (cap % 8 != 0) return PULSAR_EUNSUPPORTED;   // values are read in runs of 8 tokens
  if ((int64_t)n_self + n_new > cap) return PULSAR_EINVAL;
  if ((int64_t)batch * n_new > INT32_MAX / 2) return PULSAR_EUNSUPPORTED;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_self_cache) || !aligned16(v_self_cache))
    return PULSAR_EINVAL;
  return launch_self_append(k_new, v_new, batch, n_new, n_self, cap, a->n_kv_heads, a->head_dim,
                            self_pos0, a->rope_base, a->rope_scaling, k_self_cache, v_self_cache,
                            as_stream(stream)) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

int pulsar_phase2_decode(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                         int32_t shard_len, const uint16_t* qq, int32_t q_len,
                         const uint16_t* k_cache, const uint16_t* v_cache,
                         const uint16_t* k_self_cache, const uint16_t* v_self_cache, int32_t cap,
                         int32_t n_self, int64_t self_pos0, float* o_part, float* lse_part,
                         int32_t n_parts, void* ws, size_t ws_bytes, void* stream) {
  const int32_t want = pulsar_phase2_num_parts(a, batch, n_shards, shard_len, q_len, 1);
  if (want <= 0) return want < 0 ? want : PULSAR_EINVAL;
  if (n_parts != want) return PULSAR_EINVAL;
  if (q_len > n_self || n_self > cap || cap < 8 || self_pos0 < 0) return PULSAR_EINVAL;
  if (cap % 8 != 0) return PULSAR_EUNSUPPORTED;
  if (!aligned16(qq) || !aligned16(o_part) || !lse_part || !aligned16(k_self_cache) ||
      !aligned16(v_self_cache))
    return PULSAR_EINVAL;
  if (n_shards > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) return PULSAR_EINVAL;
  if (n_shards > 0 && shard_len % 8 != 0) return PULSAR_EUNSUPPORTED;
  if ((int64_t)batch * n_shards * shard_len * a->n_kv_heads > INT32_MAX) return PULSAR_EUNSUPPORTED;
  if ((int64_t)shard_len * a->head_dim * 2 > UINT32_MAX) return PULSAR_EUNSUPPORTED;  // slab bytes
  if ((int64_t)batch * q_len > INT32_MAX / 2) return PULSAR_EUNSUPPORTED;
  Phase2Geometry pg = phase2_geometry(batch, n_shards, n_shards > 0 ? shard_len : 1, q_len,
                                      a->n_q_heads, a->n_kv_heads, a->head_dim, 1);
  if (!phase2_grid_ok(pg)) return PULSAR_EUNSUPPORTED;
  const Layout2 l = layout2(pg);
  if (!ws || ws_bytes < l.k_rot) return PULSAR_EWORKSPACE;   // the rotated query only
  if (!aligned16(ws)) return PULSAR_EINVAL;
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + l.q_rot);
  hipStream_t s = as_stream(stream);
  // query token t is self token n_self - q_len + t
  const int64_t q_pos0 = self_pos0 + n_self - q_len;
  // The decode form rotates the query rows inside the attention launch; other
  // shapes rotate them into the workspace first.
  const bool rotate_inside = phase2_decode_form(pg);
  if (!rotate_inside &&
      launch_phase2_prep(qq, nullptr, nullptr, batch, q_len, a->n_q_heads, a->n_kv_heads,
                         a->head_dim, q_pos0, a->rope_base, a->rope_scaling, 8, q_rot, nullptr,
                         nullptr, s))
    return PULSAR_EHIP;
  const RawQuery raw{qq, q_pos0, a->rope_base, a->rope_scaling};
  SelfShard self{};
  self.k = k_self_cache;
  self.v = v_self_cache;
  self.k_seq = (int64_t)cap * a->n_kv_heads * a->head_dim;
  self.v_seq = (int64_t)a->n_kv_heads * a->head_dim * cap;
  self.n = n_self;
  self.v_ld = cap;
  return launch_phase2(pg, q_rot, k_cache, v_cache, self, o_part, lse_part, s,
                       rotate_inside ? &raw : nullptr) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

size_t pulsar_decode_step_workspace_bytes(const pulsar_attn* a, int32_t batch, int32_t q_len) {
  if (check_attn(a) != PULSAR_OK || batch < 1 || q_len < 1) return 0;
  Phase2Geometry pg = phase2_geometry(batch, 1, 1, q_len, a->n_q_heads, a->n_kv_heads,
                                      a->head_dim, 1);
  // the rotated query, for shapes that rotate it outside the attention launch
  return layout2(pg).k_rot;
}

int pulsar_decode_step(const pulsar_attn* a, int32_t batch, int32_t n_shards, int32_t shard_len,
                       const uint16_t* qq, const uint16_t* k_new, const uint16_t* v_new,
                       int32_t q_len, const uint16_t* k_cache, const uint16_t* v_cache,
                       uint16_t* k_self_cache, uint16_t* v_self_cache, int32_t cap,
                       int32_t n_self, int64_t self_pos0, float* o_part, float* lse_part,
                       int32_t n_parts, float* o, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  if (check_attn(a) != PULSAR_OK) return check_attn(a);
  if (q_len < 1 || n_self < 0 || (int64_t)n_self + q_len > cap) return PULSAR_EINVAL;
  const int32_t want = pulsar_phase2_num_parts(a, batch, n_shards, shard_len, q_len, 1);
  if (want <= 0) return want < 0 ? want : PULSAR_EINVAL;
  if (n_parts != want || cap < 8 || self_pos0 < 0) return PULSAR_EINVAL;
  if (cap % 8 != 0) return PULSAR_EUNSUPPORTED;
  if (!aligned16(qq) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(o_part) ||
      !lse_part || !aligned16(k_self_cache) || !aligned16(v_self_cache) || !aligned16(o))
    return PULSAR_EINVAL;
  if (n_shards > 0 && (!aligned16(k_cache) || !aligned16(v_cache))) return PULSAR_EINVAL;
  if (n_shards > 0 && shard_len % 8 != 0) return PULSAR_EUNSUPPORTED;
  if ((int64_t)batch * n_shards * shard_len * a->n_kv_heads > INT32_MAX) return PULSAR_EUNSUPPORTED;
  if ((int64_t)shard_len * a->head_dim * 2 > UINT32_MAX) return PULSAR_EUNSUPPORTED;  // slab bytes
  if ((int64_t)batch * q_len > INT32_MAX / 2) return PULSAR_EUNSUPPORTED;
  if ((int64_t)q_len * a->n_q_heads > INT32_MAX) return PULSAR_EUNSUPPORTED;
  const int32_t n_after = n_self + q_len;
  Phase2Geometry pg = phase2_geometry(batch, n_shards, n_shards > 0 ? shard_len : 1, q_len,
                                      a->n_q_heads, a->n_kv_heads, a->head_dim, 1);
  if (!phase2_grid_ok(pg)) return PULSAR_EUNSUPPORTED;
  if (!ws || ws_bytes < pulsar_decode_step_workspace_bytes(a, batch, q_len)) return PULSAR_EWORKSPACE;
  if (!aligned16(ws)) return PULSAR_EINVAL;
  hipStream_t s = as_stream(stream);
  const int64_t q_pos0 = self_pos0 + n_self;   // the new tokens are the queries
  SelfShard self{};
  self.k = k_self_cache;
  self.v = v_self_cache;
  self.k_seq = (int64_t)cap * a->n_kv_heads * a->head_dim;
  self.v_seq = (int64_t)a->n_kv_heads * a->head_dim * cap;
  self.n = n_after;
  self.v_ld = cap;
  if (phase2_decode_form(pg) && q_len <= 32) {
    // the attention launch appends the new tokens itself, then the merge
    const RawQuery raw{qq, q_pos0, a->rope_base, a->rope_scaling};
    const FusedStep step{k_new, v_new, k_self_cache, v_self_cache};
    if (launch_phase2(pg, nullptr, k_cache, v_cache, self, o_part, lse_part, s, &raw, &step))
      return PULSAR_EHIP;
    return launch_merge(batch, n_parts, q_len, a->n_q_heads, a->head_dim, o_part, lse_part, o,
                        lse, s) == 0
               ? PULSAR_OK
               : PULSAR_EHIP;
  }
  // other shapes: append, rotate the query, attend, merge
  if (launch_self_append(k_new, v_new, batch, q_len, n_self, cap, a->n_kv_heads, a->head_dim,
                         self_pos0, a->rope_base, a->rope_scaling, k_self_cache, v_self_cache, s))
    return PULSAR_EHIP;
  uint16_t* q_rot = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + layout2(pg).q_rot);
  if (launch_phase2_prep(qq, nullptr, nullptr, batch, q_len, a->n_q_heads, a->n_kv_heads,
                         a->head_dim, q_pos0, a->rope_base, a->rope_scaling, 8, q_rot, nullptr,
                         nullptr, s))
    return PULSAR_EHIP;
  if (launch_phase2(pg, q_rot, k_cache, v_cache, self, o_part, lse_part, s)) return PULSAR_EHIP;
  return launch_merge(batch, n_parts, q_len, a->n_q_heads, a->head_dim, o_part, lse_part, o, lse,
                      s) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

int pulsar_lse_merge(int32_t batch, int32_t n_parts, int32_t q_len, int32_t n_q_heads,
                     int32_t head_dim, const float* o_part, const float* lse_part, float* o,
                     float* lse, void* stream) {
  if (batch < 1 || n_parts < 1 || q_len < 1 || n_q_heads < 1) return PULSAR_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PULSAR_EUNSUPPORTED;
  if (!aligned16(o_part) || !lse_part || !aligned16(o)) return PULSAR_EINVAL;
  // rows of one sequence are counted in 32 bits; one wave per row, four rows a workgroup
  if ((int64_t)q_len * n_q_heads > INT32_MAX) return PULSAR_EUNSUPPORTED;
  if ((int64_t)batch * q_len * n_q_heads > (int64_t)INT32_MAX * 4) return PULSAR_EUNSUPPORTED;
  return launch_merge(batch, n_parts, q_len, n_q_heads, head_dim, o_part, lse_part, o, lse,
                      as_stream(stream)) == 0
             ? PULSAR_OK
             : PULSAR_EHIP;
}

const char* pulsar_strerror(int code) {
  switch (code) {
    case PULSAR_OK: return "ok";
    case PULSAR_EINVAL: return "invalid argument (geometry, null or misaligned pointer)";
    case PULSAR_EWORKSPACE: return "workspace missing or too small";
    case PULSAR_EHIP: return "HIP runtime error while launching";
    case PULSAR_EUNSUPPORTED: return "valid request outside what the kernels implement";
    default: return "unknown error code";
  }
}

}  // extern "C"
