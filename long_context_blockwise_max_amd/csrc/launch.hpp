// Internal launchers (host side) behind the C ABI.  Each returns 0 or -3
// (a HIP launch error).  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pulsar {

// chunk_score [N][n_chunks]: receives every chunk's min df (the caller's
// chunk_min_df output or workspace scratch); df [V] (output or scratch); scratch: bits
// [N][ceil(V / 32)] words
int launch_select(const int32_t* tok, int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                  int32_t kept, int32_t vocab, int32_t* sel, int32_t* chunk_score, int32_t* df,
                  uint32_t* bits, int32_t* status, hipStream_t stream);

// method 1 mean IDF, 2 entropy, 3 uniform (seeded), 4 evenly spaced.  Scratch:
// df [vocab] and bits [N][ceil(V / 32)] words (mean IDF), keys [N][n_chunks][8]
// (16-byte aligned), ranks [N][n_chunks]; status[0] is cleared and flags
// out-of-range ids
int launch_select_method(int32_t method, uint64_t seed, const int32_t* tok, int32_t n_blocks,
                         int32_t block_size, int32_t chunk_size, int32_t kept, int32_t vocab,
                         int32_t* sel, int32_t* df, uint32_t* bits, uint32_t* keys,
                         int32_t* ranks, int32_t* status, hipStream_t stream);

int launch_rope_fill(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t L,
                     int32_t block_size, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     double rope_base, int32_t scaling, uint16_t* q_rot, uint16_t* k_cache,
                     uint16_t* v_cache, hipStream_t stream);

// Phase-2 prep: q_rot [B][Lq][Hq][d] and k_rot [B][Lq][Hkv][d] rotated at positions
// pos0 + t; v_t the d-major self values [B][Hkv][d][lq_pad].  k_self == NULL: no self shard
// (k_rot, v_self and v_t unused)
int launch_phase2_prep(const uint16_t* qq, const uint16_t* k_self, const uint16_t* v_self,
                       int32_t batch, int32_t q_len, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t head_dim, int64_t pos0, double rope_base, int32_t scaling,
                       int32_t lq_pad, uint16_t* q_rot, uint16_t* k_rot, uint16_t* v_t,
                       hipStream_t stream);

struct Phase1Geometry {
  int32_t n_blocks, block_size, chunk_size, kept, sink_size;
  int32_t n_q_heads, n_kv_heads, head_dim;
  int32_t heads_per_wg, n_head_sub, rows_per_wg, n_row_tiles;
};
Phase1Geometry phase1_geometry(int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                               int32_t kept, int32_t sink_size, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim);

// total number of prefix entries over all blocks (the prefix index list length)
int64_t phase1_prefix_total(const Phase1Geometry& g);

// work order of the (block, row tile) pairs and the prefix index lists
// (prefix_rows holds 2 * phase1_prefix_total entries: key rows, then value columns)
int launch_phase1_lists(const Phase1Geometry& g, const int32_t* sel, int32_t* prefix_rows,
                        int32_t* order, hipStream_t stream);

// the attention kernel proper; reads what launch_rope_fill and launch_phase1_lists wrote
int launch_phase1_attend(const Phase1Geometry& g, const uint16_t* q_rot, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* prefix_rows,
                         const int32_t* order, float* o, hipStream_t stream);

// number of prefix rows: the last block's prefix length (0 for one block)
int64_t phase1_prefix_rows_len(const Phase1Geometry& g);

// attention output of every prefix row, o_prefix [P][Hq][d]; reads what
// launch_rope_fill and launch_phase1_lists wrote
int launch_phase1_prefix_rows(const Phase1Geometry& g, const uint16_t* q_rot,
                              const uint16_t* k_cache, const uint16_t* v_cache,
                              const int32_t* prefix_rows, float* o_prefix, hipStream_t stream);

struct Phase2Geometry {
  int32_t batch, n_shards, shard_len, q_len, n_q_heads, n_kv_heads, head_dim;
  int32_t has_self, nq, n_row_groups, splits, n_parts, self_pad;
};
Phase2Geometry phase2_geometry(int32_t batch, int32_t n_shards, int32_t shard_len,
                               int32_t q_len, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t has_self);

// The query host's own shard: n tokens (the Lq queries are the last Lq of them).
// Keys rotated, token j of sequence b at k + b * k_seq + j * Hkv * d; values
// d-major, the (b, head, d) row at v + b * v_seq + (head * d + d) * v_ld, with
// columns n .. round_up(n, 8) - 1 finite.  k == nullptr: no self shard.
struct SelfShard {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_seq, v_seq;
  int32_t n, v_ld;
};

// Pre-RoPE query rows for the kernel to rotate itself (token t at pos0 + t).
struct RawQuery {
  const uint16_t* q;
  int64_t pos0;
  double base;
  int32_t scaling;
};

// true when the launch takes the decode form: every query row of a KV head fits
// one 32-row wave (at most 32 query tokens)
bool phase2_decode_form(const Phase2Geometry& g);

// The append of a generation step folded into the decode-form launch: the query
// tokens are the last lq self tokens, and the launch appends them itself before
// it stages any tile (k_new / v_new [B][lq][Hkv][d] pre-RoPE into the self
// caches k_self [B][cap][Hkv][d] and d-major v_self [B][Hkv][d][cap]).
struct FusedStep {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_self;
  uint16_t* v_self;
};

// q_rot [B][Lq][Hq][d] already rotated; or raw != nullptr (decode form only):
// the kernel rotates raw->q [B][Lq][Hq][d] itself and q_rot is not read.
// step != nullptr (needs raw): the append above in the same launch.
int launch_phase2(const Phase2Geometry& g, const uint16_t* q_rot, const uint16_t* k_cache,
                  const uint16_t* v_cache, const SelfShard& self, float* o_part,
                  float* lse_part, hipStream_t stream, const RawQuery* raw = nullptr,
                  const FusedStep* step = nullptr);

// Append n_new tokens to self caches of capacity cap holding n_self tokens:
// k_new / v_new [B][n_new][Hkv][d] pre-RoPE, token j at position pos0 + n_self + j;
// k_cache [B][cap][Hkv][d] receives the rotated keys, v_cache [B][Hkv][d][cap] the
// values (d-major); columns past the last token up to the next multiple of 8 are
// zeroed.
int launch_self_append(const uint16_t* k_new, const uint16_t* v_new, int32_t batch,
                       int32_t n_new, int32_t n_self, int32_t cap, int32_t n_kv_heads,
                       int32_t head_dim, int64_t pos0, double rope_base, int32_t scaling,
                       uint16_t* k_cache, uint16_t* v_cache, hipStream_t stream);

int launch_merge(int32_t batch, int32_t n_parts, int32_t q_len, int32_t n_q_heads,
                 int32_t head_dim, const float* o_part, const float* lse_part, float* o,
                 float* lse, hipStream_t stream);

}  // namespace pulsar
