// Internal launchers (host side) behind the C ABI.  Each returns 0 or -3
// (a HIP launch error).  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pulsar {

int launch_select(const int32_t* tok, int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                  int32_t kept, int32_t vocab, int32_t* sel, int32_t* chunk_min_df, int32_t* df,
                  int32_t* status, hipStream_t stream);

int launch_rope_fill(const uint16_t* k, const uint16_t* v, int64_t L, int32_t block_size,
                     int32_t n_kv_heads, int32_t head_dim, double rope_base, float* rope_cs,
                     uint16_t* k_cache, uint16_t* v_cache, hipStream_t stream);

struct Phase1Geometry {
  int32_t n_blocks, block_size, chunk_size, kept, sink_size;
  int32_t n_q_heads, n_kv_heads, head_dim;
  int32_t heads_per_wg, n_head_sub, rows_per_wg, n_row_tiles;
};
Phase1Geometry phase1_geometry(int32_t n_blocks, int32_t block_size, int32_t chunk_size,
                               int32_t kept, int32_t sink_size, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim);

int launch_phase1(const Phase1Geometry& g, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* sel, const float* rope_cs,
                  int32_t* order, float* o, hipStream_t stream);

struct Phase2Geometry {
  int32_t batch, n_shards, shard_len, q_len, n_q_heads, n_kv_heads, head_dim;
  int32_t has_self, nq, n_row_groups, splits, n_parts;
};
Phase2Geometry phase2_geometry(int32_t batch, int32_t n_shards, int32_t shard_len,
                               int32_t q_len, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t has_self);

int launch_phase2(const Phase2Geometry& g, const uint16_t* qq, int64_t q_pos0,
                  const uint16_t* k_cache, const uint16_t* v_cache, const uint16_t* k_self,
                  const uint16_t* v_self, double rope_base, float* o_part, float* lse_part,
                  hipStream_t stream);

int launch_merge(int32_t batch, int32_t n_parts, int32_t q_len, int32_t n_q_heads,
                 int32_t head_dim, const float* o_part, const float* lse_part, float* o,
                 float* lse, hipStream_t stream);

}  // namespace pulsar
