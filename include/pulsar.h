/*
 * pulsar.h -- C ABI of the Pulsar Attention hot path on AMD Instinct MI355X (gfx950).
 *
 * The calls follow the method's own statement of the problem in "Dropping the
 * Anchor: Statistical Context Summarization for Distributed Systems via Pulsar
 * Attention":
 *   pulsar_select         Section 2.1: Max-IDF summary selection from token IDs
 *                         (pulsar_select_method: the ablation's other scores)
 *   pulsar_phase1_encode  Section 2 / 2.1: each block attends over
 *                         [sink || summaries of earlier blocks || own block] at
 *                         original positions and keeps only its own KV
 *   pulsar_phase2_query   Section 2.2: the query attends to every retained shard
 *                         (local attention per shard, partial results out)
 *   pulsar_lse_merge      Section 2.2 and the Star Attention review's distributed
 *                         online-softmax aggregation: exact log-sum-exp merge
 * All "hosts" of the method are one batched launch on one GPU.
 *
 * Conventions shared by every call
 *  - Tensor arguments are DEVICE pointers owned by the caller.  bf16 tensors are
 *    passed as their raw 16-bit patterns (uint16_t).  Layouts are row-major in
 *    the bracketed order.  Every tensor pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on that stream and returns; nothing synchronises the host.
 *  - Return value: PULSAR_OK or a negative PULSAR_E* code.  Arguments are
 *    validated on the host before anything is enqueued, so an error return
 *    means nothing was launched (except PULSAR_EHIP, which reports a launch
 *    error raised after work was enqueued).  No call prints, throws or exits.
 *  - The library allocates no device memory.  Scratch space is the caller's
 *    workspace (size from pulsar_workspace_bytes); calls that share one
 *    workspace must be ordered on one stream.
 *  - Query head h reads KV head h / (n_q_heads / n_kv_heads) (grouped heads).
 *  - RoPE is the rotate-half form with inverse frequencies base^(-2i/d),
 *    angles derived in float64; rotated keys/queries are rounded to bf16.
 */
#ifndef PULSAR_H
#define PULSAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PULSAR_OK 0
#define PULSAR_EINVAL -1      /* bad geometry, null or misaligned pointer */
#define PULSAR_EWORKSPACE -2  /* workspace missing or smaller than required */
#define PULSAR_EHIP -3        /* the HIP runtime reported an error */
#define PULSAR_EUNSUPPORTED -4 /* valid request outside what the kernels implement */

/* Context geometry of one sequence.
 *   n_blocks      N >= 1 blocks ("hosts"), each of block_size tokens; L = N * block_size
 *   block_size    b, a multiple of chunk_size
 *   chunk_size    tokens per chunk (32 is the method's value); a multiple of 8
 *   budget_chunks k chunks kept per block (12.5 % of b is k = b / 256); k >= n_chunks
 *                 keeps every chunk; 0 keeps none (Star Attention's anchor setting)
 *   sink_size     S first tokens of the sequence prepended to every block i > 0;
 *                 a multiple of 8, 0 <= S <= L
 *   vocab_size    V, token ids must lie in [0, V); V <= 1,048,576
 */
typedef struct pulsar_geom {
  int32_t n_blocks;
  int32_t block_size;
  int32_t chunk_size;
  int32_t budget_chunks;
  int32_t sink_size;
  int32_t vocab_size;
} pulsar_geom;

/* Attention geometry.  head_dim 64 or 128; n_q_heads = G * n_kv_heads with the
 * group size G in {1, 2, 4} or a multiple of 8; L * n_kv_heads * head_dim < 2^31.
 * rope_scaling: 0 plain RoPE; 1 the Llama-3.1 frequency scaling (factor 8, low-
 * and high-frequency factors 1 and 4, original context 8192: frequencies with a
 * wavelength under 2048 positions kept, over 8192 divided by 8, blended between),
 * for use with Llama-3.1 weights. */
typedef struct pulsar_attn {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t rope_scaling;   /* 0 or 1 */
  double rope_base;       /* > 1, e.g. 500000 */
} pulsar_attn;

/* Bytes of workspace pulsar_select and pulsar_phase1_encode need for this
 * geometry (one workspace serves both; a == NULL gives the smaller size that
 * pulsar_select alone needs).  The Phase-1 part holds the rotated queries
 * (L * Hq * d bf16), the prefix index lists and the work order.  Returns 0 if
 * the geometry is invalid. */
size_t pulsar_workspace_bytes(const pulsar_geom* g, const pulsar_attn* a);

/* Number of chunks kept per block: min(budget_chunks, block_size / chunk_size). */
int32_t pulsar_kept_chunks(const pulsar_geom* g);

/* Max-IDF summary selection ("Dropping the Anchor ..." Section 2.1, Figure 2).
 * Each block is a document; df(t) = number of blocks containing token t (all N
 * blocks); each chunk is scored by its rarest token, max idf = log(N / min df),
 * so the kernel ranks chunks by the integer min df; the k best chunks of each
 * block (lowest min df, earlier chunk first among equals) are returned in
 * ascending chunk order.
 *   tok          [L] int32 token ids
 *   sel          [N][kept] int32 out: chunk indices within the block, ascending
 *   chunk_min_df [N][n_chunks] int32 out, or NULL
 *   df           [V] int32 out, or NULL
 *   ws           workspace of at least pulsar_workspace_bytes(g, NULL-safe a) bytes;
 *                its first 4 bytes become a status word: 0, or 1 if some token id
 *                was outside [0, V) (such ids are skipped by the count)
 * Errors: PULSAR_EINVAL, PULSAR_EWORKSPACE, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
int pulsar_select(const pulsar_geom* g, const int32_t* tok, int32_t* sel,
                  int32_t* chunk_min_df, int32_t* df, void* ws, size_t ws_bytes,
                  void* stream);

/* Summary selection by another chunk score: the alternatives the Dutch technical
 * summary's ablation compares Max-IDF against ("Dropping the Anchor ..." Section
 * 2.1 contrasts the maximum with the mean).  The output feeds Phase 1 exactly as
 * pulsar_select's does.
 *   PULSAR_SELECT_MAX_IDF   the method's score, as pulsar_select
 *   PULSAR_SELECT_MEAN_IDF  mean over the chunk's tokens of ln(N / df(t)); an id
 *                           outside the vocabulary counts as idf 0 (df = N).
 *                           TF-IDF with term counts within the chunk ranks the same
 *   PULSAR_SELECT_ENTROPY   Shannon entropy of the chunk's token histogram
 *                           (more diverse chunks first)
 *   PULSAR_SELECT_UNIFORM   k chunks per block uniformly at random: chunk c of
 *                           block j is keyed by the SplitMix64 output with counter
 *                           j * n_chunks + c + 1 from `seed` (Steele, Lea and
 *                           Flood, 2014); the k smallest keys are kept
 *   PULSAR_SELECT_EVEN      chunks floor(m * n_chunks / k), m = 0 .. k-1
 * Higher scores win; equal scores go to the earlier chunk, decided exactly (mean
 * IDF and entropy are ranked by integer products over the chunk's positions).
 * Kept chunks are returned in ascending order, k = pulsar_kept_chunks(g).
 *   tok   [L] int32 token ids (not read by UNIFORM and EVEN)
 *   sel   [N][kept] int32 out
 *   seed  UNIFORM only
 *   ws    at least pulsar_workspace_bytes(g, NULL) bytes (it holds 36 bytes of
 *         scratch per chunk for these methods, and for MEAN_IDF the df table and
 *         the per-block vocabulary bitmaps); its first word is the status word,
 *         set to 1 when a token id lies outside [0, vocab_size)
 *         (MAX_IDF, MEAN_IDF and ENTROPY read the ids)
 * Errors: PULSAR_EINVAL (also an unknown method), PULSAR_EWORKSPACE,
 * PULSAR_EUNSUPPORTED (mean IDF with N^chunk >= 2^256, entropy with
 * chunk^chunk >= 2^256), PULSAR_EHIP. */
#define PULSAR_SELECT_MAX_IDF 0
#define PULSAR_SELECT_MEAN_IDF 1
#define PULSAR_SELECT_ENTROPY 2
#define PULSAR_SELECT_UNIFORM 3
#define PULSAR_SELECT_EVEN 4
int pulsar_select_method(const pulsar_geom* g, int32_t method, uint64_t seed, const int32_t* tok,
                         int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* Phase-1 context encoding ("Dropping the Anchor ..." Section 2 and 2.1).
 * Block i > 0 attends over [first S tokens || kept chunks of blocks 0..i-1 in
 * order || own block], causally, every token at its original position; block
 * 0 attends over itself only.  Prefix entries are not de-duplicated.  Only the
 * block rows are queries.  The kept KV is the block's own keys (rotated, bf16)
 * and values.
 *   q        [L][Hq][d] bf16, pre-RoPE
 *   k, v     [L][Hkv][d] bf16, pre-RoPE keys and values
 *   sel      [N][kept] int32 from pulsar_select (ascending within each block)
 *   o        [L][Hq][d] float32 out: attention output of every block row
 *   k_cache  [N][Hkv][b][d] bf16 out: RoPE(k) rounded to bf16
 *   v_cache  [N][Hkv][d][b] bf16 out: v, stored d-major (each value row is a
 *            column), so that the P.V contraction reads it in 16-byte runs
 *   ws       workspace (pulsar_workspace_bytes); ws_bytes its size
 * Errors: PULSAR_EINVAL, PULSAR_EWORKSPACE, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
int pulsar_phase1_encode(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const int32_t* sel,
                         float* o, uint16_t* k_cache, uint16_t* v_cache, void* ws,
                         size_t ws_bytes, void* stream);

/* The two halves of pulsar_phase1_encode, for callers that schedule or time
 * them apart (same arguments, same workspace; encode is prepare then attend on
 * one stream).
 * pulsar_phase1_prepare writes the rotated keys into k_cache, the d-major
 * values into v_cache, and the rotated queries, the prefix index lists
 * (sink and kept chunks of earlier blocks, Section 2.1) and the work order into
 * the workspace.
 * pulsar_phase1_attend runs the attention of every block row over
 * [sink || summaries || own block] from what prepare left in k_cache, v_cache
 * and ws; it must follow a prepare of the same geometry on the same workspace
 * and caches (stream-ordered), which it cannot check.
 * Errors: as pulsar_phase1_encode. */
int pulsar_phase1_prepare(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* q,
                          const uint16_t* k, const uint16_t* v, const int32_t* sel,
                          uint16_t* k_cache, uint16_t* v_cache, void* ws, size_t ws_bytes,
                          void* stream);
int pulsar_phase1_attend(const pulsar_geom* g, const pulsar_attn* a, const uint16_t* k_cache,
                         const uint16_t* v_cache, float* o, void* ws, size_t ws_bytes,
                         void* stream);

/* Prefix rows.  In the method each host runs one forward pass over
 * [prefix_i || B_i] ("Dropping the Anchor ..." Section 2; the Dutch technical
 * summary writes the input as [S_sink || Sigma_0 || ... || Sigma_{i-1} || B_i]),
 * so its prefix rows are queries too; their outputs are what a next layer needs.
 * Every host's prefix is a leading part of the last block's prefix, so one pass
 * over that list gives them all: list entry e (a position p_e, duplicates kept)
 * attends to entries 0 .. e, at original positions.
 * pulsar_prefix_rows_len: the number of rows, sink_size + chunk_size * kept *
 * (n_blocks - 1) for n_blocks >= 2, else 0 (-1 for an invalid geometry).
 * pulsar_phase1_prefix_rows writes o_prefix [rows][Hq][d] float32, row e the
 * output of list entry e; it reads what pulsar_phase1_prepare left in k_cache,
 * v_cache and ws (same geometry, same stream) and does nothing for 0 rows.
 * Errors: as pulsar_phase1_encode. */
int64_t pulsar_prefix_rows_len(const pulsar_geom* g);
int pulsar_phase1_prefix_rows(const pulsar_geom* g, const pulsar_attn* a,
                              const uint16_t* k_cache, const uint16_t* v_cache, float* o_prefix,
                              void* ws, size_t ws_bytes, void* stream);

/* Number of partial results pulsar_phase2_query and pulsar_phase2_decode write
 * per sequence for this shape: the key tiles of every retained shard, in shard
 * order, followed by the self shard's tiles, are cut into this many contiguous
 * ranges of (almost) equal length, so a part may span two shards or a shard and
 * the self shard.  It does not depend on has_self or on the self length, except
 * that with no shard (n_shards = 0, has_self != 0) there is one part.  A part
 * whose keys a query token may not see (the self shard is causal) holds LSE
 * -inf and a zero output for that token.  Returns <= 0 on error. */
int32_t pulsar_phase2_num_parts(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                                int32_t shard_len, int32_t q_len, int32_t has_self);

/* Bytes of workspace pulsar_phase2_query needs (rotated query, rotated self keys
 * and a d-major copy of the self values).  Returns 0 on invalid arguments. */
size_t pulsar_phase2_workspace_bytes(const pulsar_attn* a, int32_t batch, int32_t q_len,
                                     int32_t has_self);

/* Phase-2 query attention over retained shards ("Dropping the Anchor ..."
 * Section 2.2).  Query token t of sequence s sits at position q_pos0 + t.  For
 * every part (a contiguous range of the shards' and the self shard's keys, as
 * pulsar_phase2_num_parts describes) the call writes the softmax-normalised
 * partial output and its log-sum-exp (natural log of sum exp(q.k / sqrt(d))
 * over the part's keys that the token sees).  The self shard holds
 * the query tokens' own keys and values, attended causally (token t sees self
 * keys 0..t); pass k_self = v_self = NULL to attend to the retained shards only.
 *   qq               [B][Lq][Hq][d] bf16, pre-RoPE
 *   k_cache          [B][n_shards][Hkv][shard_len][d] bf16, keys already rotated
 *   v_cache          [B][n_shards][Hkv][d][shard_len] bf16, d-major (the layout
 *                    pulsar_phase1_encode writes); shard_len a multiple of 8
 *   k_self, v_self   [B][Lq][Hkv][d] bf16 pre-RoPE, or both NULL
 *   o_part           [B][n_parts][Lq][Hq][d] float32 out
 *   lse_part         [B][n_parts][Lq][Hq] float32 out
 *   n_parts          must equal pulsar_phase2_num_parts(...) for this shape
 *   ws               workspace of pulsar_phase2_workspace_bytes(...) bytes
 * Errors: PULSAR_EINVAL, PULSAR_EWORKSPACE, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
int pulsar_phase2_query(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                        int32_t shard_len, const uint16_t* qq, int32_t q_len,
                        int64_t q_pos0, const uint16_t* k_cache, const uint16_t* v_cache,
                        const uint16_t* k_self, const uint16_t* v_self, float* o_part,
                        float* lse_part, int32_t n_parts, void* ws, size_t ws_bytes,
                        void* stream);

/* pulsar_phase2_query for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops and harnesses that forbid allocation.
 * Same arguments, results and errors as pulsar_phase2_query, without ws and
 * ws_bytes: the workspace (rotated query, rotated self keys, d-major self values)
 * lives in a fixed device array inside the library, one per device, held until
 * the process ends.  The call allocates and frees nothing.
 *  - Limit: pulsar_phase2_workspace_bytes(a, batch, q_len, has_self) must not
 *    exceed pulsar_phase2_noalloc_max_bytes() (8 MiB: e.g. up to 678 query
 *    tokens with their self shard at 32 query / 8 KV heads, d = 128); larger
 *    requests return PULSAR_EUNSUPPORTED before anything is enqueued.
 *  - The first call on a device (that device current) looks up the array's
 *    device address; PULSAR_EHIP if that fails.
 *  - Every call on one device uses the same array, which keeps the last call's
 *    contents (nothing in it needs clearing: each call writes what it reads).
 *    Calls that overlap on one device -- on different streams, or from several
 *    threads without ordering -- race; order them on one stream. */
int pulsar_phase2_query_noalloc(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                                int32_t shard_len, const uint16_t* qq, int32_t q_len,
                                int64_t q_pos0, const uint16_t* k_cache, const uint16_t* v_cache,
                                const uint16_t* k_self, const uint16_t* v_self, float* o_part,
                                float* lse_part, int32_t n_parts, void* stream);
/* Size in bytes of the fixed array behind pulsar_phase2_query_noalloc. */
size_t pulsar_phase2_noalloc_max_bytes(void);

/* Generation ("Dropping the Anchor ..." Section 2.2, with the generated tokens
 * of Section 5's --tokens_to_generate): the query host keeps its own tokens --
 * the query, then every generated token -- in a self cache, and each new token
 * attends to every retained shard plus, causally, the self cache.
 *
 * pulsar_self_append appends n_new tokens to self caches that hold n_self:
 *   k_new, v_new   [B][n_new][Hkv][d] bf16, pre-RoPE; token j sits at position
 *                  self_pos0 + n_self + j (self_pos0 = position of self token 0)
 *   k_self_cache   [B][cap][Hkv][d] bf16: receives the rotated keys
 *   v_self_cache   [B][Hkv][d][cap] bf16, d-major: receives the values; the
 *                  columns from n_self + n_new up to the next multiple of 8 are
 *                  zeroed (the attention reads values in runs of 8 tokens), so
 *                  these caches must only be written through this call
 *   cap            capacity in tokens, a multiple of 8; n_self + n_new <= cap
 * Errors: PULSAR_EINVAL, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
int pulsar_self_append(const pulsar_attn* a, int32_t batch, int32_t cap, int32_t n_self,
                       int32_t n_new, int64_t self_pos0, const uint16_t* k_new,
                       const uint16_t* v_new, uint16_t* k_self_cache, uint16_t* v_self_cache,
                       void* stream);

/* Phase-2 attention of the last q_len self tokens (1 <= q_len <= n_self; one
 * generated token per step is q_len = 1).  Query token t is self token
 * n_self - q_len + t, at position self_pos0 + n_self - q_len + t; it attends to
 * every key of the retained shards and to self tokens 0 .. n_self - q_len + t.
 * Writes partials exactly as pulsar_phase2_query with a self shard (the self
 * cache's tiles follow the shards' in the parts), to be merged with
 * pulsar_lse_merge.
 *   qq                 [B][q_len][Hq][d] bf16, pre-RoPE
 *   k_cache, v_cache   retained shards, as in pulsar_phase2_query
 *   k_self_cache, v_self_cache, cap   filled by pulsar_self_append, n_self tokens
 *   n_parts            pulsar_phase2_num_parts(a, batch, n_shards, shard_len, q_len, 1)
 *   ws                 at least pulsar_phase2_workspace_bytes(a, batch, q_len, 0) bytes
 * Errors: PULSAR_EINVAL, PULSAR_EWORKSPACE, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
int pulsar_phase2_decode(const pulsar_attn* a, int32_t batch, int32_t n_shards,
                         int32_t shard_len, const uint16_t* qq, int32_t q_len,
                         const uint16_t* k_cache, const uint16_t* v_cache,
                         const uint16_t* k_self_cache, const uint16_t* v_self_cache, int32_t cap,
                         int32_t n_self, int64_t self_pos0, float* o_part, float* lse_part,
                         int32_t n_parts, void* ws, size_t ws_bytes, void* stream);

/* One generation step as one call ("Dropping the Anchor ..." Section 2.2; the
 * generated tokens of Section 5's --tokens_to_generate): the q_len new tokens
 * are appended to the self caches, their queries attend to every retained shard
 * and, causally, the self cache, and the parts are merged.  The same results,
 * bit for bit, as pulsar_self_append (n_new = q_len) followed by
 * pulsar_phase2_decode (n_self + q_len self tokens) and pulsar_lse_merge.  For
 * one-token steps (every query row of a KV head in one wave, q_len <= 32) the
 * attention launch appends the new tokens itself, so the step is two launches
 * (attention, merge) instead of three.
 *   qq, k_new, v_new     [B][q_len][H][d] bf16, pre-RoPE: the new tokens, at
 *                        positions self_pos0 + n_self + t
 *   k_self_cache, v_self_cache, cap   as for pulsar_self_append; they hold n_self
 *                        tokens before the call and n_self + q_len after it
 *   o_part, lse_part     [B][n_parts][q_len][Hq][d] / [B][n_parts][q_len][Hq]
 *                        float32 scratch for the partials
 *   n_parts              pulsar_phase2_num_parts(a, batch, n_shards, shard_len, q_len, 1)
 *   o, lse               [B][q_len][Hq][d], [B][q_len][Hq] float32 out (lse may be NULL)
 *   ws                   pulsar_decode_step_workspace_bytes(a, batch, q_len) bytes
 * Errors: PULSAR_EINVAL, PULSAR_EWORKSPACE, PULSAR_EUNSUPPORTED, PULSAR_EHIP. */
size_t pulsar_decode_step_workspace_bytes(const pulsar_attn* a, int32_t batch, int32_t q_len);
int pulsar_decode_step(const pulsar_attn* a, int32_t batch, int32_t n_shards, int32_t shard_len,
                       const uint16_t* qq, const uint16_t* k_new, const uint16_t* v_new,
                       int32_t q_len, const uint16_t* k_cache, const uint16_t* v_cache,
                       uint16_t* k_self_cache, uint16_t* v_self_cache, int32_t cap,
                       int32_t n_self, int64_t self_pos0, float* o_part, float* lse_part,
                       int32_t n_parts, float* o, float* lse, void* ws, size_t ws_bytes,
                       void* stream);

/* Exact log-sum-exp merge of partial attention results (the Star Attention
 * review's corrected update: weight exp(s_h - s_global) on the normalised A_h):
 *   lse = ln sum_p exp(lse_part[p]),  o = sum_p exp(lse_part[p] - lse) * o_part[p]
 *   o_part [B][n_parts][Lq][Hq][d] float32, lse_part [B][n_parts][Lq][Hq] float32
 *   o      [B][Lq][Hq][d] float32 out, lse [B][Lq][Hq] float32 out (may be NULL)
 * Errors: PULSAR_EINVAL (a size below 1, a null or misaligned pointer),
 * PULSAR_EUNSUPPORTED (d other than 64 or 128, Lq * Hq above 2^31 - 1, or
 * B * Lq * Hq above 4 (2^31 - 1)), PULSAR_EHIP. */
int pulsar_lse_merge(int32_t batch, int32_t n_parts, int32_t q_len, int32_t n_q_heads,
                     int32_t head_dim, const float* o_part, const float* lse_part, float* o,
                     float* lse, void* stream);

/* Static description of an error code. */
const char* pulsar_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* PULSAR_H */
