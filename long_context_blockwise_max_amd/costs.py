"""Algorithmic work of the hot path: FLOPs and bytes the method itself must
compute or move (not what a particular kernel happens to do).

Phase-1 cost ("Dropping the Anchor ..." Abstract and Table 3: Phase-1 cost
per layer on the critical host).  Attention over an input of n tokens with a
causal mask costs 2 * d * H * n(n+1)/2 multiply-adds for Q.K and the same for
P.V, i.e. 4 d H n(n+1)/2 FLOPs.  Two counts are kept:
  * rows:  only the block's own rows are queries (they see the whole prefix
           plus their own causal part) -- what the encode call computes;
  * host:  every row of [prefix || block] is a query, as a full forward pass
           on one host does -- the basis of the pages' per-host comparison.
"""
from __future__ import annotations


def prefix_len(i: int, sink: int, chunk: int, k: int) -> int:
    """Prefix length of block i: 0 for block 0, sink + chunk * k * i otherwise."""
    return 0 if i == 0 else sink + chunk * k * i


def phase1_flops_rows(n_blocks, block_size, sink, chunk, k, n_q_heads, head_dim) -> float:
    b = block_size
    tot = 0
    for i in range(n_blocks):
        p = prefix_len(i, sink, chunk, k)
        tot += b * p + b * (b + 1) // 2
    return 4.0 * head_dim * n_q_heads * tot


def host_causal_flops(n_tokens, n_q_heads, head_dim) -> float:
    return 4.0 * head_dim * n_q_heads * n_tokens * (n_tokens + 1) / 2


def phase1_flops_hosts(n_blocks, block_size, sink, chunk, k, n_q_heads, head_dim) -> float:
    return sum(host_causal_flops(prefix_len(i, sink, chunk, k) + block_size, n_q_heads, head_dim)
               for i in range(n_blocks))


def critical_host_ratio_star_vs_pulsar(context_len, n_hosts, summary_tokens, sink=64,
                                       n_q_heads=32, head_dim=128) -> float:
    """Phase-1 attention FLOPs on the last (critical) host, Star Attention
    (anchor = a full copy of block 0, input 2b) over Pulsar (sink + one summary
    of `summary_tokens` per earlier block, input b + sink + (n-1) * summary)."""
    b = context_len // n_hosts
    star = host_causal_flops(2 * b, n_q_heads, head_dim)
    pulsar = host_causal_flops(b + sink + (n_hosts - 1) * summary_tokens, n_q_heads, head_dim)
    return star / pulsar


def phase2_flops(batch, q_len, context_len, n_q_heads, head_dim, with_self=True) -> float:
    keys = context_len + ((q_len + 1) / 2 if with_self else 0)
    return 4.0 * head_dim * n_q_heads * q_len * keys * batch


def phase2_bytes(batch, n_shards, shard_len, q_len, n_q_heads, n_kv_heads, head_dim,
                 with_self=True) -> int:
    """Retained K+V (bf16) + query (bf16) + merged output (fp32) + self K/V (bf16)."""
    kv = 2 * 2 * n_shards * n_kv_heads * shard_len * head_dim
    q = 2 * q_len * n_q_heads * head_dim
    o = 4 * q_len * n_q_heads * head_dim
    s = 2 * 2 * q_len * n_kv_heads * head_dim if with_self else 0
    return batch * (kv + q + o + s)


def phase2_kv_bytes(batch, n_shards, shard_len, n_kv_heads, head_dim) -> int:
    return batch * 2 * 2 * n_shards * n_kv_heads * shard_len * head_dim


def phase1_kernel_bytes(n_blocks, block_size, sink, chunk, k, n_q_heads, n_kv_heads,
                        head_dim) -> int:
    """Least bytes the Phase-1 attention launch moves: rotated queries (bf16), the
    block's keys and values (bf16) and each block's prefix keys and values once,
    the prefix index lists (two int32 per entry) and the float32 output."""
    L = n_blocks * block_size
    q = 2 * L * n_q_heads * head_dim
    kv = 2 * 2 * L * n_kv_heads * head_dim
    p = sum(prefix_len(i, sink, chunk, k) for i in range(1, n_blocks))
    pre = 2 * 2 * p * n_kv_heads * head_dim + 2 * 4 * p
    o = 4 * L * n_q_heads * head_dim
    return q + kv + pre + o


def phase2_kernel_bytes(batch, n_shards, shard_len, q_len, n_q_heads, n_kv_heads, head_dim,
                        with_self=True) -> int:
    """Least bytes of the Phase-2 query launch: the method's Phase-2 bytes (retained
    K/V, query, self K/V, merged output); split-KV partials are overhead on top."""
    return phase2_bytes(batch, n_shards, shard_len, q_len, n_q_heads, n_kv_heads, head_dim,
                        with_self)


def prefix_rows_flops(n_rows, n_q_heads, head_dim) -> float:
    """Prefix rows: list entry e attends to entries 0..e, 4 d Hq FLOPs per pair."""
    return 4.0 * head_dim * n_q_heads * n_rows * (n_rows + 1) / 2
