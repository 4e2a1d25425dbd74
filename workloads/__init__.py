"""Seeded synthetic inputs for the Pulsar Attention hot path.

This module only draws random numbers and stores them in the bf16 / int32
representations the kernels and the CPU oracle both consume.  It holds none
of the method's arithmetic (no document frequency, no RoPE, no softmax).

Every tensor is generated block by block from its own child seed, so any
block of any tensor can be regenerated alone (the oracle uses that to check
sampled rows of a 512K-token context without materialising all of it).

Shapes follow the efficiency setting of "Dropping the Anchor: Statistical
Context Summarization for Distributed Systems via Pulsar Attention"
(Section 3 Results, Section 4 Efficiency): Llama-3.1-8B attention geometry
(32 query heads, 8 KV heads, head dim 128), contexts split into 4 blocks up
to 64K and 8 blocks at 128K, a 64-token sink, 32-token chunks and a 12.5 %
summary budget (Section 2.1).  Token IDs are a truncated Zipf(1.1) stream in
place of text; Q/K/V are standard normal in place of model activations.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# child indices of SeedSequence(seed).spawn(...)
_S_TOKENS, _S_PLANT, _S_Q, _S_K, _S_V, _S_QQ, _S_KQ, _S_VQ = range(8)
_N_BASE_STREAMS = 8


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    n_blocks: int
    block_size: int
    sink_size: int
    chunk_size: int
    budget_chunks: int
    vocab_size: int
    n_planted: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    batch: int
    rope_base: float = 500000.0
    zipf_s: float = 1.1
    rope_scaling: int = 0      # 1: Llama-3.1 frequency scaling

    @property
    def context_len(self) -> int:
        return self.n_blocks * self.block_size

    @property
    def n_chunks(self) -> int:
        return self.block_size // self.chunk_size

    @property
    def k_eff(self) -> int:
        return min(self.budget_chunks, self.n_chunks)

    def prefix_len(self, i: int) -> int:
        """Length of block i's gathered prefix (block 0 has none)."""
        if i == 0:
            return 0
        return self.sink_size + self.chunk_size * self.k_eff * i


def budget_chunks_for(block_size: int, chunk_size: int = 32, frac: float = 0.125) -> int:
    """Summary budget of 12.5 % of the block, expressed in whole chunks."""
    return int(block_size * frac) // chunk_size


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4, 1024, 64, 32, 4, 32000, 16, 4, 2, 64, 32, 1),
    "32k": Workload("32k", 2, 4, 8192, 64, 32, 32, 128256, 0, 32, 8, 128, 64, 1),
    "128k": Workload("128k", 3, 8, 16384, 64, 32, 64, 128256, 0, 32, 8, 128, 64, 1),
    # Star Attention anchor baseline: the prefix is a full copy of block 0 and
    # no summaries; same seed, so every tensor equals the 128k one.
    "128k_star": Workload("128k_star", 3, 8, 16384, 16384, 32, 0, 128256, 0, 32, 8, 128, 64, 1),
    "512k": Workload("512k", 5, 16, 32768, 64, 32, 128, 128256, 0, 32, 8, 128, 1, 8),
}


# ----------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ------------------------------------------------------------------- streams
def _children(w: Workload):
    n_extra = 2 * max(0, w.batch - 1)
    return np.random.SeedSequence(w.seed).spawn(_N_BASE_STREAMS + n_extra)


def _block_rng(w: Workload, stream: int, j: int) -> np.random.Generator:
    child = _children(w)[stream]
    return np.random.default_rng(child.spawn(max(w.n_blocks, 1))[j])


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


# -------------------------------------------------------------------- tokens
def zipf_probs(n: int, s: float) -> np.ndarray:
    r = np.arange(1, n + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


def tokens(w: Workload) -> np.ndarray:
    """int32[L]: truncated Zipf(s) ids over the first V - n_planted ids, plus
    n_planted ids (the top of the vocabulary) each planted once, spread evenly
    over the blocks, each in a distinct chunk at a seeded offset."""
    ch = _children(w)
    v_sample = w.vocab_size - w.n_planted
    rng = np.random.default_rng(ch[_S_TOKENS])
    t = rng.choice(v_sample, size=w.context_len, p=zipf_probs(v_sample, w.zipf_s)).astype(np.int32)
    if w.n_planted:
        assert w.n_planted % w.n_blocks == 0
        per = w.n_planted // w.n_blocks
        prng = np.random.default_rng(ch[_S_PLANT])
        for j in range(w.n_blocks):
            cs = prng.choice(w.n_chunks, size=per, replace=False)
            offs = prng.integers(0, w.chunk_size, size=per)
            for m in range(per):
                pos = j * w.block_size + int(cs[m]) * w.chunk_size + int(offs[m])
                t[pos] = v_sample + j * per + m
    return t


def planted_positions(w: Workload) -> np.ndarray:
    t = tokens(w)
    return np.nonzero(t >= w.vocab_size - w.n_planted)[0] if w.n_planted else np.zeros(0, np.int64)


# ----------------------------------------------------------------- Q / K / V
def _heads(w: Workload, which: str) -> int:
    return w.n_q_heads if which == "q" else w.n_kv_heads


def qkv_block(w: Workload, which: str, j: int) -> np.ndarray:
    """uint16 bf16 bits [block_size][H][d] of context tensor `which` ('q','k','v') for block j."""
    stream = {"q": _S_Q, "k": _S_K, "v": _S_V}[which]
    rng = _block_rng(w, stream, j)
    return _normal_bf16(rng, (w.block_size, _heads(w, which), w.head_dim))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def qkv(w: Workload, which: str) -> np.ndarray:
    """uint16 bf16 bits [L][H][d] of the whole context tensor (blocks drawn in parallel)."""
    out = np.empty((w.context_len, _heads(w, which), w.head_dim), np.uint16)

    def fill(j):
        out[j * w.block_size:(j + 1) * w.block_size] = qkv_block(w, which, j)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(w.n_blocks)))
    return out


def extra_cache(w: Workload, seq: int, which: str) -> np.ndarray:
    """Whole retained cache [S][Hkv][b][d] of extra sequence `seq` (shards in parallel)."""
    out = np.empty((w.n_blocks, w.n_kv_heads, w.block_size, w.head_dim), np.uint16)

    def fill(s):
        out[s] = extra_cache_shard(w, seq, which, s)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(w.n_blocks)))
    return out


def query(w: Workload):
    """Phase-2 query-host tensors, pre-RoPE bf16 bits:
    qq [B][Lq][Hq][d], k_self [B][Lq][Hkv][d], v_self [B][Lq][Hkv][d]."""
    ch = _children(w)
    qq = _normal_bf16(np.random.default_rng(ch[_S_QQ]), (w.batch, w.q_len, w.n_q_heads, w.head_dim))
    kq = _normal_bf16(np.random.default_rng(ch[_S_KQ]), (w.batch, w.q_len, w.n_kv_heads, w.head_dim))
    vq = _normal_bf16(np.random.default_rng(ch[_S_VQ]), (w.batch, w.q_len, w.n_kv_heads, w.head_dim))
    return qq, kq, vq


def extra_cache_shard(w: Workload, seq: int, which: str, shard: int) -> np.ndarray:
    """Retained cache of an extra sequence (seq >= 1) for the batched decode
    workload: bf16 bits [Hkv][block_size][d], drawn N(0,1) directly (a rotation
    of an isotropic Gaussian pair has the same distribution, so these stand in
    for post-RoPE keys)."""
    assert 1 <= seq < w.batch
    stream = _N_BASE_STREAMS + 2 * (seq - 1) + (0 if which == "k" else 1)
    child = _children(w)[stream]
    rng = np.random.default_rng(child.spawn(w.n_blocks)[shard])
    return _normal_bf16(rng, (w.n_kv_heads, w.block_size, w.head_dim))


# ------------------------------------------- structured selection token streams
def small_vocab_tokens(seed: int, n_blocks: int, block_size: int, vocab: int) -> np.ndarray:
    """Uniform ids over a small vocabulary, so chunk min-df spreads over 1..N."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 11]))
    return rng.integers(0, vocab, size=n_blocks * block_size, dtype=np.int64).astype(np.int32)


def filler_planted_tokens(seed: int, n_blocks: int, block_size: int, chunk: int,
                          per_block: int, pool: int = 32, vocab: int = 4096):
    """Every block drawn from one small shared pool (each pool id lands in every
    block), plus `per_block` ids unique to each block, each in its own chunk.
    Returns (tokens, planted chunk indices [N][per_block] sorted)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 12]))
    n_chunks = block_size // chunk
    t = np.empty(n_blocks * block_size, np.int32)
    planted = np.zeros((n_blocks, per_block), np.int64)
    for j in range(n_blocks):
        blk = rng.integers(0, pool, size=block_size).astype(np.int32)
        blk[:pool] = np.arange(pool, dtype=np.int32)  # every pool id present in every block
        rng.shuffle(blk)
        cs = np.sort(rng.choice(n_chunks, size=per_block, replace=False))
        for m, c in enumerate(cs):
            blk[c * chunk + int(rng.integers(0, chunk))] = pool + j * per_block + m
        planted[j] = cs
        assert np.unique(blk[blk < pool]).size == pool, "a pool id vanished from a block"
        t[j * block_size:(j + 1) * block_size] = blk
    assert pool + n_blocks * per_block <= vocab
    return t, planted


def with_(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def generated(w: Workload, n_tokens: int):
    """Tokens generated after the query (one per decode step), pre-RoPE bf16 bits:
    q [n][B][1][Hq][d], k [n][B][1][Hkv][d], v [n][B][1][Hkv][d].  Drawn from a
    seed sequence of their own, so the other tensors do not change with n."""
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 0x6E6]))
    q = _normal_bf16(rng, (n_tokens, w.batch, 1, w.n_q_heads, w.head_dim))
    k = _normal_bf16(rng, (n_tokens, w.batch, 1, w.n_kv_heads, w.head_dim))
    v = _normal_bf16(rng, (n_tokens, w.batch, 1, w.n_kv_heads, w.head_dim))
    return q, k, v
