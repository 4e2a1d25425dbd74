"""Other ways to pick each block's summary chunks (test infrastructure only).

"Dropping the Anchor ..." Section 2.1 contrasts the maximum with the mean: it
takes the maximum IDF over a chunk's tokens because averaging divides a single
rare token's signal by the chunk length.  The Dutch technical summary lists the
alternatives its ablation beat: TF-IDF, BM25, entropy and uniform sampling; the
project page adds evenly spaced chunks.  Only the mean is defined on the pages;
the rest follow named textbook definitions:

  mean_idf  the mean over the chunk's tokens of idf(t) = ln(N / df(t)), with df
            as for Max-IDF (an id outside the vocabulary counts as a token of
            every block, idf 0).  Higher is better.
  entropy   the Shannon entropy of the chunk's token histogram,
            H = -sum_v (c_v / C) ln(c_v / C) over the distinct ids v with counts
            c_v in a chunk of C tokens.  Higher (more diverse) is better.
  uniform   a uniformly random k-subset per block: every chunk gets the
            SplitMix64 output with counter j * n_chunks + c + 1 (Steele, Lea and
            Flood, "Fast splittable pseudorandom number generators", 2014) from
            the caller's seed, and the k smallest outputs are kept.
  even      chunks floor(m * n_chunks / k) for m = 0 .. k-1.

TF-IDF with term counts taken within the chunk is the mean IDF times the chunk
length (sum over distinct terms of tf * idf = sum over positions of idf), so it
ranks exactly as mean_idf.  BM25 scores documents against a query, which the
query-free selection does not have.

As for Max-IDF, ties go to the earlier chunk and the kept chunks are returned in
ascending order; with k >= n_chunks every chunk is kept.

The exact output sequence of `splitmix64` is pinned by the generator's
published known-answer values (the first outputs from one seed and the float
bucket counts of 100,000 outputs from another, as the Rosetta Code task
"Pseudo-random numbers/Splitmix64" states them); the statistical pins fix what
the uniform method needs from it (every chunk kept with probability k / C,
seeds that repeat and differ, balanced and uncorrelated bits).

Exact ranking: mean_idf = ln N - (1/C) ln prod_pos df(t_pos), and
H = ln C - (1/C) ln prod_v c_v^c_v = ln C - (1/C) ln prod_pos c(t_pos), where
c(t_pos) is the count of the token at that position within its chunk.  Both
scores fall as an integer product over the chunk's positions rises, so the
chunks are ordered by those products, computed exactly with Python integers;
equal scores are equal products.
"""
import numpy as np

from .selection import document_frequency

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed, n):
    """The n-th output (n >= 1) of SplitMix64 started from `seed`: the state
    advances by the golden gamma per output and goes through the variant-13
    finaliser."""
    z = (seed + n * GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _keep_smallest(keys, k):
    """Indices of the k smallest keys (ties: lower index first), ascending."""
    order = sorted(range(len(keys)), key=lambda c: (keys[c], c))
    return sorted(order[:min(k, len(keys))])


def mean_idf_scores(tokens, n_blocks, block_size, chunk_size, vocab_size):
    """float64 [N][C] mean idf of each chunk (the definition, for reading)."""
    tokens = np.asarray(tokens)
    df = document_frequency(tokens, n_blocks, block_size, vocab_size)
    n_chunks = block_size // chunk_size
    out = np.empty((n_blocks, n_chunks))
    for j in range(n_blocks):
        for c in range(n_chunks):
            ids = tokens[j * block_size + c * chunk_size:j * block_size + (c + 1) * chunk_size]
            d = [df[t] if 0 <= t < vocab_size else n_blocks for t in ids]
            out[j, c] = np.mean([np.log(n_blocks / x) for x in d])
    return out


def entropy_scores(tokens, n_blocks, block_size, chunk_size):
    """float64 [N][C] Shannon entropy (nats) of each chunk's token histogram."""
    tokens = np.asarray(tokens)
    n_chunks = block_size // chunk_size
    out = np.empty((n_blocks, n_chunks))
    for j in range(n_blocks):
        for c in range(n_chunks):
            ids = tokens[j * block_size + c * chunk_size:j * block_size + (c + 1) * chunk_size]
            _, counts = np.unique(ids, return_counts=True)
            p = counts / chunk_size
            out[j, c] = -np.sum(p * np.log(p))
    return out


def mean_idf_keys(tokens, n_blocks, block_size, chunk_size, vocab_size):
    """Exact order keys of mean_idf: prod over positions of df (smaller = better)."""
    tokens = np.asarray(tokens)
    df = document_frequency(tokens, n_blocks, block_size, vocab_size)
    n_chunks = block_size // chunk_size
    keys = []
    for j in range(n_blocks):
        row = []
        for c in range(n_chunks):
            prod = 1
            for t in tokens[j * block_size + c * chunk_size:j * block_size + (c + 1) * chunk_size]:
                prod *= int(df[t]) if 0 <= t < vocab_size else n_blocks
            row.append(prod)
        keys.append(row)
    return keys


def entropy_keys(tokens, n_blocks, block_size, chunk_size):
    """Exact order keys of entropy: prod over positions of the position's token
    count within the chunk, = prod_v c_v^c_v (smaller = better)."""
    tokens = np.asarray(tokens)
    n_chunks = block_size // chunk_size
    keys = []
    for j in range(n_blocks):
        row = []
        for c in range(n_chunks):
            ids = tokens[j * block_size + c * chunk_size:j * block_size + (c + 1) * chunk_size].tolist()
            prod = 1
            for t in ids:
                prod *= ids.count(t)
            row.append(prod)
        keys.append(row)
    return keys


def uniform_keys(seed, n_blocks, n_chunks):
    return [[splitmix64(seed, j * n_chunks + c + 1) for c in range(n_chunks)]
            for j in range(n_blocks)]


def select_variant(method, tokens, n_blocks, block_size, chunk_size, budget_chunks, vocab_size,
                   seed=0):
    """int64 [N][min(k, C)]: the kept chunks of every block, ascending."""
    n_chunks = block_size // chunk_size
    k = min(budget_chunks, n_chunks)
    if method == "even":
        row = [m * n_chunks // k for m in range(k)] if k > 0 else []
        return np.array([row] * n_blocks, dtype=np.int64).reshape(n_blocks, k)
    if method == "mean_idf":
        keys = mean_idf_keys(tokens, n_blocks, block_size, chunk_size, vocab_size)
    elif method == "entropy":
        keys = entropy_keys(tokens, n_blocks, block_size, chunk_size)
    elif method == "uniform":
        keys = uniform_keys(seed, n_blocks, n_chunks)
    else:
        raise ValueError(method)
    return np.array([_keep_smallest(keys[j], k) for j in range(n_blocks)],
                    dtype=np.int64).reshape(n_blocks, k)
