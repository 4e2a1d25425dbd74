"""Max-IDF summary selection (test infrastructure only).

Follows "Dropping the Anchor ..." Section 2.1 (Selecting summaries with
Max-IDF) and Figure 2:
  * every block is a document; df(t) is the number of the N blocks that
    contain token t, computed over the token IDs of the full sequence;
  * idf(t) = log(N / df(t)): Figure 2 prints 0 for a token in all four blocks,
    log 2 for one in two blocks and log 4 for one in a single block, which
    fixes this form (no smoothing; the log base does not change the order);
  * each block is cut into non-overlapping 32-token chunks, and a chunk's
    score is the IDF of its rarest token, i.e. the maximum IDF over its tokens;
  * the top-k chunks of each block, kept in their original order, form that
    block's summary; the budget is 12.5 % of the block size.
The page leaves the order among equal scores open; here the earlier chunk
wins.  When the budget is at least the number of chunks, every chunk is kept.

`chunk_min_df` is the integer form of the same score (max idf = log(N / min df)),
which the GPU path reports; a pin checks that both orders agree.
"""
import numpy as np


def document_frequency(tokens, n_blocks, block_size, vocab_size):
    """df[t] = number of blocks j in [0, N) whose tokens include t.  Ids outside
    [0, vocab_size) name no vocabulary entry and are not counted."""
    tokens = np.asarray(tokens)
    df = np.zeros(vocab_size, dtype=np.int64)
    for j in range(n_blocks):
        present = np.unique(tokens[j * block_size:(j + 1) * block_size])
        df[present[(present >= 0) & (present < vocab_size)]] += 1
    return df


def idf(df, n_blocks):
    """idf[t] = log(N / df[t]) in float64 (infinite for tokens that never occur,
    which no chunk can contain)."""
    df = np.asarray(df, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(n_blocks / df)


def chunk_max_idf(tokens, idf_table, n_blocks, block_size, chunk_size):
    """score[j][c] = max over the chunk's tokens of idf (the Max-IDF score)."""
    tokens = np.asarray(tokens)
    n_chunks = block_size // chunk_size
    score = np.empty((n_blocks, n_chunks), dtype=np.float64)
    for j in range(n_blocks):
        for c in range(n_chunks):
            start = j * block_size + c * chunk_size
            score[j, c] = idf_table[tokens[start:start + chunk_size]].max()
    return score


def chunk_min_df(tokens, df, n_blocks, block_size, chunk_size):
    """mindf[j][c] = min over the chunk's tokens of df (integer form of the score)."""
    tokens = np.asarray(tokens)
    n_chunks = block_size // chunk_size
    out = np.empty((n_blocks, n_chunks), dtype=np.int64)
    for j in range(n_blocks):
        for c in range(n_chunks):
            start = j * block_size + c * chunk_size
            out[j, c] = df[tokens[start:start + chunk_size]].min()
    return out


def top_k_in_order(score, k):
    """Per block: the k highest-scoring chunks (earlier chunk first among equal
    scores), returned in original (ascending) order.  int64 [N][min(k, C)]."""
    score = np.asarray(score)
    n_blocks, n_chunks = score.shape
    k_eff = min(k, n_chunks)
    sel = np.empty((n_blocks, k_eff), dtype=np.int64)
    for j in range(n_blocks):
        ranked = sorted(range(n_chunks), key=lambda c: (-score[j, c], c))
        sel[j] = sorted(ranked[:k_eff])
    return sel


def select(tokens, n_blocks, block_size, chunk_size, budget_chunks, vocab_size):
    """Full Max-IDF selection.  Returns (sel, df, max-idf scores)."""
    df = document_frequency(tokens, n_blocks, block_size, vocab_size)
    score = chunk_max_idf(tokens, idf(df, n_blocks), n_blocks, block_size, chunk_size)
    return top_k_in_order(score, budget_chunks), df, score


def prefix_positions(sel, n_blocks, block_size, chunk_size, sink_size):
    """Original positions of the prefix each block prepends in Phase 1.

    Block i > 0 prepends [sink || summary of block 0 || ... || summary of
    block i-1] ("Dropping the Anchor ..." Section 2 Method; the Dutch technical
    summary writes the host input as [S_sink || Sigma_0 || ... || Sigma_{i-1} || B_i]).
    The sink is the first `sink_size` tokens of the sequence; a summary is its
    selected chunks in original order.  Block 0 prepends nothing: its sink
    would be its own first tokens (Star Attention likewise leaves the first
    block without an anchor).  Entries are not de-duplicated, so a chunk of
    block 0 inside the sink appears twice, which keeps the prefix length fixed
    at sink + k * chunk * i.
    """
    out = [np.zeros(0, dtype=np.int64)]
    for i in range(1, n_blocks):
        parts = [np.arange(sink_size, dtype=np.int64)]
        for j in range(i):
            for c in sel[j]:
                start = j * block_size + int(c) * chunk_size
                parts.append(np.arange(start, start + chunk_size, dtype=np.int64))
        out.append(np.concatenate(parts))
    return out
