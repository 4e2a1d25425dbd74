"""Pins of the selection oracle against what the pages and plain counting fix.

Sources: "Dropping the Anchor ..." Section 2.1 and Figure 2 (Max-IDF), Section 4
(the 1,600-token prefix), and the Star Attention review (the anchor input).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import selection as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(s):
    return {"0": 0.0, "log 2": math.log(2.0), "log 4": math.log(4.0)}[s]


def test_figure2_toy_idf_scores_and_answer_selected():
    g = json.load(open(os.path.join(GOLDEN, "fig2_toy.json")))
    t = np.array(g["tokens"])
    N, b, c, k, V = g["n_blocks"], g["block_size"], g["chunk_size"], g["budget_chunks"], g["vocab_size"]
    sel, df, score = S.select(t, N, b, c, k, V)
    idf = S.idf(df, N)
    for tok, want in g["expected_idf"].items():
        assert idf[int(tok)] == pytest.approx(_val(want), abs=1e-15)
    want_scores = np.array([[_val(x) for x in row] for row in g["expected_chunk_scores"]])
    np.testing.assert_allclose(score, want_scores, atol=1e-15)
    assert sel.shape == (N, 1)
    assert sel[g["answer_block"], 0] == g["answer_chunk"]
    # every other block keeps its best chunk: the distractor where present,
    # otherwise (all filler, all ties) the earliest chunk
    assert sel[:, 0].tolist() == [0, 1, 2, 0]


def _brute_force_select(score, k):
    """A chunk is kept iff fewer than k chunks beat it (higher score, or equal
    score and earlier position)."""
    n_blocks, n_chunks = score.shape
    out = []
    for j in range(n_blocks):
        keep = []
        for c in range(n_chunks):
            better = sum(1 for c2 in range(n_chunks)
                         if score[j, c2] > score[j, c] or (score[j, c2] == score[j, c] and c2 < c))
            if better < k:
                keep.append(c)
        out.append(keep)
    return out


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_brute_force_and_min_df_order(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 7))
    chunk = int(rng.choice([2, 4, 8]))
    C = int(rng.integers(1, 9))
    b = chunk * C
    V = int(rng.integers(3, 40))
    t = rng.integers(0, V, size=N * b)
    k = int(rng.integers(0, C + 2))
    sel, df, score = S.select(t, N, b, chunk, k, V)
    bf = _brute_force_select(score, k)
    assert [list(r) for r in sel] == bf
    # the integer score orders chunks exactly as max idf does (ties included)
    mindf = S.chunk_min_df(t, df, N, b, chunk)
    sel2 = S.top_k_in_order(-mindf, k)
    np.testing.assert_array_equal(sel, sel2)
    np.testing.assert_allclose(score, np.log(N / mindf), rtol=0, atol=1e-15)


def test_df_counts_blocks_by_brute_force():
    rng = np.random.default_rng(5)
    N, b, V = 5, 24, 30
    t = rng.integers(0, V, size=N * b)
    df = S.document_frequency(t, N, b, V)
    for tok in range(V):
        want = sum(1 for j in range(N) if tok in set(t[j * b:(j + 1) * b].tolist()))
        assert df[tok] == want
    # sum of df = sum over blocks of distinct tokens; 1 <= df <= N where present
    assert df.sum() == sum(len(set(t[j * b:(j + 1) * b].tolist())) for j in range(N))
    present = np.unique(t)
    assert df[present].min() >= 1 and df.max() <= N


@pytest.mark.parametrize("name", ["tiny"])
def test_summary_length_equals_budget_and_order(name):
    w = W.WORKLOADS[name]
    t = W.tokens(w)
    sel, df, score = S.select(t, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks, w.vocab_size)
    assert sel.shape == (w.n_blocks, w.budget_chunks)
    # 12.5 % of the block, in tokens
    assert sel.shape[1] * w.chunk_size == w.block_size // 8
    for j in range(w.n_blocks):
        assert np.all(np.diff(sel[j]) > 0)
        assert sel[j].min() >= 0 and sel[j].max() < w.n_chunks
    # planted ids are unique to one block, so every planted chunk scores log N
    pp = W.planted_positions(w)
    for p in pp:
        j, c = p // w.block_size, (p % w.block_size) // w.chunk_size
        assert score[j, c] == pytest.approx(math.log(w.n_blocks))


@pytest.mark.parametrize("per_block", [1, 3, 4])
def test_filler_stream_selects_exactly_the_planted_chunks(per_block):
    N, b, chunk = 4, 1024, 32
    t, planted = W.filler_planted_tokens(7 + per_block, N, b, chunk, per_block)
    sel, df, score = S.select(t, N, b, chunk, per_block, 4096)
    np.testing.assert_array_equal(sel, planted)
    assert df[:32].tolist() == [N] * 32


def test_budget_edge_cases():
    rng = np.random.default_rng(3)
    N, b, chunk = 3, 64, 32
    t = rng.integers(0, 50, size=N * b)
    sel0, _, _ = S.select(t, N, b, chunk, 0, 50)
    assert sel0.shape == (N, 0)
    sel_all, _, _ = S.select(t, N, b, chunk, 5, 50)
    np.testing.assert_array_equal(sel_all, np.tile(np.arange(2), (N, 1)))
    # all ties: the first k chunks
    t_same = np.zeros(N * b, np.int64)
    sel_tie, _, _ = S.select(t_same, N, b, 8, 3, 4)
    np.testing.assert_array_equal(sel_tie, np.tile(np.arange(3), (N, 1)))


def test_prefix_is_1600_tokens_for_last_of_four_hosts():
    """Section 4: each host adds a fixed 1,600-token prefix: 64 sink tokens
    plus three 512-token summaries (4K blocks, 16 chunks of 32 tokens)."""
    N, b, chunk, k, sink = 4, 4096, 32, 16, 64
    t = np.random.default_rng(0).integers(0, 1000, size=N * b)
    sel, _, _ = S.select(t, N, b, chunk, k, 1000)
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    assert len(pre[3]) == 1600
    assert [len(p) for p in pre] == [0, 64 + 512, 64 + 1024, 1600]
    # original positions: the sink is positions 0..63; summaries follow in block order
    assert pre[3][:64].tolist() == list(range(64))
    assert np.all(np.diff(pre[3][64:]) > 0)
    assert pre[3][-1] < 3 * b


def test_star_anchor_special_case():
    """Sink = a whole block and no summaries reproduces Star Attention's anchor
    input: block 0 is encoded alone, every later block is prefixed with block 0
    at its original indices (the review's c'_1 = c_1, c'_i = [c_1 || c_i])."""
    N, b, chunk = 4, 128, 32
    sel = np.zeros((N, 0), np.int64)
    pre = S.prefix_positions(sel, N, b, chunk, sink_size=b)
    assert len(pre[0]) == 0
    for i in range(1, N):
        assert pre[i].tolist() == list(range(b))
        assert len(pre[i]) + b == 2 * b


def test_sink_overlap_is_not_deduplicated():
    N, b, chunk, sink = 3, 128, 32, 64
    sel = np.array([[0, 3], [1, 2], [0, 1]])
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    assert len(pre[2]) == sink + 2 * 2 * chunk
    counts = np.bincount(pre[2])
    assert counts[:32].tolist() == [2] * 32      # chunk 0 of block 0 is also sink
    assert counts[32:64].tolist() == [1] * 32


def test_zipf_stream_is_reproducible_and_bounded():
    w = W.WORKLOADS["tiny"]
    t1, t2 = W.tokens(w), W.tokens(w)
    np.testing.assert_array_equal(t1, t2)
    assert t1.min() >= 0 and t1.max() < w.vocab_size
    assert len(W.planted_positions(w)) == w.n_planted


def test_df_skips_ids_outside_the_vocabulary():
    t = np.array([0, 1, 7, -2, 1, 8, 0, 3], np.int64)       # V = 8: ids 8 and -2 name no entry
    df = S.document_frequency(t, 2, 4, 8)
    assert df.tolist() == [2, 2, 0, 1, 0, 0, 0, 1]
