"""Pins of the other selection methods (mean IDF, entropy, uniform, evenly spaced)
against what the pages, library routines and plain counting fix.

Sources: "Dropping the Anchor ..." Section 2.1 and Figure 2 (the maximum against
the mean), the Dutch technical summary's ablation list (TF-IDF, BM25, entropy,
uniform sampling), Steele, Lea and Flood 2014 (SplitMix64)."""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import chisquare
from scipy.stats import entropy as scipy_entropy

from oracle import selection as S
from oracle import selection_variants as V

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rank_by_float(scores, k, tol=1e-9):
    """Keep the k best of float scores (higher better, ties to the earlier chunk);
    None when two scores are closer than tol without being equal."""
    s = np.asarray(scores)
    if any(0 < abs(a - b) < tol for a in s for b in s):
        return None
    order = sorted(range(len(s)), key=lambda c: (-s[c], c))
    return sorted(order[:min(k, len(s))])


def _random_case(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(2, 7))
    chunk = int(rng.choice([4, 8]))
    C = int(rng.integers(2, 9))
    b = chunk * C
    V_ = int(rng.integers(3, 30))
    t = rng.integers(0, V_, size=N * b)
    k = int(rng.integers(1, C + 1))
    return t, N, b, chunk, k, V_


@pytest.mark.parametrize("seed", range(10))
def test_mean_idf_exact_order_equals_the_float_definition(seed):
    t, N, b, chunk, k, V_ = _random_case(seed)
    sel = V.select_variant("mean_idf", t, N, b, chunk, k, V_)
    scores = V.mean_idf_scores(t, N, b, chunk, V_)
    checked = 0
    for j in range(N):
        want = _rank_by_float(scores[j], k)
        if want is not None:
            assert sel[j].tolist() == want
            checked += 1
    assert checked > 0


def test_mean_idf_loses_the_answer_of_figure2():
    """Section 2.1: averaging divides a rare token's signal by the chunk length.
    In the Figure-2 toy the answer chunk (one log-4 token among fillers) ties with
    a distractor chunk (two log-2 tokens) under the mean and loses on position,
    while the maximum keeps the answer."""
    g = json.load(open(os.path.join(GOLDEN, "fig2_toy.json")))
    t = np.array(g["tokens"])
    N, b, c, k, Vs = g["n_blocks"], g["block_size"], g["chunk_size"], g["budget_chunks"], g["vocab_size"]
    mean = V.mean_idf_scores(t, N, b, c, Vs)
    assert mean[2, 1] == pytest.approx(math.log(4) / 4, abs=1e-15)
    assert mean[2, 2] == pytest.approx(math.log(4) / 4, abs=1e-15)
    keys = V.mean_idf_keys(t, N, b, c, Vs)
    assert keys[2][1] == keys[2][2]                       # an exact tie
    sel_mean = V.select_variant("mean_idf", t, N, b, c, k, Vs)
    sel_max, _, _ = S.select(t, N, b, c, k, Vs)
    assert sel_max[2, 0] == g["answer_chunk"] == 2
    assert sel_mean[2, 0] == 1


@pytest.mark.parametrize("seed", range(10))
def test_entropy_exact_order_equals_scipy_entropy(seed):
    t, N, b, chunk, k, V_ = _random_case(100 + seed)
    sel = V.select_variant("entropy", t, N, b, chunk, k, V_)
    checked = 0
    for j in range(N):
        h = []
        for c in range(b // chunk):
            ids = t[j * b + c * chunk:j * b + (c + 1) * chunk]
            _, counts = np.unique(ids, return_counts=True)
            h.append(scipy_entropy(counts))                 # nats, normalised counts
        want = _rank_by_float(h, k)
        if want is not None:
            assert sel[j].tolist() == want
            checked += 1
    assert checked > 0
    np.testing.assert_allclose(V.entropy_scores(t, N, b, chunk)[0, 0],
                               scipy_entropy(np.unique(t[:chunk], return_counts=True)[1]),
                               rtol=1e-12)


def test_entropy_closed_forms():
    """A chunk of one repeated id has entropy 0, a chunk of distinct ids ln C;
    the key prod_v c_v^c_v is 1 for distinct ids and C^C for one id."""
    chunk = 8
    t = np.array([5] * 8 + list(range(8)) + [1, 1, 2, 2, 3, 3, 4, 4] + [9] * 4 + [8] * 4)
    N, b = 1, 32
    h = V.entropy_scores(t, N, b, chunk)[0]
    np.testing.assert_allclose(h, [0.0, math.log(8), math.log(4), math.log(2)], atol=1e-15)
    assert V.entropy_keys(t, N, b, chunk)[0] == [8 ** 8, 1, 2 ** 8, 4 ** 8]
    assert V.select_variant("entropy", t, N, b, chunk, 1, 16)[0].tolist() == [1]
    assert V.select_variant("entropy", t, N, b, chunk, 3, 16)[0].tolist() == [1, 2, 3]


def test_uniform_selection_is_uniform_and_seeded():
    N, C, k = 1, 16, 4
    b = C * 8
    counts = np.zeros(C)
    seen = set()
    for seed in range(3000):
        sel = V.select_variant("uniform", np.zeros(N * b, np.int64), N, b, 8, k, 4, seed=seed)[0]
        assert len(set(sel.tolist())) == k and np.all(np.diff(sel) > 0)
        counts[sel] += 1
        seen.add(tuple(sel.tolist()))
    # every chunk is kept with probability k / C
    assert chisquare(counts).pvalue > 1e-4
    assert len(seen) > 1000                 # many different subsets
    a = V.select_variant("uniform", np.zeros(2 * b, np.int64), 2, b, 8, k, 4, seed=7)
    b2 = V.select_variant("uniform", np.zeros(2 * b, np.int64), 2, b, 8, k, 4, seed=7)
    np.testing.assert_array_equal(a, b2)
    assert a[0].tolist() != a[1].tolist() or k == C  # blocks draw different counters


def test_splitmix64_known_answers():
    """The published known-answer values of SplitMix64 (tests/golden/splitmix64_kat.json):
    the first five outputs from one seed, and the float bucket counts of 100,000
    outputs from another.  A wrong constant, shift or increment changes both."""
    with open(os.path.join(GOLDEN, "splitmix64_kat.json")) as f:
        kat = json.load(f)
    got = [V.splitmix64(kat["seed"], n) for n in range(1, 6)]
    assert got == [int(x) for x in kat["first_outputs"]]
    nb = kat["histogram_buckets"]
    counts = [0] * nb
    for n in range(1, kat["histogram_n"] + 1):
        counts[int(V.splitmix64(kat["histogram_seed"], n) / 2.0 ** 64 * nb)] += 1
    assert counts == kat["histogram_counts"]


def test_splitmix64_outputs_are_balanced():
    bits = np.array([[(V.splitmix64(99, n) >> i) & 1 for i in range(64)] for n in range(1, 4001)])
    frac = bits.mean(axis=0)
    assert np.all(np.abs(frac - 0.5) < 0.04)
    # consecutive outputs are uncorrelated at the bit level
    agree = (bits[1:] == bits[:-1]).mean()
    assert abs(agree - 0.5) < 0.01


def test_even_spacing_closed_form():
    N, chunk = 2, 4
    for C, k in [(8, 4), (8, 8), (10, 3), (7, 1), (12, 5)]:
        b = C * chunk
        sel = V.select_variant("even", np.zeros(N * b, np.int64), N, b, chunk, k, 4)
        assert sel.shape == (N, k)
        want = [m * C // k for m in range(k)]
        assert sel[0].tolist() == want == sel[1].tolist()
        gaps = np.diff(want + [C])
        assert set(gaps.tolist()) <= {C // k, -(-C // k)}
    assert V.select_variant("even", np.zeros(32, np.int64), 1, 32, 4, 4, 4)[0].tolist() == [0, 2, 4, 6]
    assert V.select_variant("even", np.zeros(32, np.int64), 1, 32, 4, 20, 4)[0].tolist() == list(range(8))


def test_tf_idf_with_chunk_term_counts_ranks_as_mean_idf():
    """TF-IDF of a chunk, sum over its distinct terms of count * idf, equals the
    chunk length times the mean IDF, so both keep the same chunks."""
    t, N, b, chunk, k, Vs = _random_case(7)
    df = S.document_frequency(t, N, b, Vs)
    mean = V.mean_idf_scores(t, N, b, chunk, Vs)
    for j in range(N):
        for c in range(b // chunk):
            ids = t[j * b + c * chunk:j * b + (c + 1) * chunk]
            terms, counts = np.unique(ids, return_counts=True)
            tfidf = sum(n * math.log(N / df[v]) for v, n in zip(terms, counts))
            assert tfidf == pytest.approx(chunk * mean[j, c], abs=1e-12)
