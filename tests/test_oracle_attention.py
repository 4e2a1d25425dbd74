"""Pins of the RoPE, bf16 and attention oracle against closed forms, textbook
special cases and library routines (never against a retyped copy of itself)."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import attention as A
from oracle import selection as S
from oracle.bf16 import round_bf16
from oracle.rope import rope


# ------------------------------------------------------------------ bf16
def test_round_bf16_ties_to_even_worked_values():
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    assert round_bf16(1.0 + ulp / 2) == 1.0          # tie -> even (1.0)
    assert round_bf16(1.0 + 1.5 * ulp) == 1.0 + 2 * ulp   # tie -> even
    assert round_bf16(1.0 + 0.51 * ulp) == 1.0 + ulp
    assert round_bf16(-3.0) == -3.0
    assert round_bf16(0.0) == 0.0


def test_round_bf16_matches_torch_on_float32_values():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * 37.0
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), want)


# ------------------------------------------------------------------ RoPE
def test_rope_position_zero_is_identity_and_norm_preserved():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 64))
    np.testing.assert_array_equal(rope(x, np.zeros(5), 500000.0), x)
    y = rope(x, rng.integers(0, 600000, 5), 500000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_equals_complex_rotation():
    """Pair (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2}, multiplied
    by exp(j * pos * base^(-2i/d))."""
    rng = np.random.default_rng(2)
    d, base = 16, 10000.0
    x = rng.standard_normal((7, 2, d))
    pos = rng.integers(0, 5000, 7)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freqs = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    z = z * np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    want = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(rope(x, pos, base), want, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_only_on_offset():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    base = 500000.0
    s1 = (rope(q, [1000], base) * rope(k, [400], base)).sum()
    s2 = (rope(q, [600600], base) * rope(k, [600000], base)).sum()
    assert s1 == pytest.approx(s2, rel=1e-9, abs=1e-9)


# ------------------------------------------------------------ attention
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _bf(x):
    return round_bf16(x)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (8, 2)])
def test_single_block_phase1_is_plain_causal_attention(hq, hkv):
    """With one block there is no prefix: Phase 1 is ordinary causal attention.
    Checked against torch's scaled_dot_product_attention (float64, causal,
    grouped-query heads)."""
    b, d, base = 48, 32, 500000.0
    q, k, v = _bf(_rand((b, hq, d), 1)), _bf(_rand((b, hkv, d), 2)), _bf(_rand((b, hkv, d), 3))
    pos = np.arange(b)
    k_hat = A.rotate_bf16(k, pos, base)
    got = A.phase1_rows(q, k_hat, v, [np.zeros(0, np.int64)], [(0, r) for r in range(b)], b, base)
    qh = torch.from_numpy(A.rotate_bf16(q, pos, base)).permute(1, 0, 2)[None]
    kh = torch.from_numpy(k_hat).permute(1, 0, 2)[None]
    vh = torch.from_numpy(v).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, is_causal=True,
                                                            enable_gqa=(hq != hkv))
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_gather_form_equals_dense_form_with_multiplicity_bias():
    N, b, chunk, sink, hq, hkv, d, base = 3, 64, 16, 32, 4, 2, 16, 500000.0
    L = N * b
    q, k, v = _bf(_rand((L, hq, d), 4)), _bf(_rand((L, hkv, d), 5)), _bf(_rand((L, hkv, d), 6))
    sel = np.array([[0, 2], [1, 3], [0, 1]])     # chunk 0 of block 0 lies inside the sink
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    k_hat = A.rotate_bf16(k, np.arange(L), base)
    for i in range(N):
        dense = A.phase1_block_dense(q, k_hat, v, pre[i], i, b, base)
        rows = A.phase1_rows(q, k_hat, v, pre, [(i, r) for r in range(b)], b, base)
        np.testing.assert_allclose(rows, dense, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(4, 2), (8, 2)])
def test_rows_in_block_single_block_is_plain_causal_attention(hq, hkv):
    """The several-rows form on one block (no prefix) against torch's causal
    scaled_dot_product_attention in float64, on a subset of the rows."""
    b, d, base = 48, 32, 500000.0
    q, k, v = _bf(_rand((b, hq, d), 11)), _bf(_rand((b, hkv, d), 12)), _bf(_rand((b, hkv, d), 13))
    pos = np.arange(b)
    k_hat = A.rotate_bf16(k, pos, base)
    rows = [0, 1, 5, 31, 32, 47]
    got = A.phase1_rows_in_block(q, k_hat, v, np.zeros(0, np.int64), 0, rows, b, base)
    qh = torch.from_numpy(A.rotate_bf16(q, pos, base)).permute(1, 0, 2)[None]
    kh = torch.from_numpy(k_hat).permute(1, 0, 2)[None]
    vh = torch.from_numpy(v).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, is_causal=True,
                                                            enable_gqa=(hq != hkv))
    want = want[0].permute(1, 0, 2).numpy()[rows]
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_rows_in_block_equals_dense_form_with_multiplicity_bias():
    """Row subsets (unsorted, repeated, ending below the block's end) of every
    block against the dense twin, with a kept chunk inside the sink."""
    N, b, chunk, sink, hq, hkv, d, base = 3, 64, 16, 32, 4, 2, 16, 500000.0
    L = N * b
    q, k, v = _bf(_rand((L, hq, d), 14)), _bf(_rand((L, hkv, d), 15)), _bf(_rand((L, hkv, d), 16))
    sel = np.array([[0, 2], [1, 3], [0, 1]])
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    k_hat = A.rotate_bf16(k, np.arange(L), base)
    for i in range(N):
        dense = A.phase1_block_dense(q, k_hat, v, pre[i], i, b, base)
        for rows in ([0], [b - 1, 3, 17, 3], list(range(b)), [5, 40, 41]):
            got = A.phase1_rows_in_block(q, k_hat, v, pre[i], i, rows, b, base)
            np.testing.assert_allclose(got, dense[rows], rtol=1e-10, atol=1e-12)


def test_rows_in_block_zero_keys_average_exactly_the_visible_values():
    """K = 0: each output is the mean of the visible value rows (duplicates
    counted), so position-coded values reveal the visible set."""
    N, b, chunk, sink, d, base = 3, 64, 16, 32, 8, 500000.0
    L = N * b
    q = _bf(_rand((L, 2, d), 17))
    k = np.zeros((L, 1, d))
    v = np.zeros((L, 1, d))
    v[:, 0, 0] = np.arange(L)
    v[:, 0, 1] = np.arange(L) ** 2
    sel = np.array([[0, 2], [1, 3], [0, 1]])
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    for i in range(N):
        rows = [0, 1, 17, b - 1]
        got = A.phase1_rows_in_block(q, k, v, pre[i], i, rows, b, base)
        for n, r in enumerate(rows):
            vis = np.concatenate([np.asarray(pre[i], np.int64), np.arange(i * b, i * b + r + 1)])
            np.testing.assert_allclose(got[n, :, 0], vis.mean(), rtol=1e-12)
            np.testing.assert_allclose(got[n, :, 1], (vis.astype(float) ** 2).mean(), rtol=1e-12)


def test_zero_keys_give_uniform_weights_over_the_visible_set():
    """K = 0 makes every score 0, so each output is the plain mean of the
    visible V rows, counting duplicates; with V encoding the position, the
    output reveals exactly which keys a row saw (K = 0 is RoPE-invariant)."""
    N, b, chunk, sink, d, base = 3, 64, 16, 32, 8, 500000.0
    L = N * b
    q = _bf(_rand((L, 2, d), 7))
    k = np.zeros((L, 1, d))
    v = np.zeros((L, 1, d))
    v[:, 0, 0] = np.arange(L)
    v[:, 0, 1] = np.arange(L) ** 2
    sel = np.array([[0, 2], [1, 3], [0, 1]])
    pre = S.prefix_positions(sel, N, b, chunk, sink)
    k_hat = A.rotate_bf16(k, np.arange(L), base)
    for i in range(N):
        for r in [0, 1, 17, b - 1]:
            keys = list(pre[i]) + list(range(i * b, i * b + r + 1))
            o = A.phase1_rows(q, k_hat, v, pre, [(i, r)], b, base)[0]
            assert o[0, 0] == pytest.approx(np.mean(keys), rel=1e-12)
            assert o[1, 1] == pytest.approx(np.mean(np.square(keys)), rel=1e-12)
    # Phase 2: lse of a shard of n keys with zero scores is ln n
    kc = np.zeros((2, 1, 40, d))
    vc = _rand((2, 1, 40, d), 8)
    parts = A.phase2_partials(_rand((3, 2, d), 9), 1000, kc, vc, None, None, base)
    for o, lse in parts:
        np.testing.assert_allclose(lse, math.log(40), rtol=1e-12)


def _phase2_case(seed, n_shards=3, n=37, lq=5, hq=4, hkv=2, d=16, base=500000.0):
    rng = np.random.default_rng(seed)
    kc = _bf(rng.standard_normal((n_shards, hkv, n, d)))
    vc = _bf(rng.standard_normal((n_shards, hkv, n, d)))
    qq = _bf(rng.standard_normal((lq, hq, d)))
    ks = _bf(rng.standard_normal((lq, hkv, d)))
    vs = _bf(rng.standard_normal((lq, hkv, d)))
    return qq, kc, vc, ks, vs, base


@pytest.mark.parametrize("with_self", [True, False])
def test_lse_merge_of_shards_equals_dense_attention(with_self):
    """Section 2.2: the merge of per-shard partials is exact attention over all
    retained shards (plus the causal self shard)."""
    qq, kc, vc, ks, vs, base = _phase2_case(10)
    if not with_self:
        ks = vs = None
    parts = A.phase2_partials(qq, 5000, kc, vc, ks, vs, base)
    o, lse = A.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    o2, lse2 = A.dense_query_attention(qq, 5000, kc, vc, ks, vs, base)
    np.testing.assert_allclose(o, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-12)


def test_merge_is_independent_of_shard_order_and_split_points():
    qq, kc, vc, ks, vs, base = _phase2_case(11, n_shards=2, n=40)
    whole = A.phase2_partials(qq, 100, kc, vc, None, None, base)
    o1, l1 = A.lse_merge([p[0] for p in whole], [p[1] for p in whole])
    # split every shard at an arbitrary point and reverse the order
    pieces_k = [kc[s][:, a:b_] for s in range(2) for (a, b_) in [(0, 13), (13, 40)]][::-1]
    pieces_v = [vc[s][:, a:b_] for s in range(2) for (a, b_) in [(0, 13), (13, 40)]][::-1]
    parts = []
    for pk, pv in zip(pieces_k, pieces_v):
        parts += A.phase2_partials(qq, 100, pk[None], pv[None], None, None, base)
    o2, l2 = A.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)


def test_one_shard_is_plain_attention_and_lse_is_logsumexp():
    qq, kc, vc, ks, vs, base = _phase2_case(12, n_shards=1)
    (o, lse), = A.phase2_partials(qq, 77, kc, vc, None, None, base)
    lq, hq, d = qq.shape
    q_hat = A.rotate_bf16(qq, 77 + np.arange(lq), base)
    qh = torch.from_numpy(q_hat).permute(1, 0, 2)[None]
    kh = torch.from_numpy(kc[0])[None]
    vh = torch.from_numpy(vc[0])[None]
    want = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, enable_gqa=True)
    np.testing.assert_allclose(o, want[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)
    for h in range(hq):
        s = q_hat[:, h, :] @ kc[0, h // 2].T / math.sqrt(d)
        np.testing.assert_allclose(lse[:, h], logsumexp(s, axis=1), rtol=1e-12)


def test_self_shard_is_causal():
    """The first query token sees only itself among the query tokens, so with a
    single self key its self-shard output is that key's value row."""
    qq, kc, vc, ks, vs, base = _phase2_case(13)
    parts = A.phase2_partials(qq, 9000, kc, vc, ks, vs, base)
    o_self, lse_self = parts[-1]
    for h in range(qq.shape[1]):
        np.testing.assert_allclose(o_self[0, h], vs[0, h // 2], rtol=1e-12)


def test_retained_cache_does_not_depend_on_selection():
    """The kept KV is the block's own rotated keys and values whatever the
    prefix (Section 2.2: the retained cache is identical to Star Attention's)."""
    N, b, d, base = 2, 32, 8, 500000.0
    k, v = _bf(_rand((N * b, 2, d), 14)), _bf(_rand((N * b, 2, d), 15))
    kc, vc = A.retained_cache(k, v, N, b, base)
    assert kc.shape == (N, 2, b, d)
    np.testing.assert_array_equal(vc[1, 0], v[b:, 0])
    np.testing.assert_array_equal(kc[1, 1, 3], A.rotate_bf16(k[b + 3:b + 4], [b + 3], base)[0, 1])


def _decode_case(seed, n_shards=2, n=24, hq=4, hkv=2, d=16, n_self=7, lq=3):
    rng = np.random.default_rng(seed)
    kc = round_bf16(rng.standard_normal((n_shards, hkv, n, d)))
    vc = round_bf16(rng.standard_normal((n_shards, hkv, n, d)))
    qq = round_bf16(rng.standard_normal((lq, hq, d)))
    ks = round_bf16(rng.standard_normal((n_self, hkv, d)))
    vs = round_bf16(rng.standard_normal((n_self, hkv, d)))
    return qq, kc, vc, ks, vs


@pytest.mark.parametrize("n_self,lq", [(7, 3), (5, 1), (1, 1), (4, 4)])
def test_decode_merge_equals_masked_dense_attention(n_self, lq):
    qq, kc, vc, ks, vs = _decode_case(11 + n_self, n_self=n_self, lq=lq)
    parts = A.decode_partials(qq, kc, vc, ks, vs, 1000, 1e4)
    o, lse = A.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    o2, lse2 = A.dense_decode_attention(qq, kc, vc, ks, vs, 1000, 1e4)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_decode_with_self_equal_to_query_is_the_query_phase():
    qq, kc, vc, ks, vs = _decode_case(5, n_self=3, lq=3)
    a = A.decode_partials(qq, kc, vc, ks, vs, 500, 1e4)
    b = A.phase2_partials(qq, 500, kc, vc, ks, vs, 1e4)
    for (oa, la), (ob, lb) in zip(a, b):
        np.testing.assert_allclose(oa, ob, atol=1e-13)
        np.testing.assert_allclose(la, lb, atol=1e-13)


def test_decode_zero_keys_average_exactly_the_visible_values():
    # zero keys: every visible key scores 0, so each query row averages the
    # values it may see: all retained ones and self tokens up to itself
    qq, kc, vc, ks, vs = _decode_case(9, n_self=6, lq=2)
    kc = np.zeros_like(kc)
    ks = np.zeros_like(ks)
    o, lse = A.dense_decode_attention(qq, kc, vc, ks, vs, 40, 1e4)
    n_ret = kc.shape[0] * kc.shape[2]
    for t in range(2):
        n_vis_self = 6 - 2 + t + 1
        for h in range(qq.shape[1]):
            g = h // 2
            want = (vc[:, g].reshape(-1, vc.shape[-1]).sum(0) + vs[:n_vis_self, g].sum(0)) / (n_ret + n_vis_self)
            np.testing.assert_allclose(o[t, h], want, atol=1e-12)
            assert abs(lse[t, h] - np.log(n_ret + n_vis_self)) < 1e-12


def _prefix_case(seed, L=96, hq=4, hkv=2, d=16):
    rng = np.random.default_rng(seed)
    q = round_bf16(rng.standard_normal((L, hq, d)))
    k = round_bf16(rng.standard_normal((L, hkv, d)))
    v = round_bf16(rng.standard_normal((L, hkv, d)))
    khat = A.rotate_bf16(k, np.arange(L), 1e4)
    return q, khat, v


def test_prefix_rows_of_a_contiguous_prefix_are_textbook_causal_attention():
    # Star setting: the prefix is block 0 itself, so its rows are plain causal
    # attention over block 0 (float64 softmax of QK^T/sqrt(d) with a causal mask)
    q, khat, v = _prefix_case(3)
    n = 40
    got = A.prefix_rows(q, khat, v, np.arange(n), range(n), 1e4)
    qh = A.rotate_bf16(q[:n], np.arange(n), 1e4)
    for h in range(q.shape[1]):
        g = h // 2
        s = qh[:, h, :] @ khat[:n, g, :].T / math.sqrt(q.shape[2])
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
        want = torch.softmax(torch.from_numpy(s), dim=1).numpy() @ v[:n, g, :]
        np.testing.assert_allclose(got[:, h, :], want, atol=1e-12)


def test_prefix_rows_gather_equals_multiplicity_bias_dense():
    # a sink of 16 positions followed by chunks of 8, one of them inside the sink
    # (kept twice, as the method's prefix does)
    q, khat, v = _prefix_case(7)
    pre = np.concatenate([np.arange(16), np.arange(8, 16), np.arange(40, 48), np.arange(72, 80)])
    got = A.prefix_rows(q, khat, v, pre, range(len(pre)), 1e4)
    want = A.prefix_rows_dense(q, khat, v, pre, 1e4)
    np.testing.assert_allclose(got, want, atol=1e-12)


# ------------------------------------------------------ Llama-3.1 scaling
def test_llama3_scaling_regimes_at_base_500000_d128():
    # wavelength 2 pi * 500000^(i/64): below 2048 for i <= 28, above 8192 for i >= 35
    from oracle.rope import Llama3Base, inv_freq
    plain = inv_freq(128, 500000.0)
    scaled = inv_freq(128, Llama3Base(500000.0))
    assert np.array_equal(scaled[:29], plain[:29])
    np.testing.assert_allclose(scaled[35:], plain[35:] / 8.0, rtol=1e-15)
    mid = scaled[29:35] / plain[29:35]
    assert np.all((mid > 1.0 / 8.0) & (mid < 1.0)) and np.all(np.diff(mid) < 0)


def test_llama3_scaled_low_frequencies_rotate_as_one_eighth_of_the_position():
    from oracle.rope import Llama3Base
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 2, 128))
    pos = np.array([0, 8, 800, 8000, 131072])
    a = rope(x, pos, Llama3Base(500000.0))
    b = rope(x, pos // 8, 500000.0)
    for i in range(35, 64):   # the low-frequency pairs (i, i + 64)
        np.testing.assert_allclose(a[..., [i, i + 64]], b[..., [i, i + 64]], atol=1e-12)
    np.testing.assert_allclose(a[..., :29], rope(x, pos, 500000.0)[..., :29], atol=1e-12)
