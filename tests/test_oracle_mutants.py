"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by replacing one of its
functions for the duration of the test) and runs the pins that guard that part;
at least one of them must fail.  The mistakes are the kind a reading of the
pages could make: a dropped term, a wrong sign or index, a swapped operand, a
different tie-break, an off-by-one mask, a wrong logarithm base.
"""
import math

import numpy as np
import pytest

import oracle.attention as A
import oracle.bf16 as OB
import oracle.rope as R
import oracle.selection as S
from tests import test_oracle_attention as TA
from tests import test_oracle_selection as TS


def _replace(monkeypatch, original, replacement):
    """Point every module-level name bound to `original` (in the oracle and the
    pin modules) at `replacement`."""
    for mod in (A, OB, R, S, TA, TS):
        for name, val in list(vars(mod).items()):
            if val is original:
                monkeypatch.setattr(mod, name, replacement)


def _failing(pins):
    failed = []
    for pin in pins:
        fn, args = (pin if isinstance(pin, tuple) else (pin, ()))
        try:
            fn(*args)
        except AssertionError:
            failed.append(fn.__name__)
    return failed


def _caught(monkeypatch, original, replacement, pins):
    _replace(monkeypatch, original, replacement)
    failed = _failing(pins)
    assert failed, f"no pin caught the planted mistake in {original.__name__}"
    return failed


SELECTION_PINS = [TS.test_figure2_toy_idf_scores_and_answer_selected,
                  (TS.test_topk_equals_brute_force_and_min_df_order, (0,)),
                  (TS.test_topk_equals_brute_force_and_min_df_order, (3,)),
                  TS.test_df_counts_blocks_by_brute_force,
                  (TS.test_summary_length_equals_budget_and_order, ("tiny",)),
                  (TS.test_filler_stream_selects_exactly_the_planted_chunks, (3,)),
                  TS.test_budget_edge_cases]
PREFIX_PINS = [TS.test_prefix_is_1600_tokens_for_last_of_four_hosts,
               TS.test_star_anchor_special_case,
               TS.test_sink_overlap_is_not_deduplicated]
ROPE_PINS = [TA.test_rope_position_zero_is_identity_and_norm_preserved,
             TA.test_rope_equals_complex_rotation,
             TA.test_rope_scores_depend_only_on_offset]
PHASE1_PINS = [(TA.test_single_block_phase1_is_plain_causal_attention, (4, 2)),
               (TA.test_single_block_phase1_is_plain_causal_attention, (8, 2)),
               TA.test_gather_form_equals_dense_form_with_multiplicity_bias,
               TA.test_zero_keys_give_uniform_weights_over_the_visible_set]
ROWS_IN_BLOCK_PINS = [(TA.test_rows_in_block_single_block_is_plain_causal_attention, (4, 2)),
                      TA.test_rows_in_block_equals_dense_form_with_multiplicity_bias,
                      TA.test_rows_in_block_zero_keys_average_exactly_the_visible_values]
PHASE2_PINS = [(TA.test_lse_merge_of_shards_equals_dense_attention, (True,)),
               (TA.test_lse_merge_of_shards_equals_dense_attention, (False,)),
               TA.test_merge_is_independent_of_shard_order_and_split_points,
               TA.test_one_shard_is_plain_attention_and_lse_is_logsumexp,
               TA.test_self_shard_is_causal]


# ------------------------------------------------------------- selection
def test_df_counting_occurrences_instead_of_blocks_is_caught(monkeypatch):
    def bad(tokens, n_blocks, block_size, vocab_size):
        return np.bincount(np.asarray(tokens)[:n_blocks * block_size], minlength=vocab_size)
    _caught(monkeypatch, S.document_frequency, bad, SELECTION_PINS)


def test_smoothed_idf_is_caught(monkeypatch):
    def bad(df, n_blocks):
        return np.log((n_blocks + 1.0) / (np.asarray(df, np.float64) + 1.0))
    _caught(monkeypatch, S.idf, bad, SELECTION_PINS)


def test_mean_instead_of_max_idf_is_caught(monkeypatch):
    def bad(tokens, idf_table, n_blocks, block_size, chunk_size):
        t = np.asarray(tokens)[:n_blocks * block_size]
        return idf_table[t].reshape(n_blocks, block_size // chunk_size, chunk_size).mean(axis=2)
    _caught(monkeypatch, S.chunk_max_idf, bad, SELECTION_PINS)


def test_later_chunk_winning_ties_is_caught(monkeypatch):
    def bad(score, k):
        score = np.asarray(score)
        n_blocks, n_chunks = score.shape
        k_eff = min(k, n_chunks)
        sel = np.empty((n_blocks, k_eff), np.int64)
        for j in range(n_blocks):
            ranked = sorted(range(n_chunks), key=lambda c: (-score[j, c], -c))
            sel[j] = sorted(ranked[:k_eff])
        return sel
    _caught(monkeypatch, S.top_k_in_order, bad, SELECTION_PINS)


def test_summary_in_rank_order_is_caught(monkeypatch):
    def bad(score, k):
        score = np.asarray(score)
        n_blocks, n_chunks = score.shape
        k_eff = min(k, n_chunks)
        sel = np.empty((n_blocks, k_eff), np.int64)
        for j in range(n_blocks):
            sel[j] = sorted(range(n_chunks), key=lambda c: (-score[j, c], c))[:k_eff]
        return sel
    _caught(monkeypatch, S.top_k_in_order, bad, SELECTION_PINS)


# ---------------------------------------------------------------- prefix
def _prefix(sel, n_blocks, block_size, chunk_size, sink_size, first=1, dedup=False, rev=False):
    out = [np.zeros(0, np.int64)] * first
    for i in range(first, n_blocks):
        parts = [np.arange(sink_size, dtype=np.int64)]
        order = range(i - 1, -1, -1) if rev else range(i)
        for j in order:
            for c in sel[j]:
                s = j * block_size + int(c) * chunk_size
                parts.append(np.arange(s, s + chunk_size, dtype=np.int64))
        p = np.concatenate(parts)
        out.append(np.unique(p) if dedup else p)
    return out


def test_block_zero_with_a_sink_prefix_is_caught(monkeypatch):
    _caught(monkeypatch, S.prefix_positions,
            lambda *a, **k: _prefix(*a, **k, first=0), PREFIX_PINS)


def test_deduplicated_sink_overlap_is_caught(monkeypatch):
    _caught(monkeypatch, S.prefix_positions,
            lambda *a, **k: _prefix(*a, **k, dedup=True), PREFIX_PINS)


def test_summaries_in_reverse_block_order_are_caught(monkeypatch):
    _caught(monkeypatch, S.prefix_positions,
            lambda *a, **k: _prefix(*a, **k, rev=True), PREFIX_PINS)


# ------------------------------------------------------------------ RoPE
def _rope_with(pairs="half", sign=1.0, exponent=2.0):
    def bad(x, pos, base):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        half = d // 2
        f = float(base) ** (-exponent * np.arange(half) / d)
        th = np.asarray(pos, np.float64)[:, None] * f[None, :]
        c, s = np.cos(th)[:, None, :], sign * np.sin(th)[:, None, :]
        if pairs == "half":
            x1, x2 = x[..., :half], x[..., half:]
            return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
        x1, x2 = x[..., 0::2], x[..., 1::2]           # interleaved pairs (x_2i, x_2i+1)
        y = np.empty_like(x)
        y[..., 0::2] = x1 * c - x2 * s
        y[..., 1::2] = x2 * c + x1 * s
        return y
    return bad


@pytest.mark.parametrize("kind", ["interleaved", "sign", "exponent"])
def test_rope_mistakes_are_caught(monkeypatch, kind):
    bad = {"interleaved": _rope_with(pairs="interleaved"), "sign": _rope_with(sign=-1.0),
           "exponent": _rope_with(exponent=1.0)}[kind]
    _caught(monkeypatch, R.rope, bad, ROPE_PINS)


def test_round_toward_zero_bf16_is_caught(monkeypatch):
    def bad(x):
        x = np.asarray(x, np.float64)
        m, e = np.frexp(x)
        scale = np.ldexp(1.0, e - 8)
        return np.where(x == 0.0, 0.0, np.trunc(x / scale) * scale)
    _caught(monkeypatch, OB.round_bf16, bad,
            [TA.test_round_bf16_ties_to_even_worked_values,
             TA.test_round_bf16_matches_torch_on_float32_values])


def test_llama3_factor_four_is_caught(monkeypatch):
    def bad(f):
        factor, low, high, orig = 4.0, 1.0, 4.0, 8192.0
        wavelen = 2.0 * np.pi / f
        smooth = (orig / wavelen - low) / (high - low)
        mid = (1.0 - smooth) * f / factor + smooth * f
        return np.where(wavelen < orig / high, f, np.where(wavelen > orig / low, f / factor, mid))
    _caught(monkeypatch, R._llama3, bad,
            [TA.test_llama3_scaling_regimes_at_base_500000_d128,
             TA.test_llama3_scaled_low_frequencies_rotate_as_one_eighth_of_the_position])


# ------------------------------------------------------------- attention
def _attend_with(scale=True, gqa="floor", log=np.log):
    def bad(q_hat, k_hat, v):
        q_hat, k_hat, v = (np.asarray(x, np.float64) for x in (q_hat, k_hat, v))
        hq, d = q_hat.shape
        hkv = k_hat.shape[1]
        out, lse = np.empty((hq, d)), np.empty(hq)
        for h in range(hq):
            g = h // (hq // hkv) if gqa == "floor" else h % hkv
            s = k_hat[:, g, :] @ q_hat[h] / (np.sqrt(d) if scale else 1.0)
            m = s.max()
            w = np.exp(s - m)
            out[h] = (w @ v[:, g, :]) / w.sum()
            lse[h] = m + log(w.sum())
        return out, lse
    return bad


@pytest.mark.parametrize("kind", ["no_scale", "gqa_modulo"])
def test_phase1_score_mistakes_are_caught(monkeypatch, kind):
    bad = _attend_with(scale=False) if kind == "no_scale" else _attend_with(gqa="modulo")
    _caught(monkeypatch, A.attend, bad, PHASE1_PINS)


@pytest.mark.parametrize("kind", ["no_diagonal", "no_prefix"])
def test_phase1_visible_set_mistakes_are_caught(monkeypatch, kind):
    def bad(prefix_i, i, r, block_size):
        lo = i * block_size
        if kind == "no_prefix":
            return np.arange(lo, lo + r + 1, dtype=np.int64)
        # the row misses itself (a row with nothing else visible keeps itself)
        keys = np.concatenate([np.asarray(prefix_i, np.int64), np.arange(lo, lo + r, dtype=np.int64)])
        return keys if len(keys) else np.array([lo], np.int64)
    _caught(monkeypatch, A.phase1_key_positions, bad, PHASE1_PINS)


def test_log2_lse_is_caught(monkeypatch):
    orig = A._shard_attend

    def bad(q_hat, k_hat, v, causal, offset=0):
        o, lse = orig(q_hat, k_hat, v, causal, offset)
        return o, lse / math.log(2.0)
    _caught(monkeypatch, orig, bad, PHASE2_PINS)


def test_unweighted_merge_is_caught(monkeypatch):
    def bad(o_parts, lse_parts):
        o_parts, lse_parts = np.asarray(o_parts), np.asarray(lse_parts)
        m = lse_parts.max(axis=0)
        return o_parts.mean(axis=0), m + np.log(np.exp(lse_parts - m).sum(axis=0))
    _caught(monkeypatch, A.lse_merge, bad, PHASE2_PINS)


def test_merge_sign_error_is_caught(monkeypatch):
    def bad(o_parts, lse_parts):
        o_parts, lse_parts = np.asarray(o_parts), np.asarray(lse_parts)
        m = lse_parts.max(axis=0)
        lse = m + np.log(np.exp(lse_parts - m).sum(axis=0))
        w = np.exp(lse[None] - lse_parts)             # exp(s_global - s_h): the inverted weight
        w = w / w.sum(axis=0, keepdims=True)
        return (w[..., None] * o_parts).sum(axis=0), lse
    _caught(monkeypatch, A.lse_merge, bad, PHASE2_PINS)


def test_non_causal_self_shard_is_caught(monkeypatch):
    orig = A._shard_attend

    def bad(q_hat, k_hat, v, causal, offset=0):
        return orig(q_hat, k_hat, v, False, offset)
    _caught(monkeypatch, orig, bad, PHASE2_PINS)


def test_decode_self_offset_mistake_is_caught(monkeypatch):
    orig = A._shard_attend

    def bad(q_hat, k_hat, v, causal, offset=0):
        return orig(q_hat, k_hat, v, causal, 0)       # query t sees self tokens 0..t only
    _caught(monkeypatch, orig, bad,
            [(TA.test_decode_merge_equals_masked_dense_attention, (7, 3)),
             TA.test_decode_zero_keys_average_exactly_the_visible_values])


def test_prefix_row_without_itself_is_caught(monkeypatch):
    def bad(q, k_hat, v, prefix_last, rows, base):
        prefix_last = np.asarray(prefix_last, np.int64)
        outs = []
        for e in rows:
            keys = prefix_last[:max(e, 1)]
            p = prefix_last[e]
            q_hat = A.rotate_bf16(np.asarray(q[np.array([p])], np.float64), np.array([p]), base)[0]
            outs.append(A.attend(q_hat, k_hat[keys], v[keys])[0])
        return np.stack(outs)
    _caught(monkeypatch, A.prefix_rows, bad,
            [TA.test_prefix_rows_of_a_contiguous_prefix_are_textbook_causal_attention,
             TA.test_prefix_rows_gather_equals_multiplicity_bias_dense])


def _rows_in_block_variant(strict_mask=False, drop_prefix=False, kv_mod=False):
    def bad(q, k_hat, v, prefix_i, i, rows, block_size, base):
        rows = np.asarray(rows, np.int64)
        lo = i * block_size
        r_max = int(rows.max())
        prefix_i = np.asarray(prefix_i, np.int64)[:0 if drop_prefix else None]
        keys = np.concatenate([prefix_i, np.arange(lo, lo + r_max + 1, dtype=np.int64)])
        kh = np.asarray(k_hat[keys], np.float64)
        vv = np.asarray(v[keys], np.float64)
        pos = lo + rows
        q_hat = A.rotate_bf16(np.asarray(q[pos], np.float64), pos, base)
        hq, d = q_hat.shape[1], q_hat.shape[2]
        hkv = kh.shape[1]
        own = np.arange(r_max + 1)[None, :]
        vis = np.ones((len(rows), len(keys)), bool)
        vis[:, len(prefix_i):] = (own < rows[:, None]) if strict_mask else (own <= rows[:, None])
        vis[:, len(prefix_i)] |= strict_mask       # keep every row non-empty
        out = np.empty((len(rows), hq, d))
        for h in range(hq):
            g = h % hkv if kv_mod else h // (hq // hkv)
            sc = np.where(vis, q_hat[:, h, :] @ kh[:, g, :].T / np.sqrt(d), -np.inf)
            w = np.exp(sc - sc.max(axis=1, keepdims=True))
            out[:, h, :] = (w @ vv[:, g, :]) / w.sum(axis=1, keepdims=True)
        return out
    return bad


@pytest.mark.parametrize("kind", ["strict_mask", "drop_prefix", "kv_mod"])
def test_rows_in_block_mistakes_are_caught(monkeypatch, kind):
    _caught(monkeypatch, A.phase1_rows_in_block, _rows_in_block_variant(**{kind: True}),
            ROWS_IN_BLOCK_PINS)


# ------------------------------------------------------ selection methods
from oracle import selection_variants as SV
from tests import test_oracle_selection_variants as TV

VARIANT_PINS = [(TV.test_mean_idf_exact_order_equals_the_float_definition, (0,)),
                (TV.test_mean_idf_exact_order_equals_the_float_definition, (4,)),
                TV.test_mean_idf_loses_the_answer_of_figure2,
                (TV.test_entropy_exact_order_equals_scipy_entropy, (0,)),
                (TV.test_entropy_exact_order_equals_scipy_entropy, (4,)),
                TV.test_entropy_closed_forms,
                TV.test_uniform_selection_is_uniform_and_seeded,
                TV.test_splitmix64_known_answers,
                TV.test_even_spacing_closed_form]


def _replace_variant(monkeypatch, original, replacement):
    for mod in (SV, TV):
        for name, val in list(vars(mod).items()):
            if val is original:
                monkeypatch.setattr(mod, name, replacement)


def _caught_variant(monkeypatch, original, replacement):
    _replace_variant(monkeypatch, original, replacement)
    assert _failing(VARIANT_PINS), f"no pin caught the planted mistake in {original.__name__}"


def test_mean_idf_key_of_the_maximum_df_is_caught(monkeypatch):
    orig = SV.mean_idf_keys

    def bad(tokens, n_blocks, block_size, chunk_size, vocab_size):
        # the product replaced by the largest df: the chunk's most common token
        tokens = np.asarray(tokens)
        df = S.document_frequency(tokens, n_blocks, block_size, vocab_size)
        n_chunks = block_size // chunk_size
        return [[max(int(df[t]) for t in tokens[j * block_size + c * chunk_size:
                                                   j * block_size + (c + 1) * chunk_size])
                 for c in range(n_chunks)] for j in range(n_blocks)]
    _caught_variant(monkeypatch, orig, bad)


def test_entropy_key_of_distinct_count_is_caught(monkeypatch):
    def bad(tokens, n_blocks, block_size, chunk_size):
        # fewer distinct ids as the better chunk: the order inverted
        tokens = np.asarray(tokens)
        n_chunks = block_size // chunk_size
        return [[len(set(tokens[j * block_size + c * chunk_size:
                                j * block_size + (c + 1) * chunk_size].tolist()))
                 for c in range(n_chunks)] for j in range(n_blocks)]
    _caught_variant(monkeypatch, SV.entropy_keys, bad)


def test_uniform_keys_without_the_block_in_the_counter_is_caught(monkeypatch):
    def bad(seed, n_blocks, n_chunks):
        # every block draws the same counters
        return [[SV.splitmix64(seed, c + 1) for c in range(n_chunks)] for _ in range(n_blocks)]
    _caught_variant(monkeypatch, SV.uniform_keys, bad)


def test_splitmix64_with_a_wrong_finaliser_shift_is_caught(monkeypatch):
    def bad(seed, n):
        # still a good generator (balanced, uncorrelated bits): only the last
        # xor-shift of the finaliser differs from the published one
        z = (seed + n * SV.GOLDEN_GAMMA) & SV.MASK64
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & SV.MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & SV.MASK64
        return z ^ (z >> 29)
    _caught_variant(monkeypatch, SV.splitmix64, bad)


def test_splitmix64_counting_from_zero_is_caught(monkeypatch):
    orig = SV.splitmix64

    def bad(seed, n):
        return orig(seed, n - 1)       # the state read before its first advance
    _caught_variant(monkeypatch, SV.splitmix64, bad)


def test_even_spacing_off_by_half_is_caught(monkeypatch):
    orig = SV.select_variant

    def bad(method, tokens, n_blocks, block_size, chunk_size, budget_chunks, vocab_size, seed=0):
        if method != "even":
            return orig(method, tokens, n_blocks, block_size, chunk_size, budget_chunks, vocab_size, seed)
        n_chunks = block_size // chunk_size
        k = min(budget_chunks, n_chunks)
        row = [min(n_chunks - 1, (2 * m + 1) * n_chunks // (2 * k)) for m in range(k)]
        return np.array([row] * n_blocks, dtype=np.int64).reshape(n_blocks, k)
    _caught_variant(monkeypatch, orig, bad)
