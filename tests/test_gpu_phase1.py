"""GPU parity of Phase-1 encoding and the retained cache against the oracle.

Small geometries are compared on every row and head (they span several
64-key tiles and end on ragged prefix / block tails); the full-size workloads
run in the benchmark's launch configuration and are compared on sampled rows
(tile edges, first/last rows of every block, seeded rows), all heads."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import selection as OS
from tests.gpu_cases import (Case, F32Rows, assert_close, dense_rows, log, rope_spec,
                              torch_cuda)

pytestmark = pytest.mark.gpu


def _cache_check(case):
    """Retained K must be the oracle's bf16 rotation (float32 vs float64 rotation may
    round a rare element to the neighbouring bf16 value); retained V is an exact copy."""
    w = case.w
    kc = case.path.k_cache[0].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    vc = case.path.v_cache[0].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    # retained values are stored d-major: [N][Hkv][d][b]
    want_v = case.v.reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim).transpose(0, 2, 3, 1)
    np.testing.assert_array_equal(vc, want_v)
    khat = case.oracle_khat().reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim)
    khat = khat.transpose(0, 2, 1, 3)
    got = W.bf16_bits_to_f32(kc)
    diff = got != khat
    frac = diff.mean()
    log(f"[parity] retained K: {diff.sum()} of {diff.size} elements differ by rounding ({frac:.2e})")
    assert frac < 1e-3
    if diff.any():
        ulp = np.abs(khat[diff]) * 2.0 ** -7
        assert np.all(np.abs(got[diff] - khat[diff]) <= ulp * 1.0001)
    return khat


def _full_compare(case):
    w = case.w
    sel, _, _ = case.oracle_selection()
    pre = OS.prefix_positions(sel, w.n_blocks, w.block_size, w.chunk_size, w.sink_size)
    khat = case.oracle_khat().astype(np.float64)
    q = W.bf16_bits_to_f64(case.q)
    v = W.bf16_bits_to_f64(case.v)
    o = case.path.o.cpu().numpy()
    for i in range(w.n_blocks):
        want = OA.phase1_block_dense(q, khat, v, pre[i], i, w.block_size, w.rope_base)
        assert_close(o[i * w.block_size:(i + 1) * w.block_size], want, f"{w.name} phase1 block {i}")


def _sampled_compare(case, rows):
    """Sampled rows against the oracle, all heads, one block at a time (the rows
    of a block share their key list, so the oracle takes them together)."""
    import torch
    w = case.w
    sel, _, _ = case.oracle_selection()
    got_sel = case.path.sel[:, :w.k_eff].cpu().numpy()
    np.testing.assert_array_equal(got_sel, sel)
    pre = OS.prefix_positions(sel, w.n_blocks, w.block_size, w.chunk_size, w.sink_size)
    khat = case.oracle_khat()
    q, v = F32Rows(case.q), F32Rows(case.v)
    got_all, want_all = [], []
    for i in sorted({i for i, _ in rows}):
        rr = [r for (j, r) in rows if j == i]
        pos = torch.tensor([i * w.block_size + r for r in rr], device="cuda")
        got_all.append(case.path.o.index_select(0, pos).cpu().numpy())
        want_all.append(OA.phase1_rows_in_block(q, khat, v, pre[i], i, rr, w.block_size,
                                                rope_spec(w)))
    assert_close(np.concatenate(got_all), np.concatenate(want_all),
                 f"{w.name} phase1 sampled rows ({len(rows)} rows x {w.n_q_heads} heads)")


SMALL = {
    # name: geometry overrides of the tiny workload
    "tiny": {},
    "ragged_g2_d64": dict(n_blocks=3, block_size=320, budget_chunks=3, n_planted=0),
    "g1_d64": dict(n_blocks=3, block_size=256, n_q_heads=2, n_kv_heads=2, budget_chunks=2, n_planted=0),
    "g4_d128": dict(n_blocks=3, block_size=384, n_q_heads=8, n_kv_heads=2, head_dim=128,
                    budget_chunks=5, n_planted=0),
    "g8_d128": dict(n_blocks=2, block_size=256, n_q_heads=8, n_kv_heads=1, head_dim=128,
                    budget_chunks=1, n_planted=0),
    "single_block": dict(n_blocks=1, block_size=448, n_planted=0, budget_chunks=4),
    "star_small": dict(n_blocks=4, block_size=256, sink_size=256, budget_chunks=0, n_planted=0),
    "sink96_odd": dict(n_blocks=4, block_size=192, sink_size=96, budget_chunks=1, n_planted=0),
    # no sink: block i > 0 sees only the summaries of earlier blocks
    "no_sink": dict(n_blocks=3, block_size=256, sink_size=0, budget_chunks=2, n_planted=0),
    # 16-token chunks; a block of 5.5 key tiles ends on a half tile
    "ragged_352_chunk16": dict(n_blocks=3, block_size=352, chunk_size=16, budget_chunks=5,
                               n_planted=0),
    # 16 query heads on one KV head: two head groups per workgroup row tile
    "g16_d64": dict(n_blocks=2, block_size=192, n_q_heads=16, n_kv_heads=1, budget_chunks=1,
                    n_planted=0),
    # budget above the chunk count: every chunk kept, so the sink tokens appear
    # twice in the prefix (once as the sink, once inside block 0's summary)
    "keep_all": dict(n_blocks=3, block_size=128, budget_chunks=100, n_planted=0),
    # d = 128 with a block of 5.5 key tiles: the last own tile of the last KV head
    # of the last block runs past the cache, and prefixes end on half tiles
    "ragged_d128": dict(n_blocks=3, block_size=352, n_q_heads=8, n_kv_heads=2, head_dim=128,
                        budget_chunks=3, n_planted=0),
    # d = 128, a 96-token sink: every prefix ends on a half tile
    "sink96_d128": dict(n_blocks=4, block_size=192, sink_size=96, n_q_heads=4, n_kv_heads=2,
                        head_dim=128, budget_chunks=1, n_planted=0),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_phase1_small_all_rows(name):
    w = W.with_(W.WORKLOADS["tiny"], name=name, **SMALL[name])
    case = Case(w)
    case.run()
    _cache_check(case)
    _full_compare(case)


def test_phase1_is_deterministic():
    torch = torch_cuda()
    case = Case(W.WORKLOADS["tiny"])
    case.run()
    a = case.path.o.clone()
    case.run()
    assert torch.equal(a, case.path.o)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["32k", "128k", "128k_star", "512k"])
def test_phase1_full_size_sampled(name):
    """Full-size workloads in the benchmark's launch configuration: the first and
    last 64 rows of a block plus one seeded row in every 96 rows (every row tile),
    all heads, on every block (512K: on the first, a middle and the last block,
    and a sparse sample of the others)."""
    w = W.WORKLOADS[name]
    case = Case(w, extra_seqs=False)
    case.run()
    blocks = None if w.n_blocks <= 8 else [0, w.n_blocks // 2, w.n_blocks - 1]
    rows = dense_rows(w, blocks=blocks, seed=w.seed)
    _sampled_compare(case, rows)


def test_prepare_then_attend_equals_encode():
    """The two halves of the Phase-1 call, issued apart, give encode's results bit for bit."""
    torch = torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name="split", **SMALL["ragged_g2_d64"])
    case = Case(w)
    case.run()
    o, kc, vc = case.path.o.clone(), case.path.k_cache.clone(), case.path.v_cache.clone()
    case.path.o.zero_()
    case.path.k_cache.zero_()
    case.path.v_cache.zero_()
    case.path.phase1_prepare()
    case.path.phase1_attend()
    torch.cuda.synchronize()
    assert torch.equal(case.path.k_cache, kc) and torch.equal(case.path.v_cache, vc)
    assert torch.equal(case.path.o, o)
