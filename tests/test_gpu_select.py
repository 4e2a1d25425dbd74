"""GPU parity of Max-IDF selection: bit-exact sel, chunk min-df and df against
the oracle, on every workload and on structured inputs where the scores
spread out (the Zipf streams make almost every chunk tie at min df 1)."""
import numpy as np
import pytest

import workloads as W
from oracle import selection as OS
from tests.gpu_cases import log, torch_cuda

pytestmark = pytest.mark.gpu


def run_select(tok, n_blocks, block_size, chunk, k, vocab):
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    g = B.make_geom(n_blocks, block_size, chunk, k, 64 if block_size * n_blocks >= 64 else 0, vocab)
    kept = B.pulsar_kept_chunks(g)
    dev = torch.device("cuda")
    t = torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).to(dev)
    sel = torch.full((n_blocks, max(kept, 1)), -7, dtype=torch.int32, device=dev)
    cm = torch.full((n_blocks, block_size // chunk), -7, dtype=torch.int32, device=dev)
    df = torch.full((vocab,), -7, dtype=torch.int32, device=dev)
    ws = torch.full((B.pulsar_workspace_bytes(g, None),), 0xAB, dtype=torch.uint8, device=dev)
    log(f"[select] N={n_blocks} b={block_size} chunk={chunk} k={k} V={vocab}")
    B.pulsar_select(g, t, sel if kept > 0 else None, cm, df, ws)
    torch.cuda.synchronize()
    status = int(ws[:4].view(torch.int32).item())
    return sel[:, :kept].cpu().numpy(), cm.cpu().numpy(), df.cpu().numpy(), status


def check(tok, n_blocks, block_size, chunk, k, vocab):
    sel, cm, df, status = run_select(tok, n_blocks, block_size, chunk, k, vocab)
    want_sel, want_df, _ = OS.select(tok, n_blocks, block_size, chunk, k, vocab)
    want_cm = OS.chunk_min_df(tok, want_df, n_blocks, block_size, chunk)
    np.testing.assert_array_equal(df, want_df)
    np.testing.assert_array_equal(cm, want_cm)
    np.testing.assert_array_equal(sel, want_sel)
    assert status == 0
    return sel


@pytest.mark.parametrize("name", ["tiny", "32k", "128k", "128k_star", "512k"])
def test_select_workloads(name):
    w = W.WORKLOADS[name]
    check(W.tokens(w), w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks, w.vocab_size)


@pytest.mark.parametrize("vocab", [16, 64, 512, 4096])
def test_select_small_vocab_spreads_scores(vocab):
    tok = W.small_vocab_tokens(vocab, 5, 1024, vocab)
    check(tok, 5, 1024, 32, 4, vocab)


@pytest.mark.parametrize("per_block", [1, 4, 16])
def test_select_filler_picks_planted(per_block):
    tok, planted = W.filler_planted_tokens(per_block, 4, 2048, 32, per_block)
    sel = check(tok, 4, 2048, 32, per_block, 4096)
    np.testing.assert_array_equal(sel, planted)


def test_select_edge_budgets_and_ties():
    rng = np.random.default_rng(4)
    tok = rng.integers(0, 300, size=4 * 512).astype(np.int32)
    check(tok, 4, 512, 32, 16, 300)        # k == C: keep everything
    check(tok, 4, 512, 32, 40, 300)        # k > C
    check(tok, 4, 512, 32, 0, 300)         # Star setting: nothing kept
    check(np.zeros(4 * 512, np.int32), 4, 512, 32, 5, 8)   # all ties: first k chunks
    check(tok, 1, 2048, 32, 8, 300)        # one block: every df is 1


def test_select_sixteen_blocks_random_df():
    rng = np.random.default_rng(9)
    # per-block pools of different sizes give chunk min-df values across 1..16
    blocks = []
    for j in range(16):
        pool = rng.integers(0, 2000, size=int(rng.integers(20, 400)))
        blocks.append(rng.choice(pool, size=2048))
    tok = np.concatenate(blocks).astype(np.int32)
    check(tok, 16, 2048, 32, 8, 2000)


def test_select_ragged_chunk_count_and_large_vocab():
    rng = np.random.default_rng(5)
    tok = rng.integers(0, 700000, size=3 * 32 * 300).astype(np.int32)   # 300 chunks: not a wave multiple
    check(tok, 3, 32 * 300, 32, 37, 700000)


def test_select_flags_out_of_range_ids():
    tok = np.arange(4 * 256, dtype=np.int32) % 50
    tok[17] = 50          # == V
    tok[300] = -3
    sel, cm, df, status = run_select(tok, 4, 256, 32, 2, 50)
    assert status == 1
    ok = tok.copy()
    # the count skips the bad ids
    want_df = np.zeros(50, np.int64)
    for j in range(4):
        blk = ok[j * 256:(j + 1) * 256]
        want_df[np.unique(blk[(blk >= 0) & (blk < 50)])] += 1
    np.testing.assert_array_equal(df, want_df)


def test_select_is_deterministic():
    w = W.WORKLOADS["128k"]
    tok = W.tokens(w)
    a = run_select(tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks, w.vocab_size)
    b = run_select(tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks, w.vocab_size)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("chunk", [8, 16, 24, 40, 64, 96])
def test_select_chunk_sizes(chunk):
    """Chunk sizes that divide the 64-lane wave (one lane per token, a min over
    the chunk's lanes) and sizes that do not (one thread per chunk), with scores
    spread over 1..N by a small vocabulary."""
    n_blocks, n_chunks = 6, 40
    b = chunk * n_chunks
    tok = W.small_vocab_tokens(chunk, n_blocks, b, 96)
    sel, cm, df, status = run_select(tok, n_blocks, b, chunk, 7, 96)
    want_sel, want_df, _ = OS.select(tok, n_blocks, b, chunk, 7, 96)
    np.testing.assert_array_equal(df, want_df)
    np.testing.assert_array_equal(cm, OS.chunk_min_df(tok, want_df, n_blocks, b, chunk))
    np.testing.assert_array_equal(sel, want_sel)
    assert status == 0


@pytest.mark.parametrize("n_blocks", [5, 8])
def test_select_without_chunk_scores_out(n_blocks):
    """chunk_min_df = NULL and df = NULL: the scores and df go through the
    workspace; same selection."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    tok = W.small_vocab_tokens(3, n_blocks, 1024, 64)
    g = B.make_geom(n_blocks, 1024, 32, 6, 64, 64)
    dev = torch.device("cuda")
    t = torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).to(dev)
    sel = torch.full((n_blocks, 6), -7, dtype=torch.int32, device=dev)
    ws = torch.full((B.pulsar_workspace_bytes(g, None),), 0xAB, dtype=torch.uint8, device=dev)
    B.pulsar_select(g, t, sel, None, None, ws)
    torch.cuda.synchronize()
    want_sel, _, _ = OS.select(tok, n_blocks, 1024, 32, 6, 64)
    np.testing.assert_array_equal(sel.cpu().numpy(), want_sel)
