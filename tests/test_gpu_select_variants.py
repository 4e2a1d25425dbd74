"""GPU parity of the other selection methods (mean IDF, entropy, uniform, evenly
spaced): bit-exact sel against the oracle on the workloads and on token streams
whose scores spread out, the status word for out-of-range ids, and Phase 1 fed
by a mean-IDF selection."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import selection as OS
from oracle import selection_variants as OV
from tests.gpu_cases import Case, assert_close, log, torch_cuda

pytestmark = pytest.mark.gpu

METHODS = ["mean_idf", "entropy", "uniform", "even"]


def run_method(method, tok, n_blocks, block_size, chunk, k, vocab, seed=0):
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    g = B.make_geom(n_blocks, block_size, chunk, k, 64 if block_size * n_blocks >= 64 else 0, vocab)
    kept = B.pulsar_kept_chunks(g)
    dev = torch.device("cuda")
    t = torch.from_numpy(np.ascontiguousarray(tok, dtype=np.int32)).to(dev)
    sel = torch.full((n_blocks, max(kept, 1)), -7, dtype=torch.int32, device=dev)
    ws = torch.full((B.pulsar_workspace_bytes(g, None),), 0xAB, dtype=torch.uint8, device=dev)
    log(f"[select] {method} N={n_blocks} b={block_size} chunk={chunk} k={k} V={vocab} seed={seed}")
    B.pulsar_select_method(g, method, seed, t, sel if kept > 0 else None, ws)
    torch.cuda.synchronize()
    status = int(ws[:4].view(torch.int32).item())
    return sel[:, :kept].cpu().numpy(), status


def check(method, tok, n_blocks, block_size, chunk, k, vocab, seed=0):
    sel, status = run_method(method, tok, n_blocks, block_size, chunk, k, vocab, seed)
    want = OV.select_variant(method, tok, n_blocks, block_size, chunk, k, vocab, seed=seed)
    np.testing.assert_array_equal(sel, want)
    assert status == 0
    return sel


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("name", ["tiny", "32k", "128k", "512k"])
def test_methods_on_the_workloads(method, name):
    w = W.WORKLOADS[name]
    check(method, W.tokens(w), w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
          w.vocab_size, seed=w.seed)


@pytest.mark.parametrize("method", METHODS)
@pytest.mark.parametrize("vocab", [8, 64, 4096])
def test_methods_where_scores_spread(method, vocab):
    # small vocabularies give every df in 1..N and repeated ids inside chunks
    tok = W.small_vocab_tokens(vocab, 6, 1024, vocab)
    check(method, tok, 6, 1024, 32, 5, vocab, seed=vocab)


@pytest.mark.parametrize("method", METHODS)
def test_methods_on_ragged_and_edge_budgets(method):
    rng = np.random.default_rng(11)
    tok = rng.integers(0, 40, size=3 * 16 * 300).astype(np.int32)   # 300 chunks of 16
    check(method, tok, 3, 16 * 300, 16, 37, 40, seed=3)
    check(method, tok, 3, 16 * 300, 16, 300, 40, seed=3)          # k == C: everything
    check(method, tok, 3, 16 * 300, 16, 1000, 40, seed=3)         # k > C
    check(method, tok, 3, 16 * 300, 16, 0, 40, seed=3)            # k == 0: the status word is still cleared
    check(method, np.zeros(4 * 256, np.int32), 4, 256, 32, 3, 8, seed=5)   # all ties


def test_uniform_seeds_differ_and_repeat():
    w = W.WORKLOADS["tiny"]
    tok = W.tokens(w)
    a, _ = run_method("uniform", tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
                      w.vocab_size, seed=1)
    b, _ = run_method("uniform", tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
                      w.vocab_size, seed=1)
    c, _ = run_method("uniform", tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
                      w.vocab_size, seed=2)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


@pytest.mark.parametrize("method", ["mean_idf", "entropy"])
def test_out_of_range_ids_set_the_status_word(method):
    tok = np.arange(4 * 256, dtype=np.int32) % 50
    tok[17] = 50
    tok[300] = -3
    sel, status = run_method(method, tok, 4, 256, 32, 2, 50)
    assert status == 1
    want = OV.select_variant(method, tok, 4, 256, 32, 2, 50)
    np.testing.assert_array_equal(sel, want)


def test_phase1_with_a_mean_idf_selection():
    """Phase 1 takes any selection: with the mean-IDF summaries every row equals
    the oracle's attention over the prefix those summaries give."""
    torch = torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name="mean_idf_p1", n_blocks=3, block_size=512, budget_chunks=3,
                n_planted=0, vocab_size=64)
    case = Case(w)
    case.path.select_method("mean_idf")
    case.path.phase1()
    torch.cuda.synchronize()
    sel = OV.select_variant("mean_idf", case.tok, w.n_blocks, w.block_size, w.chunk_size,
                            w.budget_chunks, w.vocab_size)
    np.testing.assert_array_equal(case.path.sel[:, :w.k_eff].cpu().numpy(), sel)
    pre = OS.prefix_positions(sel, w.n_blocks, w.block_size, w.chunk_size, w.sink_size)
    max_sel, _, _ = OS.select(case.tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
                              w.vocab_size)
    assert not np.array_equal(sel, max_sel)          # a different prefix from Max-IDF
    khat = case.oracle_khat().astype(np.float64)
    q = W.bf16_bits_to_f64(case.q)
    v = W.bf16_bits_to_f64(case.v)
    o = case.path.o.cpu().numpy()
    for i in range(w.n_blocks):
        want = OA.phase1_block_dense(q, khat, v, pre[i], i, w.block_size, w.rope_base)
        assert_close(o[i * w.block_size:(i + 1) * w.block_size], want, f"mean-IDF phase1 block {i}")
