"""GPU parity of Phase-2 query attention and the LSE merge against the oracle
(per-shard partials merged exactly; the merged output and log-sum-exp are
compared), plus the merge kernel alone on random partials."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import LSE_ABS, Case, assert_close, log, torch_cuda

pytestmark = pytest.mark.gpu


def _oracle_merged(case, seq, khat_cache=None):
    w = case.w
    if seq == 0:
        if khat_cache is None:
            khat = case.oracle_khat().astype(np.float64)
            khat_cache = khat.reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim).transpose(0, 2, 1, 3)
        kc = khat_cache
        vc = W.bf16_bits_to_f64(case.v).reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim)
        vc = vc.transpose(0, 2, 1, 3)
    else:
        kc = W.bf16_bits_to_f64(W.extra_cache(w, seq, "k"))
        vc = W.bf16_bits_to_f64(W.extra_cache(w, seq, "v"))
    qq = W.bf16_bits_to_f64(case.qq[seq])
    ks = W.bf16_bits_to_f64(case.kq[seq]) if case.with_self else None
    vs = W.bf16_bits_to_f64(case.vq[seq]) if case.with_self else None
    parts = OA.phase2_partials(qq, w.context_len, kc, vc, ks, vs, w.rope_base)
    return OA.lse_merge([p[0] for p in parts], [p[1] for p in parts])


def _compare(case, seqs):
    o = case.path.o_q.cpu().numpy()
    lse = case.path.lse_q.cpu().numpy()
    for s in seqs:
        want_o, want_lse = _oracle_merged(case, s)
        assert_close(o[s], want_o, f"{case.w.name} phase2 merged O seq {s}")
        assert_close(lse[s], want_lse, f"{case.w.name} phase2 merged LSE seq {s}",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)


SMALL = {
    "tiny": {},
    "ragged_shards": dict(n_blocks=3, block_size=1000, chunk_size=8, budget_chunks=15, n_planted=0,
                          q_len=5),
    "decode_batch": dict(n_blocks=5, block_size=512, q_len=1, batch=3, n_planted=0),
    "g4_d128_lq64": dict(n_blocks=2, block_size=640, n_q_heads=8, n_kv_heads=2, head_dim=128,
                         q_len=64, budget_chunks=2, n_planted=0),
    "g8_d128_lq40": dict(n_blocks=2, block_size=384, n_q_heads=8, n_kv_heads=1, head_dim=128,
                         q_len=40, budget_chunks=2, n_planted=0),
    # decode form (every query row of a KV head in one 32-row wave, two waves
    # splitting each tile's subtiles): a 32-key part leaves the second wave empty
    "decode_d128_short": dict(n_blocks=3, block_size=96, n_q_heads=8, n_kv_heads=2, head_dim=128,
                              q_len=1, batch=2, budget_chunks=1, n_planted=0),
    "decode_rows32": dict(n_blocks=3, block_size=256, n_q_heads=8, n_kv_heads=2, q_len=8,
                          budget_chunks=2, n_planted=0),
    "g16_lq3": dict(n_blocks=2, block_size=256, n_q_heads=16, n_kv_heads=1, q_len=3,
                    budget_chunks=1, n_planted=0),
    "no_sink_batch2": dict(n_blocks=3, block_size=256, sink_size=0, budget_chunks=2, q_len=7,
                           batch=2, n_planted=0),
    # more self tiles (5) than shard tiles (4): the parts past the shards hold self
    # tiles only, and the last one holds keys that the early query tokens must not
    # see (those rows give an empty part, LSE -inf)
    "self_spans_parts": dict(n_blocks=2, block_size=128, budget_chunks=1, q_len=300,
                             n_planted=0),
}


@pytest.mark.parametrize("with_self", [True, False])
@pytest.mark.parametrize("name", list(SMALL))
def test_phase2_small(name, with_self):
    w = W.with_(W.WORKLOADS["tiny"], name=name, **SMALL[name])
    case = Case(w, with_self=with_self)
    case.run()
    _compare(case, range(w.batch))


def test_phase2_full_size_32k():
    case = Case(W.WORKLOADS["32k"])
    case.run()
    _compare(case, [0])


@pytest.mark.timeout(600)
def test_phase2_full_size_128k_star_and_pulsar_retain_the_same_cache():
    """The 128K Pulsar and Star Attention workloads differ only in what each block
    attends to in Phase 1; each block keeps its own keys and values either way
    ("Dropping the Anchor ..." Section 2.2 and the Abstract: the retained cache is
    Star Attention's), so the retained caches must be bit-identical, and so must
    the Phase-2 answer over them.  Both are checked on the GPU, and the 128K
    Star answer against the oracle, every head."""
    torch = torch_cuda()
    pulsar = Case(W.WORKLOADS["128k"])
    pulsar.run()
    _compare(pulsar, [0])
    kc, vc = pulsar.path.k_cache.clone(), pulsar.path.v_cache.clone()
    o, lse = pulsar.path.o_q.clone(), pulsar.path.lse_q.clone()
    del pulsar
    torch.cuda.empty_cache()
    star = Case(W.WORKLOADS["128k_star"])
    star.run()
    assert torch.equal(star.path.k_cache, kc), "retained K differs between Pulsar and Star"
    assert torch.equal(star.path.v_cache, vc), "retained V differs between Pulsar and Star"
    log("[parity] 128k and 128k_star retained K/V caches bit-identical")
    assert torch.equal(star.path.o_q, o) and torch.equal(star.path.lse_q, lse)
    log("[parity] 128k and 128k_star Phase-2 merged O/LSE bit-identical")
    _compare(star, [0])


def test_phase2_full_size_decode_batch():
    w = W.WORKLOADS["512k"]
    case = Case(w)
    case.run()
    _compare(case, [0, 1, w.batch - 1])


def test_merge_kernel_alone():
    """Merge against the oracle's merge.  Empty parts (lse = -inf) carry NaN output
    rows on the device: the definition gives them weight 0, so the oracle sees any
    finite row there (zeros) and the kernel must not let the NaN through.  Part
    counts above 64 exercise the lane-strided LSE pass."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    rng = np.random.default_rng(3)
    for (bsz, n_parts, lq, hq, d) in [(2, 7, 5, 4, 64), (1, 33, 64, 32, 128), (3, 1, 1, 8, 128),
                                      (2, 70, 3, 8, 128), (1, 131, 2, 4, 64)]:
        o_part = rng.standard_normal((bsz, n_parts, lq, hq, d)).astype(np.float32)
        lse_part = (rng.standard_normal((bsz, n_parts, lq, hq)) * 30).astype(np.float32)
        o_dev = o_part.copy()
        if n_parts > 1:
            for p in {0, n_parts // 2, n_parts - 1}:
                lse_part[:, p, 0, 0] = -np.inf       # an empty part contributes nothing
                o_part[:, p, 0, 0] = 0.0
                o_dev[:, p, 0, 0] = np.nan
        dev = torch.device("cuda")
        op, lp = torch.from_numpy(o_dev).to(dev), torch.from_numpy(lse_part).to(dev)
        o = torch.empty((bsz, lq, hq, d), device=dev)
        lse = torch.empty((bsz, lq, hq), device=dev)
        log(f"[merge] B={bsz} parts={n_parts} Lq={lq} Hq={hq} d={d}")
        B.pulsar_lse_merge(bsz, n_parts, lq, hq, d, op, lp, o, lse)
        torch.cuda.synchronize()
        want_o, want_lse = OA.lse_merge(np.moveaxis(o_part, 1, 0), np.moveaxis(lse_part, 1, 0))
        assert_close(o.cpu().numpy(), want_o, "merge O", max_abs=1e-5, mean_abs=1e-6)
        assert_close(lse.cpu().numpy(), want_lse, "merge LSE", max_abs=1e-4, mean_abs=1e-5)


def test_merge_of_only_empty_parts_is_zero_with_lse_minus_inf():
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    dev = torch.device("cuda")
    op = torch.full((1, 3, 1, 2, 64), float("nan"), device=dev)
    lp = torch.full((1, 3, 1, 2), float("-inf"), device=dev)
    o = torch.empty((1, 1, 2, 64), device=dev)
    lse = torch.empty((1, 1, 2), device=dev)
    B.pulsar_lse_merge(1, 3, 1, 2, 64, op, lp, o, lse)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item()
    assert torch.all(lse == float("-inf")).item()


@pytest.mark.parametrize("hq,hkv,d,lq", [(4, 2, 64, 150), (8, 2, 128, 70), (4, 2, 64, 1)])
def test_query_over_the_self_shard_only(hq, hkv, d, lq):
    """No retained shard (n_shards = 0): one part, the causal self shard, spread
    over several tiles for the longer queries (the last case is the decode form)."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    w = W.with_(W.WORKLOADS["tiny"], name="self_only", n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                q_len=lq, batch=2)
    qq, kq, vq = W.query(w)
    attn = B.make_attn(hq, hkv, d, w.rope_base, 0)
    n_parts = B.pulsar_phase2_num_parts(attn, w.batch, 0, 0, lq, True)
    assert n_parts == 1
    dev = torch.device("cuda")
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    o_part = torch.full((w.batch, 1, lq, hq, d), float("nan"), device=dev)
    lse_part = torch.full((w.batch, 1, lq, hq), float("nan"), device=dev)
    ws = torch.empty(B.pulsar_phase2_workspace_bytes(attn, w.batch, lq, True), dtype=torch.uint8,
                     device=dev)
    log(f"[self-only] hq={hq} hkv={hkv} d={d} lq={lq}")
    B.pulsar_phase2_query(attn, w.batch, 0, 0, bf(qq), lq, w.context_len, None, None, bf(kq), bf(vq),
                          o_part, lse_part, n_parts, ws)
    torch.cuda.synchronize()
    o, lse = o_part.cpu().numpy(), lse_part.cpu().numpy()
    empty = np.zeros((0, hkv, 8, d))
    for s in range(w.batch):
        (want_o, want_lse), = OA.phase2_partials(W.bf16_bits_to_f64(qq[s]), w.context_len, empty, empty,
                                                 W.bf16_bits_to_f64(kq[s]), W.bf16_bits_to_f64(vq[s]),
                                                 w.rope_base)
        assert_close(o[s, 0], want_o, f"self-only O seq {s}")
        assert_close(lse[s, 0], want_lse, f"self-only LSE seq {s}", max_abs=LSE_ABS, mean_abs=LSE_ABS)
