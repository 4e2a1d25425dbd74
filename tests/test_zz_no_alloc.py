"""The no-allocation Phase-2 query (pulsar_phase2_query_noalloc) against the
workspace form (pulsar_phase2_query) through the C ABI: the same inputs give
bit-identical partial outputs and log-sum-exps, on two calls in a row, the
second on a smaller problem (the fixed array keeps the first call's contents),
and the merged result of the no-allocation call is checked against the oracle.
The entry point also replays from a HIP graph."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import LSE_ABS, assert_close, log, torch_cuda

pytestmark = pytest.mark.gpu

# (batch, n_shards, shard_len, q_len, hq, hkv, d, with_self): a large first call,
# then a smaller one
CALLS = [
    (2, 5, 1000, 100, 8, 2, 128, True),
    (1, 3, 264, 7, 4, 2, 64, True),
    (3, 2, 512, 1, 8, 2, 128, False),
]


def _inputs(batch, n_shards, shard_len, q_len, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    bf = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return (bf((batch, q_len, hq, d)), bf((batch, n_shards, hkv, shard_len, d)),
            bf((batch, n_shards, hkv, d, shard_len)), bf((batch, q_len, hkv, d)),
            bf((batch, q_len, hkv, d)))


def _run(noalloc, attn, shape, tensors):
    import torch

    from long_context_blockwise_max_amd import binding as B
    batch, n_shards, shard_len, q_len, hq, hkv, d, with_self = shape
    qq, kc, vc, ks, vs = tensors
    n_parts = B.pulsar_phase2_num_parts(attn, batch, n_shards, shard_len, q_len, with_self)
    o_part = torch.full((batch, n_parts, q_len, hq, d), float("nan"), device="cuda")
    lse_part = torch.full((batch, n_parts, q_len, hq), float("nan"), device="cuda")
    args = (attn, batch, n_shards, shard_len, qq, q_len, n_shards * shard_len, kc, vc,
            ks if with_self else None, vs if with_self else None, o_part, lse_part, n_parts)
    if noalloc:
        B.pulsar_phase2_query_noalloc(*args)
    else:
        ws = torch.empty(B.pulsar_phase2_workspace_bytes(attn, batch, q_len, with_self),
                         dtype=torch.uint8, device="cuda")
        B.pulsar_phase2_query(*args, ws)
    torch.cuda.synchronize()
    return o_part, lse_part, n_parts


def test_noalloc_query_equals_the_workspace_query():
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to("cuda")
    for j, shape in enumerate(CALLS):
        batch, n_shards, shard_len, q_len, hq, hkv, d, with_self = shape
        log(f"[noalloc] call {j}: B={batch} shards={n_shards}x{shard_len} Lq={q_len} "
            f"Hq/Hkv/d={hq}/{hkv}/{d} self={with_self}")
        host = _inputs(batch, n_shards, shard_len, q_len, hq, hkv, d, seed=40 + j)
        tensors = tuple(dev(x) for x in host)
        attn = B.make_attn(hq, hkv, d, 500000.0, 0)
        o_a, l_a, n_parts = _run(True, attn, shape, tensors)
        o_b, l_b, _ = _run(False, attn, shape, tensors)
        assert torch.equal(torch.nan_to_num(o_a, nan=7.0), torch.nan_to_num(o_b, nan=7.0))
        assert torch.equal(l_a, l_b)
        assert not torch.isnan(l_a).any()
        log(f"[noalloc] call {j}: bit-identical to the workspace form ({n_parts} parts)")
        # and the merged answer against the oracle
        o = torch.empty((batch, q_len, hq, d), device="cuda")
        lse = torch.empty((batch, q_len, hq), device="cuda")
        B.pulsar_lse_merge(batch, n_parts, q_len, hq, d, o_a, l_a, o, lse)
        torch.cuda.synchronize()
        qq, kc, vc, ks, vs = host
        for s in range(batch):
            kk = W.bf16_bits_to_f64(kc[s])
            vv = np.swapaxes(W.bf16_bits_to_f64(vc[s]), -1, -2)
            parts = OA.phase2_partials(W.bf16_bits_to_f64(qq[s]), n_shards * shard_len, kk, vv,
                                       W.bf16_bits_to_f64(ks[s]) if with_self else None,
                                       W.bf16_bits_to_f64(vs[s]) if with_self else None, 500000.0)
            want_o, want_lse = OA.lse_merge([p[0] for p in parts], [p[1] for p in parts])
            assert_close(o[s].cpu().numpy(), want_o, f"noalloc call {j} merged O seq {s}")
            assert_close(lse[s].cpu().numpy(), want_lse, f"noalloc call {j} merged LSE seq {s}",
                         max_abs=LSE_ABS, mean_abs=LSE_ABS)


def test_noalloc_query_replays_from_a_graph():
    """The callers the entry point is for capture it: a HIP graph of one call,
    replayed three times over poisoned outputs, with an eager no-allocation call of
    another shape between replays (it overwrites the fixed array), equals the eager
    call bit for bit every time."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to("cuda")
    shape, other = CALLS[1], CALLS[0]
    batch, n_shards, shard_len, q_len, hq, hkv, d, with_self = shape
    tensors = tuple(dev(x) for x in _inputs(batch, n_shards, shard_len, q_len, hq, hkv, d, seed=77))
    attn = B.make_attn(hq, hkv, d, 500000.0, 0)
    o_want, l_want, n_parts = _run(True, attn, shape, tensors)
    o_part = torch.empty_like(o_want)
    lse_part = torch.empty_like(l_want)
    qq, kc, vc, ks, vs = tensors
    args = (attn, batch, n_shards, shard_len, qq, q_len, n_shards * shard_len, kc, vc, ks, vs,
            o_part, lse_part, n_parts)
    ob = other
    other_tensors = tuple(dev(x) for x in _inputs(*ob[:7], seed=78))
    other_attn = B.make_attn(ob[4], ob[5], ob[6], 500000.0, 0)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        B.pulsar_phase2_query_noalloc(*args)
    for rep in range(3):
        o_part.fill_(float("nan"))
        lse_part.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.nan_to_num(o_part, nan=7.0), torch.nan_to_num(o_want, nan=7.0)), rep
        assert torch.equal(lse_part, l_want), rep
        log(f"[noalloc] graph replay {rep}: bit-identical to the eager call")
        _run(True, other_attn, ob, other_tensors)    # another shape through the same array
