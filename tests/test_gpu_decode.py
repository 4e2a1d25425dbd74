"""GPU parity of generation: self-cache append plus Phase-2 decode attention
and merge, step by step, against the oracle's masked dense attention over the
retained shards and the self tokens up to the new one."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import LSE_ABS, Case, assert_close, log, rope_spec, torch_cuda

pytestmark = pytest.mark.gpu


def _retained(case, seq):
    w = case.w
    if seq == 0:
        khat = case.oracle_khat().astype(np.float64)
        kc = khat.reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim).transpose(0, 2, 1, 3)
        vc = W.bf16_bits_to_f64(case.v).reshape(w.n_blocks, w.block_size, w.n_kv_heads, w.head_dim)
        return kc, vc.transpose(0, 2, 1, 3)
    return (W.bf16_bits_to_f64(W.extra_cache(w, seq, "k")),
            W.bf16_bits_to_f64(W.extra_cache(w, seq, "v")))


def _bits_to(dst, bits):
    import torch
    dst.copy_(torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
              .reshape(dst.shape))


CASES = {
    "tiny": {},
    "decode_batch": dict(n_blocks=5, block_size=512, q_len=1, batch=3, n_planted=0),
    "g4_d128": dict(n_blocks=2, block_size=640, n_q_heads=8, n_kv_heads=2, head_dim=128, q_len=5,
                    budget_chunks=2, n_planted=0, batch=2),
    # Llama-3.1 frequency scaling in the appended keys and the decoded queries
    "llama3": dict(n_blocks=3, block_size=2048, n_q_heads=8, n_kv_heads=2, head_dim=128, q_len=2,
                   budget_chunks=2, n_planted=0, rope_scaling=1),
}
# generated tokens per case (long_gen: the self cache grows past 8, 16 and 24 tokens,
# so the zero-padded tail of the value runs moves several times)
N_GEN = {"long_gen": 22}
CASES["long_gen"] = dict(n_blocks=2, block_size=256, q_len=3, batch=2, n_planted=0)
# a self cache of 201-203 tokens (4 tiles) next to 4 shard tiles: half the parts
# read self keys only
CASES["self_heavy"] = dict(n_blocks=2, block_size=128, budget_chunks=1, q_len=200, n_planted=0)
CASES["self_heavy_d128"] = dict(n_blocks=2, block_size=128, budget_chunks=1, q_len=200, n_planted=0,
                                n_q_heads=8, n_kv_heads=2, head_dim=128, batch=2)


@pytest.mark.parametrize("name", list(CASES))
def test_generation_steps_match_the_oracle(name):
    torch = torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name=name, **CASES[name])
    n_gen = N_GEN.get(name, 3)
    base = rope_spec(w)
    case = Case(w)
    case.run()
    gq, gk, gv = W.generated(w, n_gen)
    path = case.path
    path.decode_setup(n_gen)
    retained = [_retained(case, s) for s in range(w.batch)]
    for step in range(n_gen):
        _bits_to(path.q1, gq[step])
        _bits_to(path.k1, gk[step])
        _bits_to(path.v1, gv[step])
        log(f"[decode] {name}: step {step} (self tokens {w.q_len + step + 1})")
        path.decode_step()
        torch.cuda.synchronize()
        o = path.o1.cpu().numpy()
        lse = path.lse1.cpu().numpy()
        for s in range(w.batch):
            ks = np.concatenate([case.kq[s], gk[:step + 1, s, 0]], axis=0)
            vs = np.concatenate([case.vq[s], gv[:step + 1, s, 0]], axis=0)
            kc, vc = retained[s]
            want_o, want_lse = OA.dense_decode_attention(
                W.bf16_bits_to_f64(gq[step, s]), kc, vc, W.bf16_bits_to_f64(ks),
                W.bf16_bits_to_f64(vs), w.context_len, base)
            assert_close(o[s], want_o, f"{name} decode step {step} seq {s} O")
            assert_close(lse[s], want_lse, f"{name} decode step {step} seq {s} LSE",
                         max_abs=LSE_ABS, mean_abs=LSE_ABS)


def test_decode_of_the_query_tokens_is_the_query_phase():
    """With the self cache holding exactly the query tokens, decode attention of
    those tokens is the query phase with its self shard."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    w = W.with_(W.WORKLOADS["tiny"], name="consistency", **CASES["g4_d128"])
    case = Case(w)
    case.run()
    path = case.path
    path.decode_setup(0)
    g = path.geo
    o_part = torch.empty_like(path.o_part)
    lse_part = torch.empty_like(path.lse_part)
    ws = torch.empty(B.pulsar_phase2_workspace_bytes(path.cattn, g.batch, g.q_len, False),
                     dtype=torch.uint8, device="cuda")
    B.pulsar_phase2_decode(path.cattn, g.batch, g.n_blocks, g.block_size, path.qq, g.q_len,
                           path.k_cache, path.v_cache, path.k_self_cache, path.v_self_cache,
                           path.cap, path.n_self, g.context_len, o_part, lse_part, path.n_parts, ws)
    o = torch.empty_like(path.o_q)
    lse = torch.empty_like(path.lse_q)
    B.pulsar_lse_merge(g.batch, path.n_parts, g.q_len, g.n_q_heads, g.head_dim, o_part, lse_part,
                       o, lse)
    torch.cuda.synchronize()
    assert_close(o.cpu().numpy(), path.o_q.cpu().numpy().astype(np.float64), "decode == query O",
                 max_abs=1e-5, mean_abs=1e-6)
    assert_close(lse.cpu().numpy(), path.lse_q.cpu().numpy().astype(np.float64), "decode == query LSE",
                 max_abs=1e-5, mean_abs=1e-6)


def test_generation_at_128k_matches_the_oracle():
    """Two generated tokens over the full 128K workload's retained shards (all 32
    heads against a masked dense softmax over 131072 + 66 keys)."""
    torch = torch_cuda()
    w = W.WORKLOADS["128k"]
    case = Case(w, extra_seqs=False)
    case.run()
    gq, gk, gv = W.generated(w, 2)
    path = case.path
    path.decode_setup(2)
    kc, vc = _retained(case, 0)
    for step in range(2):
        _bits_to(path.q1, gq[step])
        _bits_to(path.k1, gk[step])
        _bits_to(path.v1, gv[step])
        log(f"[decode] 128k: step {step}")
        path.decode_step()
        torch.cuda.synchronize()
        ks = np.concatenate([case.kq[0], gk[:step + 1, 0, 0]], axis=0)
        vs = np.concatenate([case.vq[0], gv[:step + 1, 0, 0]], axis=0)
        want_o, want_lse = OA.dense_decode_attention(
            W.bf16_bits_to_f64(gq[step, 0]), kc, vc, W.bf16_bits_to_f64(ks),
            W.bf16_bits_to_f64(vs), w.context_len, w.rope_base)
        assert_close(path.o1.cpu().numpy()[0], want_o, f"128k decode step {step} O")
        assert_close(path.lse1.cpu().numpy()[0], want_lse, f"128k decode step {step} LSE",
                     max_abs=LSE_ABS, mean_abs=LSE_ABS)


def _three_calls(path, B, q, k, v, q_len, o, lse):
    """The generation step as pulsar_self_append + pulsar_phase2_decode + pulsar_lse_merge."""
    import torch
    g = path.geo
    n_parts = B.pulsar_phase2_num_parts(path.cattn, g.batch, g.n_blocks, g.block_size, q_len, True)
    o_part = torch.empty((g.batch, n_parts, q_len, g.n_q_heads, g.head_dim), device="cuda")
    lse_part = torch.empty((g.batch, n_parts, q_len, g.n_q_heads), device="cuda")
    ws = torch.empty(max(B.pulsar_phase2_workspace_bytes(path.cattn, g.batch, q_len, False), 256),
                     dtype=torch.uint8, device="cuda")
    B.pulsar_self_append(path.cattn, g.batch, path.cap, path.n_self, q_len, g.context_len, k, v,
                         path.k_self_cache, path.v_self_cache)
    B.pulsar_phase2_decode(path.cattn, g.batch, g.n_blocks, g.block_size, q, q_len, path.k_cache,
                           path.v_cache, path.k_self_cache, path.v_self_cache, path.cap,
                           path.n_self + q_len, g.context_len, o_part, lse_part, n_parts, ws)
    B.pulsar_lse_merge(g.batch, n_parts, q_len, g.n_q_heads, g.head_dim, o_part, lse_part, o, lse)


def _one_call(path, B, q, k, v, q_len, o, lse, ws):
    import torch
    g = path.geo
    n_parts = B.pulsar_phase2_num_parts(path.cattn, g.batch, g.n_blocks, g.block_size, q_len, True)
    o_part = torch.full((g.batch, n_parts, q_len, g.n_q_heads, g.head_dim), float("nan"), device="cuda")
    lse_part = torch.full((g.batch, n_parts, q_len, g.n_q_heads), float("nan"), device="cuda")
    B.pulsar_decode_step(path.cattn, g.batch, g.n_blocks, g.block_size, q, k, v, q_len, path.k_cache,
                         path.v_cache, path.k_self_cache, path.v_self_cache, path.cap, path.n_self,
                         g.context_len, o_part, lse_part, n_parts, o, lse, ws)


STEP_CASES = {
    # name: (workload overrides, tokens per step, steps)
    "tiny_1": ({}, 1, 3),
    "batch3_1": (CASES["decode_batch"], 1, 4),
    "long_1": (CASES["long_gen"], 1, 22),
    "self_heavy_1": (CASES["self_heavy_d128"], 1, 3),
    "llama3_1": (CASES["llama3"], 1, 2),
    # several tokens a step, still appended by the attention launch (4 heads x 5
    # tokens in one wave);
    # the new tokens can straddle a 64-token tile
    "g4_5tok": (dict(CASES["g4_d128"], q_len=62), 5, 3),
    # 8 heads x 5 tokens do not fit one wave: the three calls run inside
    "g8_5tok": (dict(n_blocks=2, block_size=256, n_q_heads=8, n_kv_heads=1, head_dim=128, q_len=3,
                     budget_chunks=1, n_planted=0), 5, 2),
}


@pytest.mark.parametrize("name", list(STEP_CASES))
def test_one_call_step_equals_the_three_calls(name):
    """pulsar_decode_step against pulsar_self_append + pulsar_phase2_decode +
    pulsar_lse_merge on the same inputs: the merged outputs and LSEs of every step
    and the self caches afterwards are bit-identical (for one-token steps the
    attention launch appends the new tokens itself)."""
    torch = torch_cuda()
    from long_context_blockwise_max_amd import binding as B
    over, q_len, n_steps = STEP_CASES[name]
    w = W.with_(W.WORKLOADS["tiny"], name=name, **over)
    rng = np.random.default_rng(7)
    bf = lambda shape: torch.from_numpy(W.f32_to_bf16_bits(
        rng.standard_normal(shape, dtype=np.float32)).view(np.int16)).view(torch.bfloat16).to("cuda")
    fused, plain = Case(w), Case(w)
    fused.run()
    plain.run()
    fused.path.decode_setup(q_len * n_steps)
    plain.path.decode_setup(q_len * n_steps)
    g = fused.path.geo
    ws = torch.empty(max(B.pulsar_decode_step_workspace_bytes(fused.path.cattn, g.batch, q_len), 256),
                     dtype=torch.uint8, device="cuda")
    for step in range(n_steps):
        q = bf((g.batch, q_len, g.n_q_heads, g.head_dim))
        k = bf((g.batch, q_len, g.n_kv_heads, g.head_dim))
        v = bf((g.batch, q_len, g.n_kv_heads, g.head_dim))
        outs = []
        for case, fn in ((fused, _one_call), (plain, _three_calls)):
            o = torch.full((g.batch, q_len, g.n_q_heads, g.head_dim), float("nan"), device="cuda")
            lse = torch.full((g.batch, q_len, g.n_q_heads), float("nan"), device="cuda")
            if fn is _one_call:
                fn(case.path, B, q, k, v, q_len, o, lse, ws)
            else:
                fn(case.path, B, q, k, v, q_len, o, lse)
            case.path.n_self += q_len
            outs.append((o, lse))
        torch.cuda.synchronize()
        (o_a, l_a), (o_b, l_b) = outs
        assert not torch.isnan(o_a).any() and not torch.isnan(l_a).any()
        assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b), f"{name} step {step}"
        log(f"[decode-step] {name} step {step}: one call == three calls (self tokens "
            f"{fused.path.n_self})")
    n = fused.path.n_self
    pad = (n + 7) // 8 * 8
    assert torch.equal(fused.path.k_self_cache[:, :n], plain.path.k_self_cache[:, :n])
    assert torch.equal(fused.path.v_self_cache[..., :pad], plain.path.v_self_cache[..., :pad])
