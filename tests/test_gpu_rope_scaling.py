"""The Llama-3.1 frequency scaling through the whole path (Phase 1, prefix rows,
Phase 2 with its self shard) against the oracle with the same scaling."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import selection as OS
from tests.gpu_cases import LSE_ABS, Case, F32Rows, assert_close, rope_spec, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_llama3_scaled_rope_matches_the_oracle(d):
    import torch
    torch_cuda()
    # positions up to ~40K, so frequencies in all three regimes turn by many periods
    w = W.with_(W.WORKLOADS["tiny"], name=f"llama3_d{d}", n_blocks=5, block_size=8192 if d == 64 else 4096,
                n_q_heads=8, n_kv_heads=2, head_dim=d, budget_chunks=2, n_planted=0, q_len=3,
                rope_scaling=1)
    base = rope_spec(w)
    case = Case(w)
    case.run()
    n_pre = case.path.prefix_rows()
    torch.cuda.synchronize()
    sel, _, _ = case.oracle_selection()
    pre = OS.prefix_positions(sel, w.n_blocks, w.block_size, w.chunk_size, w.sink_size)
    khat = case.oracle_khat()
    rows = [(i, r) for i in (0, w.n_blocks - 1) for r in (0, 1, 63, 64, w.block_size - 1)]
    pos = torch.tensor([i * w.block_size + r for i, r in rows], device="cuda")
    got = case.path.o.index_select(0, pos).cpu().numpy()
    want = OA.phase1_rows(F32Rows(case.q), khat, F32Rows(case.v), pre, rows, w.block_size, base)
    assert_close(got, want, f"{w.name} phase1 rows")
    pr = [0, 63, n_pre - 1]
    got = case.path.o_prefix[pr].cpu().numpy()
    want = OA.prefix_rows(F32Rows(case.q), khat, F32Rows(case.v), pre[-1], pr, base)
    assert_close(got, want, f"{w.name} prefix rows")
    kc = khat.astype(np.float64).reshape(w.n_blocks, w.block_size, w.n_kv_heads, d).transpose(0, 2, 1, 3)
    vc = W.bf16_bits_to_f64(case.v).reshape(w.n_blocks, w.block_size, w.n_kv_heads, d).transpose(0, 2, 1, 3)
    parts = OA.phase2_partials(W.bf16_bits_to_f64(case.qq[0]), w.context_len, kc, vc,
                               W.bf16_bits_to_f64(case.kq[0]), W.bf16_bits_to_f64(case.vq[0]), base)
    want_o, want_lse = OA.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    assert_close(case.path.o_q[0].cpu().numpy(), want_o, f"{w.name} phase2 O")
    assert_close(case.path.lse_q[0].cpu().numpy(), want_lse, f"{w.name} phase2 LSE",
                 max_abs=LSE_ABS, mean_abs=LSE_ABS)
