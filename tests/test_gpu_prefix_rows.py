"""GPU parity of the prefix rows (the last block's prefix list attended
causally in list order) against the oracle, on every row of small geometries
and on sampled rows of the full-size workloads."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import selection as OS
from tests.gpu_cases import Case, F32Rows, assert_close, log, torch_cuda
from tests.test_gpu_phase1 import SMALL

pytestmark = pytest.mark.gpu


def _run(case):
    import torch
    case.run()
    n = case.path.prefix_rows()
    torch.cuda.synchronize()
    return n


def _prefix_last(case):
    w = case.w
    sel, _, _ = case.oracle_selection()
    return OS.prefix_positions(sel, w.n_blocks, w.block_size, w.chunk_size, w.sink_size)[-1]


@pytest.mark.parametrize("name", [n for n in SMALL if SMALL[n].get("n_blocks", 4) > 1] + ["single_block"])
def test_prefix_rows_small_all_rows(name):
    torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name=name, **SMALL[name])
    case = Case(w)
    n = _run(case)
    pre = _prefix_last(case)
    assert n == (len(pre) if w.n_blocks > 1 else 0)
    if n == 0:
        return
    got = case.path.o_prefix[:n].cpu().numpy()
    want = OA.prefix_rows(F32Rows(case.q), case.oracle_khat(), F32Rows(case.v), pre, range(n),
                          w.rope_base)
    assert_close(got, want, f"{name} prefix rows ({n} rows x {w.n_q_heads} heads)")


@pytest.mark.parametrize("name", ["128k", "32k", "128k_star", "512k"])
def test_prefix_rows_full_size_sampled(name):
    torch_cuda()
    w = W.WORKLOADS[name]
    case = Case(w, extra_seqs=False)
    n = _run(case)
    pre = _prefix_last(case)
    assert n == len(pre)
    rng = np.random.default_rng(w.seed)
    rows = sorted(set(r for r in [0, 1, 31, 32, 63, 64, w.sink_size - 1, w.sink_size, n - 65,
                                  n - 64, n - 1] + [int(x) for x in rng.choice(n, size=8, replace=False)]
                      if 0 <= r < n))
    log(f"[prefix] {name}: {n} prefix rows, checking {len(rows)}")
    import torch
    got = case.path.o_prefix.index_select(0, torch.tensor(rows, device="cuda")).cpu().numpy()
    want = OA.prefix_rows(F32Rows(case.q), case.oracle_khat(), F32Rows(case.v), pre, rows,
                          w.rope_base)
    assert_close(got, want, f"{name} prefix rows sampled")
