"""HIP graphs of the library's calls (a generation loop, one whole hot-path
step): every replay, with eager work and synchronisations between replays,
reproduces the eager results exactly."""
import numpy as np
import pytest

import workloads as W
from tests.gpu_cases import Case, log, torch_cuda

pytestmark = pytest.mark.gpu


def test_generation_graph_replays_match_eager_steps():
    torch = torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name="graph", n_blocks=5, block_size=512, q_len=2, batch=2,
                n_planted=0)
    n = 4
    case = Case(w)
    case.run()
    path = case.path

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    gq, gk, gv = (dev(x) for x in W.generated(w, n))
    path.decode_setup(n)
    eager = []
    for j in range(n):
        path.decode_step(gq[j], gk[j], gv[j])
        eager.append(path.o1.clone())
    torch.cuda.synchronize()
    graph = path.capture_generation(gq, gk, gv)
    for rep in range(3):
        path.o_steps.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j in range(n):
            assert torch.equal(path.o_steps[j], eager[j]), (rep, j)
        log(f"[graph] replay {rep}: {n} steps equal the eager steps")
        path.step()                      # eager work of the library between replays
        torch.cuda.synchronize()


def test_hot_path_step_graph_replays_match_the_eager_step():
    """One whole step (selection, Phase 1, Phase-2 query, merge) captured in a HIP
    graph: every replay, with the outputs poisoned before it and eager work of the
    library after it, writes exactly what the eager step wrote."""
    torch = torch_cuda()
    w = W.with_(W.WORKLOADS["tiny"], name="graph_step", n_blocks=4, block_size=512, q_len=40,
                batch=2)
    case = Case(w)
    path = case.path
    path.step()
    torch.cuda.synchronize()
    outs = {"sel": path.sel, "chunk_min_df": path.chunk_min_df, "df": path.df, "o": path.o,
            "k_cache": path.k_cache[0], "v_cache": path.v_cache[0], "o_q": path.o_q,
            "lse_q": path.lse_q}   # (sequence 1's caches are inputs of the step)
    want = {k: t.clone() for k, t in outs.items()}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        path.step()
    for rep in range(3):
        for k, t in outs.items():
            if t.dtype == torch.int32:
                t.fill_(-7)
            elif t.dtype == torch.bfloat16:
                t.view(torch.int16).fill_(0x7FC0)   # bf16 NaN
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(t, want[k]), (rep, k)
        log(f"[graph] replay {rep}: the captured step equals the eager step")
        path.step()                      # eager work of the library between replays
        torch.cuda.synchronize()
