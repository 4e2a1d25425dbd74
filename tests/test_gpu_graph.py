"""A generation loop captured in one HIP graph: every replay, with eager work
and synchronisations between replays, reproduces the eager steps exactly."""
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
