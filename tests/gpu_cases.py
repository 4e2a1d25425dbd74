"""Shared plumbing of the GPU parity tests: seeded inputs (from `workloads`),
the oracle's expected values (from `oracle`), and the HIP path (through the
C ABI via `long_context_blockwise_max_amd`).  Nothing here computes the
method itself."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import selection as OS

# tolerances stated for the floating-point outputs (attention and LSE)
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def rope_spec(w: W.Workload):
    """The RoPE base as the oracle takes it (marked when the workload scales)."""
    from oracle.rope import Llama3Base
    return Llama3Base(w.rope_base) if w.rope_scaling == 1 else w.rope_base


def geometry_of(w: W.Workload, with_self=True):
    from long_context_blockwise_max_amd.pipeline import Geometry
    return Geometry(w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks, w.sink_size,
                    w.vocab_size, w.n_q_heads, w.n_kv_heads, w.head_dim, w.q_len, w.batch,
                    w.rope_base, with_self, w.rope_scaling)


class Case:
    """Inputs of one workload on host and device, run through the HIP path."""

    def __init__(self, w: W.Workload, with_self=True, extra_seqs=True):
        from long_context_blockwise_max_amd.pipeline import HotPath
        torch_cuda()
        self.w = w
        log(f"[case] {w.name}: generating inputs (seed {w.seed}, L={w.context_len}, "
            f"Hq/Hkv/d={w.n_q_heads}/{w.n_kv_heads}/{w.head_dim}, Lq={w.q_len}, B={w.batch})")
        self.tok = W.tokens(w)
        self.q = W.qkv(w, "q")
        self.k = W.qkv(w, "k")
        self.v = W.qkv(w, "v")
        self.qq, self.kq, self.vq = W.query(w)
        self.path = HotPath(geometry_of(w, with_self))
        self.path.upload(self.tok, self.q, self.k, self.v, self.qq,
                         self.kq if with_self else None, self.vq if with_self else None)
        if extra_seqs:
            for s in range(1, w.batch):
                self.path.upload_extra_cache(s, W.extra_cache(w, s, "k"), W.extra_cache(w, s, "v"))
        self.with_self = with_self

    def run(self):
        import torch
        log(f"[case] {self.w.name}: pulsar_select -> phase1 -> phase2 -> merge")
        self.path.step()
        torch.cuda.synchronize()
        log(f"[case] {self.w.name}: done")

    # oracle side --------------------------------------------------------
    def oracle_selection(self):
        w = self.w
        return OS.select(self.tok, w.n_blocks, w.block_size, w.chunk_size, w.budget_chunks,
                         w.vocab_size)

    def oracle_khat(self):
        """Rotated bf16 keys of the whole context, float32 (exact bf16 values)."""
        w = self.w
        out = np.empty(self.k.shape, np.float32)
        step = 8192
        for s in range(0, w.context_len, step):
            kb = W.bf16_bits_to_f64(self.k[s:s + step])
            out[s:s + step] = OA.rotate_bf16(kb, np.arange(s, s + kb.shape[0]), rope_spec(w))
        return out


def dense_rows(w: W.Workload, blocks=None, span=96, edge=64, seed=0):
    """(block, row) pairs of the dense full-size sample: in each chosen block the
    first and last `edge` rows plus one seeded row in every `span`-row stretch
    (so every 96- or 128-row tile of the block has at least one); the other
    blocks get their first rows, the edges of their first 64-row tile, their
    last row and two seeded rows."""
    rng = np.random.default_rng(seed)
    b = w.block_size
    blocks = range(w.n_blocks) if blocks is None else blocks
    rows = []
    for i in range(w.n_blocks):
        if i in blocks:
            rr = set(range(min(edge, b))) | set(range(max(0, b - edge), b))
            for lo in range(0, b, span):
                rr.add(int(rng.integers(lo, min(lo + span, b))))
        else:
            rr = {0, 63, 64, b - 1} | set(int(x) for x in rng.integers(0, b, 2))
        rows += [(i, r) for r in sorted(x for x in rr if 0 <= x < b)]
    return rows


class F32Rows:
    """Indexable view [L][H][d] of bf16 bits as float64 rows (for the oracle)."""

    def __init__(self, bits):
        self.bits = bits

    def __getitem__(self, idx):
        return W.bf16_bits_to_f64(self.bits[idx])


def assert_close(got, want, what, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    log(f"[parity] {what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} n={err.size}")
    assert err.max() <= max_abs, f"{what}: max abs err {err.max()}"
    assert err.mean() <= mean_abs, f"{what}: mean abs err {err.mean()}"
