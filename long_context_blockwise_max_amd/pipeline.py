"""Host-side orchestration of the whole hot path on one GPU.

`HotPath` owns the device buffers of one problem and enqueues, on one stream,
the four C-ABI calls in the method's order: Max-IDF selection, Phase-1
encoding (which also fills the retained cache), Phase-2 query attention over
every retained shard plus the query's own causal shard, and the exact LSE
merge.  torch is used for device memory and the stream only.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import binding as B


@dataclass(frozen=True)
class Geometry:
    n_blocks: int
    block_size: int
    chunk_size: int
    budget_chunks: int
    sink_size: int
    vocab_size: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q_len: int
    batch: int = 1
    rope_base: float = 500000.0
    with_self: bool = True
    rope_scaling: int = 0      # 1: Llama-3.1 frequency scaling

    @property
    def context_len(self):
        return self.n_blocks * self.block_size


def _bf16_empty(shape, device):
    return torch.empty(shape, dtype=torch.bfloat16, device=device)


class HotPath:
    """Device buffers + the four calls.  Sequence 0 of the Phase-2 batch is
    the sequence Phase 1 encodes (its retained cache is written in place into
    slot 0 of the batched cache); further sequences' caches are inputs."""

    def __init__(self, geo: Geometry, device="cuda"):
        self.geo = geo
        g = geo
        dev = torch.device(device)
        self.device = dev
        L, hq, hkv, d = g.context_len, g.n_q_heads, g.n_kv_heads, g.head_dim
        self.cgeom = B.make_geom(g.n_blocks, g.block_size, g.chunk_size, g.budget_chunks,
                                 g.sink_size, g.vocab_size)
        self.cattn = B.make_attn(hq, hkv, d, g.rope_base, g.rope_scaling)
        self.kept = B.pulsar_kept_chunks(self.cgeom)
        if self.kept < 0:
            raise B.PulsarError(B.PULSAR_EINVAL, "geometry")
        n_chunks = g.block_size // g.chunk_size
        ws_bytes = B.pulsar_workspace_bytes(self.cgeom, self.cattn)
        if ws_bytes == 0:
            raise B.PulsarError(B.PULSAR_EINVAL, "pulsar_workspace_bytes")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.tok = torch.empty(L, dtype=torch.int32, device=dev)
        self.sel = torch.empty((g.n_blocks, max(self.kept, 1)), dtype=torch.int32, device=dev)
        self.chunk_min_df = torch.empty((g.n_blocks, n_chunks), dtype=torch.int32, device=dev)
        self.df = torch.empty(g.vocab_size, dtype=torch.int32, device=dev)
        self.q = _bf16_empty((L, hq, d), dev)
        self.k = _bf16_empty((L, hkv, d), dev)
        self.v = _bf16_empty((L, hkv, d), dev)
        self.o = torch.empty((L, hq, d), dtype=torch.float32, device=dev)
        self.k_cache = _bf16_empty((g.batch, g.n_blocks, hkv, g.block_size, d), dev)
        # retained values are d-major: [B][N][Hkv][d][b]
        self.v_cache = _bf16_empty((g.batch, g.n_blocks, hkv, d, g.block_size), dev)
        self.qq = _bf16_empty((g.batch, g.q_len, hq, d), dev)
        self.k_self = _bf16_empty((g.batch, g.q_len, hkv, d), dev) if g.with_self else None
        self.v_self = _bf16_empty((g.batch, g.q_len, hkv, d), dev) if g.with_self else None
        self.n_parts = B.pulsar_phase2_num_parts(self.cattn, g.batch, g.n_blocks, g.block_size,
                                                 g.q_len, g.with_self)
        self.o_part = torch.empty((g.batch, self.n_parts, g.q_len, hq, d), dtype=torch.float32,
                                  device=dev)
        self.lse_part = torch.empty((g.batch, self.n_parts, g.q_len, hq), dtype=torch.float32,
                                    device=dev)
        self.ws2 = torch.empty(B.pulsar_phase2_workspace_bytes(self.cattn, g.batch, g.q_len,
                                                               g.with_self),
                               dtype=torch.uint8, device=dev)
        self.o_q = torch.empty((g.batch, g.q_len, hq, d), dtype=torch.float32, device=dev)
        self.lse_q = torch.empty((g.batch, g.q_len, hq), dtype=torch.float32, device=dev)

    # inputs -------------------------------------------------------------
    @staticmethod
    def _bits_to_dev(dst, bits):
        t = torch.from_numpy(bits.view("int16")).view(torch.bfloat16)
        dst.copy_(t.reshape(dst.shape))

    def upload(self, tok=None, q=None, k=None, v=None, qq=None, k_self=None, v_self=None):
        """Copy host arrays (int32 tokens; bf16 bit patterns as uint16) to the device."""
        if tok is not None:
            self.tok.copy_(torch.from_numpy(tok.astype("int32")))
        for dst, src in ((self.q, q), (self.k, k), (self.v, v), (self.qq, qq),
                         (self.k_self, k_self), (self.v_self, v_self)):
            if src is not None and dst is not None:
                self._bits_to_dev(dst, src)

    def upload_extra_cache(self, seq, k_bits, v_bits):
        """Retained cache of another sequence: k_bits, v_bits [N][Hkv][b][d] bf16 bits
        (values are transposed to the d-major layout on the device)."""
        self._bits_to_dev(self.k_cache[seq], k_bits)
        t = torch.from_numpy(v_bits.view("int16")).view(torch.bfloat16).to(self.device)
        self.v_cache[seq].copy_(t.transpose(-1, -2))

    # the four calls -------------------------------------------------------
    def select(self, stream=None):
        B.pulsar_select(self.cgeom, self.tok, self.sel if self.kept > 0 else None,
                        self.chunk_min_df, self.df, self.ws, stream)

    def select_method(self, method, seed=0, stream=None):
        """Selection by another chunk score (binding.SELECT_METHODS) into sel."""
        B.pulsar_select_method(self.cgeom, method, seed, self.tok,
                               self.sel if self.kept > 0 else None, self.ws, stream)

    def phase1(self, stream=None):
        B.pulsar_phase1_encode(self.cgeom, self.cattn, self.q, self.k, self.v,
                               self.sel if self.kept > 0 else None, self.o,
                               self.k_cache[0], self.v_cache[0], self.ws, stream)

    def phase1_prepare(self, stream=None):
        B.pulsar_phase1_prepare(self.cgeom, self.cattn, self.q, self.k, self.v,
                                self.sel if self.kept > 0 else None, self.k_cache[0],
                                self.v_cache[0], self.ws, stream)

    def phase1_attend(self, stream=None):
        B.pulsar_phase1_attend(self.cgeom, self.cattn, self.k_cache[0], self.v_cache[0], self.o,
                               self.ws, stream)

    def phase2(self, stream=None):
        g = self.geo
        B.pulsar_phase2_query(self.cattn, g.batch, g.n_blocks, g.block_size, self.qq, g.q_len,
                              g.context_len, self.k_cache, self.v_cache, self.k_self, self.v_self,
                              self.o_part, self.lse_part, self.n_parts, self.ws2, stream)

    def merge(self, stream=None):
        g = self.geo
        B.pulsar_lse_merge(g.batch, self.n_parts, g.q_len, g.n_q_heads, g.head_dim, self.o_part,
                           self.lse_part, self.o_q, self.lse_q, stream)

    def step(self, stream=None):
        self.select(stream)
        self.phase1(stream)
        self.phase2(stream)
        self.merge(stream)

    def prefix_rows(self, stream=None):
        """Attention output of every prefix row into o_prefix [rows][Hq][d]
        (after phase1_prepare / phase1)."""
        g = self.geo
        n = B.pulsar_prefix_rows_len(self.cgeom)
        if getattr(self, "o_prefix", None) is None or self.o_prefix.shape[0] != max(n, 1):
            self.o_prefix = torch.empty((max(n, 1), g.n_q_heads, g.head_dim), dtype=torch.float32,
                                        device=self.device)
        B.pulsar_phase1_prefix_rows(self.cgeom, self.cattn, self.k_cache[0], self.v_cache[0],
                                    self.o_prefix if n > 0 else None, self.ws, stream)
        return n

    # generation ---------------------------------------------------------
    def decode_setup(self, max_new: int):
        """Self caches for the query tokens plus up to max_new generated tokens,
        primed with the query tokens' own keys and values (self token 0 sits at
        position L, right after the context)."""
        g = self.geo
        dev = self.device
        hkv, hq, d = g.n_kv_heads, g.n_q_heads, g.head_dim
        self.cap = (g.q_len + max_new + 63) // 64 * 64
        self.k_self_cache = _bf16_empty((g.batch, self.cap, hkv, d), dev)
        self.v_self_cache = _bf16_empty((g.batch, hkv, d, self.cap), dev)
        self.n_self = 0
        self.q1 = _bf16_empty((g.batch, 1, hq, d), dev)
        self.k1 = _bf16_empty((g.batch, 1, hkv, d), dev)
        self.v1 = _bf16_empty((g.batch, 1, hkv, d), dev)
        self.n_parts1 = B.pulsar_phase2_num_parts(self.cattn, g.batch, g.n_blocks, g.block_size, 1, True)
        self.o_part1 = torch.empty((g.batch, self.n_parts1, 1, hq, d), dtype=torch.float32, device=dev)
        self.lse_part1 = torch.empty((g.batch, self.n_parts1, 1, hq), dtype=torch.float32, device=dev)
        self.ws1 = torch.empty(max(B.pulsar_phase2_workspace_bytes(self.cattn, g.batch, 1, False), 256),
                               dtype=torch.uint8, device=dev)
        self.o1 = torch.empty((g.batch, 1, hq, d), dtype=torch.float32, device=dev)
        self.lse1 = torch.empty((g.batch, 1, hq), dtype=torch.float32, device=dev)
        self.ws_step = torch.empty(max(B.pulsar_decode_step_workspace_bytes(self.cattn, g.batch, 1), 256),
                                   dtype=torch.uint8, device=dev)
        self.self_append(self.k_self, self.v_self, g.q_len)

    def self_append(self, k_new, v_new, n_new, stream=None):
        g = self.geo
        B.pulsar_self_append(self.cattn, g.batch, self.cap, self.n_self, n_new, g.context_len,
                             k_new, v_new, self.k_self_cache, self.v_self_cache, stream)
        self.n_self += n_new

    def decode_step(self, q_new=None, k_new=None, v_new=None, o_out=None, stream=None,
                    fused=True):
        """One generated token: append its key / value (default k1, v1), attend its
        query (default q1) to every retained shard and the self cache, merge into
        o_out (default o1, with its LSE in lse1).  Token tensors are [B][1][H][d]
        bf16 on the device.  fused: one pulsar_decode_step call; otherwise
        pulsar_self_append, pulsar_phase2_decode and pulsar_lse_merge."""
        g = self.geo
        q_new = self.q1 if q_new is None else q_new
        k_new = self.k1 if k_new is None else k_new
        v_new = self.v1 if v_new is None else v_new
        o = self.o1 if o_out is None else o_out
        lse = self.lse1 if o_out is None else None
        if fused:
            B.pulsar_decode_step(self.cattn, g.batch, g.n_blocks, g.block_size, q_new, k_new, v_new,
                                 1, self.k_cache, self.v_cache, self.k_self_cache,
                                 self.v_self_cache, self.cap, self.n_self, g.context_len,
                                 self.o_part1, self.lse_part1, self.n_parts1, o, lse, self.ws_step,
                                 stream)
            self.n_self += 1
            return
        self.self_append(k_new, v_new, 1, stream)
        B.pulsar_phase2_decode(self.cattn, g.batch, g.n_blocks, g.block_size, q_new, 1,
                               self.k_cache, self.v_cache, self.k_self_cache, self.v_self_cache,
                               self.cap, self.n_self, g.context_len, self.o_part1, self.lse_part1,
                               self.n_parts1, self.ws1, stream)
        B.pulsar_lse_merge(g.batch, self.n_parts1, 1, g.n_q_heads, g.head_dim, self.o_part1,
                           self.lse_part1, o, lse, stream)

    def capture_generation(self, q_new, k_new, v_new):
        """Capture n generation steps (self cache primed anew, then one step per
        token; q_new / k_new / v_new [n][B][1][H][d] on the device) into one HIP
        graph.  Every step's arguments, the self-cache length included, are fixed
        at capture, so a replay recomputes the same n steps into
        o_steps [n][B][1][Hq][d].  Only this library's kernels are captured (no memsets,
        no allocations)."""
        g = self.geo
        n = q_new.shape[0]
        self.decode_setup(n)
        self.o_steps = torch.empty((n, g.batch, 1, g.n_q_heads, g.head_dim), dtype=torch.float32,
                                   device=self.device)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        with torch.cuda.graph(graph, stream=side):
            self.n_self = 0
            self.self_append(self.k_self, self.v_self, g.q_len)
            for j in range(n):
                self.decode_step(q_new[j], k_new[j], v_new[j], o_out=self.o_steps[j])
        return graph

    def status_word(self) -> int:
        return int(self.ws[:4].view(torch.int32).item())
