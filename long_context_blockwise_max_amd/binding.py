"""Thin ctypes binding of libpulsar.so (include/pulsar.h).

Argument marshalling only: tensors are torch device tensors whose data
pointers are handed to the C ABI together with torch's current HIP stream.
Every step of the hot path runs in the library's HIP kernels.  Shapes, dtypes
and contiguity are checked here because the C ABI cannot see buffer sizes.
If the library is missing, loading fails with an error; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpulsar.so")

PULSAR_OK = 0
PULSAR_EINVAL = -1
PULSAR_EWORKSPACE = -2
PULSAR_EHIP = -3
PULSAR_EUNSUPPORTED = -4

EXPORTED = (
    "pulsar_workspace_bytes", "pulsar_kept_chunks", "pulsar_select", "pulsar_select_method",
    "pulsar_phase1_encode",
    "pulsar_phase1_prepare", "pulsar_phase1_attend", "pulsar_self_append", "pulsar_phase2_decode",
    "pulsar_prefix_rows_len", "pulsar_phase1_prefix_rows",
    "pulsar_phase2_num_parts", "pulsar_phase2_workspace_bytes", "pulsar_phase2_query",
    "pulsar_phase2_query_noalloc", "pulsar_phase2_noalloc_max_bytes",
    "pulsar_decode_step", "pulsar_decode_step_workspace_bytes",
    "pulsar_lse_merge", "pulsar_strerror",
)


class PulsarError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


class Geom(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("budget_chunks", ctypes.c_int32),
                ("sink_size", ctypes.c_int32), ("vocab_size", ctypes.c_int32)]


class Attn(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_scaling", ctypes.c_int32),
                ("rope_base", ctypes.c_double)]


_lib = None


def lib():
    """Load libpulsar.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} not built: run `python -m long_context_blockwise_max_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        G, A = ctypes.POINTER(Geom), ctypes.POINTER(Attn)
        L.pulsar_workspace_bytes.argtypes = [G, A]
        L.pulsar_workspace_bytes.restype = sz
        L.pulsar_kept_chunks.argtypes = [G]
        L.pulsar_kept_chunks.restype = i32
        L.pulsar_select.argtypes = [G, vp, vp, vp, vp, vp, sz, vp]
        L.pulsar_select_method.argtypes = [G, i32, ctypes.c_uint64, vp, vp, vp, sz, vp]
        L.pulsar_select_method.restype = ctypes.c_int
        L.pulsar_select.restype = ctypes.c_int
        L.pulsar_phase1_encode.argtypes = [G, A, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pulsar_phase1_encode.restype = ctypes.c_int
        L.pulsar_phase1_prepare.argtypes = [G, A, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pulsar_phase1_prepare.restype = ctypes.c_int
        L.pulsar_phase1_attend.argtypes = [G, A, vp, vp, vp, vp, sz, vp]
        L.pulsar_phase1_attend.restype = ctypes.c_int
        L.pulsar_phase2_num_parts.argtypes = [A, i32, i32, i32, i32, i32]
        L.pulsar_phase2_num_parts.restype = i32
        L.pulsar_phase2_workspace_bytes.argtypes = [A, i32, i32, i32]
        L.pulsar_phase2_workspace_bytes.restype = sz
        L.pulsar_phase2_query.argtypes = [A, i32, i32, i32, vp, i32, i64, vp, vp, vp, vp, vp, vp,
                                          i32, vp, sz, vp]
        L.pulsar_phase2_query.restype = ctypes.c_int
        L.pulsar_phase2_query_noalloc.argtypes = [A, i32, i32, i32, vp, i32, i64, vp, vp, vp, vp,
                                                  vp, vp, i32, vp]
        L.pulsar_phase2_query_noalloc.restype = ctypes.c_int
        L.pulsar_phase2_noalloc_max_bytes.argtypes = []
        L.pulsar_phase2_noalloc_max_bytes.restype = sz
        L.pulsar_decode_step_workspace_bytes.argtypes = [A, i32, i32]
        L.pulsar_decode_step_workspace_bytes.restype = sz
        L.pulsar_decode_step.argtypes = [A, i32, i32, i32, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32,
                                         i64, vp, vp, i32, vp, vp, vp, sz, vp]
        L.pulsar_decode_step.restype = ctypes.c_int
        L.pulsar_prefix_rows_len.argtypes = [G]
        L.pulsar_prefix_rows_len.restype = i64
        L.pulsar_phase1_prefix_rows.argtypes = [G, A, vp, vp, vp, vp, sz, vp]
        L.pulsar_phase1_prefix_rows.restype = ctypes.c_int
        L.pulsar_self_append.argtypes = [A, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp]
        L.pulsar_self_append.restype = ctypes.c_int
        L.pulsar_phase2_decode.argtypes = [A, i32, i32, i32, vp, i32, vp, vp, vp, vp, i32, i32, i64,
                                           vp, vp, i32, vp, sz, vp]
        L.pulsar_phase2_decode.restype = ctypes.c_int
        L.pulsar_lse_merge.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.pulsar_lse_merge.restype = ctypes.c_int
        L.pulsar_strerror.argtypes = [ctypes.c_int]
        L.pulsar_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().pulsar_strerror(code).decode()


def make_geom(n_blocks, block_size, chunk_size, budget_chunks, sink_size, vocab_size) -> Geom:
    return Geom(n_blocks, block_size, chunk_size, budget_chunks, sink_size, vocab_size)


def make_attn(n_q_heads, n_kv_heads, head_dim, rope_base, rope_scaling=0) -> Attn:
    return Attn(n_q_heads, n_kv_heads, head_dim, int(rope_scaling), float(rope_base))


# ----------------------------------------------------------------- helpers
def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype, numel, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _check(rc, where):
    if rc != PULSAR_OK:
        raise PulsarError(rc, where)


def _bf16_dtypes():
    import torch
    return (torch.bfloat16,)


def _bf16(t, numel, name, allow_none=False):
    import torch
    if t is not None and t.dtype == torch.int16:
        t = t.view(torch.bfloat16)
    return _ptr(t, torch.bfloat16, numel, name, allow_none)


# ---------------------------------------------------------------- the ABI
def pulsar_workspace_bytes(geom: Geom, attn: Attn | None) -> int:
    return lib().pulsar_workspace_bytes(ctypes.byref(geom), ctypes.byref(attn) if attn else None)


def pulsar_kept_chunks(geom: Geom) -> int:
    return lib().pulsar_kept_chunks(ctypes.byref(geom))


def pulsar_select(geom: Geom, tok, sel, chunk_min_df, df, ws, stream=None):
    import torch
    L = geom.n_blocks * geom.block_size
    kept = pulsar_kept_chunks(geom)
    n_chunks = geom.block_size // geom.chunk_size if geom.chunk_size > 0 else 0
    rc = lib().pulsar_select(
        ctypes.byref(geom), _ptr(tok, torch.int32, L, "tok"),
        _ptr(sel, torch.int32, geom.n_blocks * max(kept, 0), "sel", allow_none=kept <= 0),
        _ptr(chunk_min_df, torch.int32, geom.n_blocks * n_chunks, "chunk_min_df", allow_none=True),
        _ptr(df, torch.int32, geom.vocab_size, "df", allow_none=True),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_select")


SELECT_METHODS = {"max_idf": 0, "mean_idf": 1, "entropy": 2, "uniform": 3, "even": 4}


def pulsar_select_method(geom: Geom, method, seed, tok, sel, ws, stream=None):
    """method: a name of SELECT_METHODS or its number."""
    import torch
    m = SELECT_METHODS[method] if isinstance(method, str) else int(method)
    L = geom.n_blocks * geom.block_size
    kept = pulsar_kept_chunks(geom)
    rc = lib().pulsar_select_method(
        ctypes.byref(geom), m, ctypes.c_uint64(int(seed) & ((1 << 64) - 1)),
        _ptr(tok, torch.int32, L, "tok", allow_none=m in (3, 4)),
        _ptr(sel, torch.int32, geom.n_blocks * max(kept, 0), "sel", allow_none=kept <= 0),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_select_method")


def pulsar_phase1_encode(geom: Geom, attn: Attn, q, k, v, sel, o, k_cache, v_cache, ws,
                         stream=None):
    import torch
    L = geom.n_blocks * geom.block_size
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kept = pulsar_kept_chunks(geom)
    rc = lib().pulsar_phase1_encode(
        ctypes.byref(geom), ctypes.byref(attn), _bf16(q, L * hq * d, "q"), _bf16(k, L * hkv * d, "k"),
        _bf16(v, L * hkv * d, "v"),
        _ptr(sel, torch.int32, geom.n_blocks * max(kept, 0), "sel", allow_none=True),
        _ptr(o, torch.float32, L * hq * d, "o"), _bf16(k_cache, L * hkv * d, "k_cache"),
        _bf16(v_cache, L * hkv * d, "v_cache"), _ptr(ws, torch.uint8, 0, "ws"), ws.numel(),
        _stream(stream))
    _check(rc, "pulsar_phase1_encode")


def pulsar_phase1_prepare(geom: Geom, attn: Attn, q, k, v, sel, k_cache, v_cache, ws,
                          stream=None):
    import torch
    L = geom.n_blocks * geom.block_size
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kept = pulsar_kept_chunks(geom)
    rc = lib().pulsar_phase1_prepare(
        ctypes.byref(geom), ctypes.byref(attn), _bf16(q, L * hq * d, "q"), _bf16(k, L * hkv * d, "k"),
        _bf16(v, L * hkv * d, "v"),
        _ptr(sel, torch.int32, geom.n_blocks * max(kept, 0), "sel", allow_none=True),
        _bf16(k_cache, L * hkv * d, "k_cache"), _bf16(v_cache, L * hkv * d, "v_cache"),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_phase1_prepare")


def pulsar_phase1_attend(geom: Geom, attn: Attn, k_cache, v_cache, o, ws, stream=None):
    import torch
    L = geom.n_blocks * geom.block_size
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    rc = lib().pulsar_phase1_attend(
        ctypes.byref(geom), ctypes.byref(attn), _bf16(k_cache, L * hkv * d, "k_cache"),
        _bf16(v_cache, L * hkv * d, "v_cache"), _ptr(o, torch.float32, L * hq * d, "o"),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_phase1_attend")


def pulsar_phase2_num_parts(attn: Attn, batch, n_shards, shard_len, q_len, has_self) -> int:
    n = lib().pulsar_phase2_num_parts(ctypes.byref(attn), batch, n_shards, shard_len, q_len,
                                      1 if has_self else 0)
    if n <= 0:
        raise PulsarError(n, "pulsar_phase2_num_parts")
    return n


def pulsar_phase2_workspace_bytes(attn: Attn, batch, q_len, has_self) -> int:
    return lib().pulsar_phase2_workspace_bytes(ctypes.byref(attn), batch, q_len,
                                               1 if has_self else 0)


def pulsar_phase2_query(attn: Attn, batch, n_shards, shard_len, qq, q_len, q_pos0, k_cache,
                        v_cache, k_self, v_self, o_part, lse_part, n_parts, ws, stream=None):
    import torch
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kv_n = batch * n_shards * hkv * shard_len * d
    self_n = batch * q_len * hkv * d
    rows = batch * n_parts * q_len * hq
    rc = lib().pulsar_phase2_query(
        ctypes.byref(attn), batch, n_shards, shard_len, _bf16(qq, batch * q_len * hq * d, "qq"),
        q_len, int(q_pos0), _bf16(k_cache, kv_n, "k_cache", allow_none=n_shards == 0),
        _bf16(v_cache, kv_n, "v_cache", allow_none=n_shards == 0),
        _bf16(k_self, self_n, "k_self", allow_none=True),
        _bf16(v_self, self_n, "v_self", allow_none=True),
        _ptr(o_part, torch.float32, rows * d, "o_part"), _ptr(lse_part, torch.float32, rows, "lse_part"),
        n_parts, _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_phase2_query")


def pulsar_phase2_query_noalloc(attn: Attn, batch, n_shards, shard_len, qq, q_len, q_pos0,
                                k_cache, v_cache, k_self, v_self, o_part, lse_part, n_parts,
                                stream=None):
    """pulsar_phase2_query with the library's fixed scratch in place of a workspace."""
    import torch
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kv_n = batch * n_shards * hkv * shard_len * d
    self_n = batch * q_len * hkv * d
    rows = batch * n_parts * q_len * hq
    rc = lib().pulsar_phase2_query_noalloc(
        ctypes.byref(attn), batch, n_shards, shard_len, _bf16(qq, batch * q_len * hq * d, "qq"),
        q_len, int(q_pos0), _bf16(k_cache, kv_n, "k_cache", allow_none=n_shards == 0),
        _bf16(v_cache, kv_n, "v_cache", allow_none=n_shards == 0),
        _bf16(k_self, self_n, "k_self", allow_none=True),
        _bf16(v_self, self_n, "v_self", allow_none=True),
        _ptr(o_part, torch.float32, rows * d, "o_part"), _ptr(lse_part, torch.float32, rows, "lse_part"),
        n_parts, _stream(stream))
    _check(rc, "pulsar_phase2_query_noalloc")


def pulsar_phase2_noalloc_max_bytes() -> int:
    return lib().pulsar_phase2_noalloc_max_bytes()


def pulsar_prefix_rows_len(geom: Geom) -> int:
    return lib().pulsar_prefix_rows_len(ctypes.byref(geom))


def pulsar_phase1_prefix_rows(geom: Geom, attn: Attn, k_cache, v_cache, o_prefix, ws, stream=None):
    import torch
    L = geom.n_blocks * geom.block_size
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    n = pulsar_prefix_rows_len(geom)
    rc = lib().pulsar_phase1_prefix_rows(
        ctypes.byref(geom), ctypes.byref(attn), _bf16(k_cache, L * hkv * d, "k_cache"),
        _bf16(v_cache, L * hkv * d, "v_cache"),
        _ptr(o_prefix, torch.float32, max(n, 0) * hq * d, "o_prefix", allow_none=n <= 0),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_phase1_prefix_rows")


def pulsar_self_append(attn: Attn, batch, cap, n_self, n_new, self_pos0, k_new, v_new,
                       k_self_cache, v_self_cache, stream=None):
    hkv, d = attn.n_kv_heads, attn.head_dim
    new_n = batch * n_new * hkv * d
    cache_n = batch * cap * hkv * d
    rc = lib().pulsar_self_append(
        ctypes.byref(attn), batch, cap, n_self, n_new, int(self_pos0),
        _bf16(k_new, new_n, "k_new"), _bf16(v_new, new_n, "v_new"),
        _bf16(k_self_cache, cache_n, "k_self_cache"), _bf16(v_self_cache, cache_n, "v_self_cache"),
        _stream(stream))
    _check(rc, "pulsar_self_append")


def pulsar_phase2_decode(attn: Attn, batch, n_shards, shard_len, qq, q_len, k_cache, v_cache,
                         k_self_cache, v_self_cache, cap, n_self, self_pos0, o_part, lse_part,
                         n_parts, ws, stream=None):
    import torch
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kv_n = batch * n_shards * hkv * shard_len * d
    cache_n = batch * cap * hkv * d
    rows = batch * n_parts * q_len * hq
    rc = lib().pulsar_phase2_decode(
        ctypes.byref(attn), batch, n_shards, shard_len, _bf16(qq, batch * q_len * hq * d, "qq"),
        q_len, _bf16(k_cache, kv_n, "k_cache", allow_none=n_shards == 0),
        _bf16(v_cache, kv_n, "v_cache", allow_none=n_shards == 0),
        _bf16(k_self_cache, cache_n, "k_self_cache"), _bf16(v_self_cache, cache_n, "v_self_cache"),
        cap, n_self, int(self_pos0), _ptr(o_part, torch.float32, rows * d, "o_part"),
        _ptr(lse_part, torch.float32, rows, "lse_part"), n_parts, _ptr(ws, torch.uint8, 0, "ws"),
        ws.numel(), _stream(stream))
    _check(rc, "pulsar_phase2_decode")


def pulsar_decode_step_workspace_bytes(attn: Attn, batch, q_len) -> int:
    return lib().pulsar_decode_step_workspace_bytes(ctypes.byref(attn), batch, q_len)


def pulsar_decode_step(attn: Attn, batch, n_shards, shard_len, qq, k_new, v_new, q_len, k_cache,
                       v_cache, k_self_cache, v_self_cache, cap, n_self, self_pos0, o_part,
                       lse_part, n_parts, o, lse, ws, stream=None):
    import torch
    hq, hkv, d = attn.n_q_heads, attn.n_kv_heads, attn.head_dim
    kv_n = batch * n_shards * hkv * shard_len * d
    cache_n = batch * cap * hkv * d
    rows = batch * n_parts * q_len * hq
    rc = lib().pulsar_decode_step(
        ctypes.byref(attn), batch, n_shards, shard_len, _bf16(qq, batch * q_len * hq * d, "qq"),
        _bf16(k_new, batch * q_len * hkv * d, "k_new"), _bf16(v_new, batch * q_len * hkv * d, "v_new"),
        q_len, _bf16(k_cache, kv_n, "k_cache", allow_none=n_shards == 0),
        _bf16(v_cache, kv_n, "v_cache", allow_none=n_shards == 0),
        _bf16(k_self_cache, cache_n, "k_self_cache"), _bf16(v_self_cache, cache_n, "v_self_cache"),
        cap, n_self, int(self_pos0), _ptr(o_part, torch.float32, rows * d, "o_part"),
        _ptr(lse_part, torch.float32, rows, "lse_part"), n_parts,
        _ptr(o, torch.float32, batch * q_len * hq * d, "o"),
        _ptr(lse, torch.float32, batch * q_len * hq, "lse", allow_none=True),
        _ptr(ws, torch.uint8, 0, "ws"), ws.numel(), _stream(stream))
    _check(rc, "pulsar_decode_step")


def pulsar_lse_merge(batch, n_parts, q_len, n_q_heads, head_dim, o_part, lse_part, o, lse,
                     stream=None):
    import torch
    rows = batch * q_len * n_q_heads
    rc = lib().pulsar_lse_merge(
        batch, n_parts, q_len, n_q_heads, head_dim,
        _ptr(o_part, torch.float32, rows * n_parts * head_dim, "o_part"),
        _ptr(lse_part, torch.float32, rows * n_parts, "lse_part"),
        _ptr(o, torch.float32, rows * head_dim, "o"),
        _ptr(lse, torch.float32, rows, "lse", allow_none=True), _stream(stream))
    _check(rc, "pulsar_lse_merge")


def pulsar_strerror(code: int) -> str:
    return strerror(code)
