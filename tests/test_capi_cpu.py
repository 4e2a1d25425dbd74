"""The C-ABI library loads without a GPU, exports every declared entry point,
and rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

from long_context_blockwise_max_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pulsar.h")

needs_lib = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libpulsar.so not built")

FAKE = ctypes.c_void_p(0x10000)          # aligned, never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10008)      # not 16-byte aligned


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(pulsar_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("pulsar_select", "pulsar_phase1_encode", "pulsar_phase2_query", "pulsar_lse_merge"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def geom(**kw):
    d = dict(n_blocks=8, block_size=16384, chunk_size=32, budget_chunks=64, sink_size=64,
             vocab_size=128256)
    d.update(kw)
    return B.make_geom(**d)


ATTN = B.make_attn(32, 8, 128, 500000.0)


@needs_lib
def test_workspace_and_kept_chunks():
    g = geom()
    assert B.pulsar_kept_chunks(g) == 64
    assert B.pulsar_kept_chunks(geom(budget_chunks=10 ** 6)) == 512
    ws_sel = B.pulsar_workspace_bytes(g, None)
    ws_all = B.pulsar_workspace_bytes(g, ATTN)
    assert ws_sel >= 128256 * 4
    # rotated queries (L x Hq x d bf16) + prefix lists + work order
    assert ws_all >= ws_sel + 131072 * 32 * 128 * 2
    assert B.pulsar_workspace_bytes(geom(block_size=100), ATTN) == 0    # not a chunk multiple
    assert B.pulsar_workspace_bytes(geom(chunk_size=12, block_size=1200), ATTN) == 0  # chunk % 8
    assert B.pulsar_workspace_bytes(geom(sink_size=60), ATTN) == 0     # sink % 8
    assert B.pulsar_workspace_bytes(g, B.make_attn(32, 8, 96, 5e5)) == 0   # head_dim
    assert B.pulsar_workspace_bytes(g, B.make_attn(30, 8, 128, 5e5)) == 0  # Hq % Hkv


@needs_lib
@pytest.mark.parametrize("bad", [
    dict(n_blocks=0), dict(block_size=0), dict(chunk_size=0), dict(budget_chunks=-1),
    dict(sink_size=-1), dict(vocab_size=0), dict(block_size=100), dict(sink_size=10 ** 9),
])
def test_select_rejects_bad_geometry(bad):
    lib = B.lib()
    rc = lib.pulsar_select(ctypes.byref(geom(**bad)), FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert rc == B.PULSAR_EINVAL


@needs_lib
def test_select_rejects_pointers_and_small_workspace():
    lib = B.lib()
    g = geom()
    assert lib.pulsar_select(ctypes.byref(g), None, FAKE, None, None, FAKE, 1 << 30, None) == B.PULSAR_EINVAL
    assert lib.pulsar_select(ctypes.byref(g), FAKE_MIS, FAKE, None, None, FAKE, 1 << 30, None) == B.PULSAR_EINVAL
    assert lib.pulsar_select(ctypes.byref(g), FAKE, FAKE, None, None, FAKE, 16, None) == B.PULSAR_EWORKSPACE
    assert lib.pulsar_select(ctypes.byref(g), FAKE, FAKE, None, None, None, 1 << 30, None) == B.PULSAR_EWORKSPACE
    big = geom(vocab_size=(1 << 20) + 1)
    assert lib.pulsar_select(ctypes.byref(big), FAKE, FAKE, None, None, FAKE, 1 << 30, None) == B.PULSAR_EUNSUPPORTED


@needs_lib
def test_select_method_rejects_bad_arguments():
    lib = B.lib()

    def sm(g, method, tok=FAKE, sel=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.pulsar_select_method(ctypes.byref(g), method, 0, tok, sel, ws, wsb, None)

    g = geom()
    assert sm(g, 5) == B.PULSAR_EINVAL and sm(g, -1) == B.PULSAR_EINVAL   # unknown method
    assert sm(geom(n_blocks=0), 1) == B.PULSAR_EINVAL
    assert sm(g, 1, tok=None) == B.PULSAR_EINVAL            # mean IDF reads the tokens
    assert sm(g, 2, tok=FAKE_MIS) == B.PULSAR_EINVAL        # so does entropy
    assert sm(g, 1, wsb=16) == B.PULSAR_EWORKSPACE
    assert sm(g, 4, ws=None) == B.PULSAR_EWORKSPACE
    # exact order keys must fit 256 bits: N^chunk for mean IDF, chunk^chunk for entropy
    assert sm(geom(n_blocks=300, block_size=1024, budget_chunks=4), 1) == B.PULSAR_EUNSUPPORTED
    assert sm(geom(chunk_size=64), 2) == B.PULSAR_EUNSUPPORTED


@needs_lib
def test_phase1_rejects_bad_arguments():
    lib = B.lib()
    g = geom()
    args = [FAKE] * 7
    ws = B.pulsar_workspace_bytes(g, ATTN)

    def call(gg, aa, ptrs, wsb):
        return lib.pulsar_phase1_encode(ctypes.byref(gg), ctypes.byref(aa), *ptrs, FAKE, wsb, None)

    assert call(g, ATTN, args, ws - 1) == B.PULSAR_EWORKSPACE
    assert call(g, B.make_attn(32, 8, 80, 5e5), args, ws) == B.PULSAR_EUNSUPPORTED
    assert call(g, B.make_attn(24, 8, 128, 5e5), args, ws) == B.PULSAR_EUNSUPPORTED  # group of 3
    assert call(g, B.make_attn(32, 8, 128, 1.0), args, ws) == B.PULSAR_EINVAL
    bad = B.make_attn(32, 8, 128, 5e5)
    bad.rope_scaling = 2
    assert call(g, bad, args, ws) == B.PULSAR_EINVAL
    for i in range(7):
        p = list(args)
        p[i] = None if i != 4 else FAKE_MIS
        assert call(g, ATTN, p, ws) == B.PULSAR_EINVAL, i


@needs_lib
def test_phase1_halves_reject_bad_arguments():
    lib = B.lib()
    g = geom()
    ws = B.pulsar_workspace_bytes(g, ATTN)

    def prep(gg, aa, ptrs, wsb):
        return lib.pulsar_phase1_prepare(ctypes.byref(gg), ctypes.byref(aa), *ptrs, FAKE, wsb, None)

    def att(gg, aa, ptrs, wsb):
        return lib.pulsar_phase1_attend(ctypes.byref(gg), ctypes.byref(aa), *ptrs, FAKE, wsb, None)

    assert prep(g, ATTN, [FAKE] * 6, ws - 1) == B.PULSAR_EWORKSPACE
    assert att(g, ATTN, [FAKE] * 3, ws - 1) == B.PULSAR_EWORKSPACE
    assert prep(geom(block_size=100), ATTN, [FAKE] * 6, ws) == B.PULSAR_EINVAL
    assert att(g, B.make_attn(32, 8, 80, 5e5), [FAKE] * 3, ws) == B.PULSAR_EUNSUPPORTED
    for i in range(6):
        p = [FAKE] * 6
        p[i] = None
        assert prep(g, ATTN, p, ws) == B.PULSAR_EINVAL, i
    for i in range(3):
        p = [FAKE] * 3
        p[i] = FAKE_MIS
        assert att(g, ATTN, p, ws) == B.PULSAR_EINVAL, i


@needs_lib
def test_phase2_part_count_and_rejections():
    # every shard split alike; the self tiles share the shards' parts
    n = B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, 64, True)
    assert n >= 8 and n % 8 == 0
    assert B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, 64, False) == n
    assert B.pulsar_phase2_num_parts(ATTN, 8, 16, 32768, 1, True) >= 16
    assert B.pulsar_phase2_num_parts(ATTN, 2, 0, 0, 64, True) == 1     # the self shard only
    # tiny shards never get an empty part
    for shard_len in (1, 63, 64, 65, 200):
        nn = B.pulsar_phase2_num_parts(ATTN, 1, 2, shard_len, 4, False)
        assert nn // 2 <= (shard_len + 63) // 64
    lib = B.lib()
    with pytest.raises(B.PulsarError):
        B.pulsar_phase2_num_parts(ATTN, 0, 8, 16384, 64, True)
    ws2 = B.pulsar_phase2_workspace_bytes(ATTN, 1, 64, True)
    assert ws2 >= 64 * (32 + 8) * 128 * 2
    assert B.pulsar_phase2_workspace_bytes(ATTN, 1, 64, False) < ws2

    def q2(*args):
        return lib.pulsar_phase2_query(ctypes.byref(ATTN), *args)

    assert q2(1, 8, 16384, FAKE, 64, 131072, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n + 1, FAKE, ws2,
              None) == B.PULSAR_EINVAL                # wrong part count
    assert q2(1, 8, 16384, FAKE, 64, 131072, FAKE, FAKE, FAKE, None, FAKE, FAKE, n, FAKE, ws2,
              None) == B.PULSAR_EINVAL                # k_self without v_self
    assert q2(1, 8, 16384, FAKE, 64, -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n, FAKE, ws2,
              None) == B.PULSAR_EINVAL                # negative position
    assert q2(1, 8, 16384, FAKE, 64, 131072, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n, FAKE, ws2 - 1,
              None) == B.PULSAR_EWORKSPACE
    # a query so long that the grid would pass 2^31 - 1 workgroups
    # (4 sequences x 8 KV heads x 2^20 row groups x 64 parts = 2^31)
    big_q = 1 << 26
    n_big = B.pulsar_phase2_num_parts(ATTN, 4, 64, 64, big_q, False)
    assert n_big == 64
    assert q2(4, 64, 64, FAKE, big_q, 131072, FAKE, FAKE, None, None, FAKE, FAKE, n_big, FAKE,
              1 << 62, None) == B.PULSAR_EUNSUPPORTED
    n_odd = B.pulsar_phase2_num_parts(ATTN, 1, 8, 1001, 64, True)
    assert q2(1, 8, 1001, FAKE, 64, 131072, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n_odd, FAKE, ws2,
              None) == B.PULSAR_EUNSUPPORTED          # shard length not a multiple of 8


@needs_lib
def test_merge_rejections_and_strerror():
    lib = B.lib()
    assert lib.pulsar_lse_merge(0, 4, 64, 32, 128, FAKE, FAKE, FAKE, None, None) == B.PULSAR_EINVAL
    assert lib.pulsar_lse_merge(1, 4, 64, 32, 96, FAKE, FAKE, FAKE, None, None) == B.PULSAR_EUNSUPPORTED
    assert lib.pulsar_lse_merge(1, 4, 64, 32, 128, FAKE_MIS, FAKE, FAKE, None, None) == B.PULSAR_EINVAL
    # sizes whose row counts or grid would not fit the launch
    assert lib.pulsar_lse_merge(1, 4, 1 << 26, 64, 128, FAKE, FAKE, FAKE, None, None) == B.PULSAR_EUNSUPPORTED
    assert lib.pulsar_lse_merge(1 << 10, 4, 1 << 20, 32, 128, FAKE, FAKE, FAKE, None,
                                None) == B.PULSAR_EUNSUPPORTED
    for c in (0, -1, -2, -3, -4, 7):
        assert isinstance(B.strerror(c), str) and B.strerror(c)


@needs_lib
def test_generation_calls_reject_bad_arguments():
    lib = B.lib()
    A = ctypes.byref(ATTN)

    def app(batch, cap, n_self, n_new, pos0=0, ptrs=None):
        p = ptrs or [FAKE] * 4
        return lib.pulsar_self_append(A, batch, cap, n_self, n_new, pos0, *p, None)

    assert app(1, 64, 60, 5) == B.PULSAR_EINVAL            # past the capacity
    assert app(1, 60, 0, 1) == B.PULSAR_EUNSUPPORTED       # capacity not a multiple of 8
    assert app(0, 64, 0, 1) == B.PULSAR_EINVAL
    assert app(1, 64, 0, 0) == B.PULSAR_EINVAL
    assert app(1, 64, 0, 1, pos0=-1) == B.PULSAR_EINVAL
    assert app(1, 64, 0, 1, ptrs=[FAKE, FAKE, FAKE_MIS, FAKE]) == B.PULSAR_EINVAL
    n = B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, 1, True)
    ws = B.pulsar_phase2_workspace_bytes(ATTN, 1, 1, False)

    def dec(q_len, cap, n_self, n_parts=n, wsb=ws):
        return lib.pulsar_phase2_decode(A, 1, 8, 16384, FAKE, q_len, FAKE, FAKE, FAKE, FAKE, cap,
                                        n_self, 131072, FAKE, FAKE, n_parts, FAKE, wsb, None)

    assert dec(1, 128, 65, n_parts=n + 1) == B.PULSAR_EINVAL
    assert dec(1, 128, 129) == B.PULSAR_EINVAL             # more self tokens than the capacity
    assert dec(1, 120, 0) == B.PULSAR_EINVAL               # fewer self tokens than queries
    assert dec(1, 124, 65) == B.PULSAR_EUNSUPPORTED        # capacity not a multiple of 8
    assert dec(1, 128, 65, wsb=ws - 1) == B.PULSAR_EWORKSPACE


@needs_lib
def test_noalloc_query_rejects_on_the_host():
    """The no-allocation Phase-2 query validates like pulsar_phase2_query, and
    rejects a workspace larger than its fixed array before touching a device."""
    lib = B.lib()
    cap = B.pulsar_phase2_noalloc_max_bytes()
    assert cap == 8 << 20
    A = ctypes.byref(ATTN)

    def q2(batch, q_len, n_parts, has_self=True, pos0=131072):
        s = FAKE if has_self else None
        return lib.pulsar_phase2_query_noalloc(A, batch, 8, 16384, FAKE, q_len, pos0, FAKE, FAKE, s,
                                               s, FAKE, FAKE, n_parts, None)

    fits = max(q for q in range(1, 2000) if B.pulsar_phase2_workspace_bytes(ATTN, 1, q, True) <= cap)
    assert fits == 678
    n_big = B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, fits + 1, True)
    assert q2(1, fits + 1, n_big) == B.PULSAR_EUNSUPPORTED       # workspace above the array
    n8 = B.pulsar_phase2_num_parts(ATTN, 8, 8, 16384, 100, True)
    assert q2(8, 100, n8) == B.PULSAR_EUNSUPPORTED               # 800 tokens of batch 8
    n = B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, 64, True)
    assert q2(1, 64, n + 1) == B.PULSAR_EINVAL                   # wrong part count
    assert q2(1, 64, n, pos0=-1) == B.PULSAR_EINVAL
    assert lib.pulsar_phase2_query_noalloc(A, 1, 8, 16384, FAKE, 64, 0, FAKE, FAKE, FAKE, None,
                                           FAKE, FAKE, n, None) == B.PULSAR_EINVAL


@needs_lib
def test_decode_step_rejects_on_the_host():
    lib = B.lib()
    A = ctypes.byref(ATTN)
    n = B.pulsar_phase2_num_parts(ATTN, 1, 8, 16384, 1, True)
    ws = B.pulsar_decode_step_workspace_bytes(ATTN, 1, 1)
    assert ws >= 32 * 128 * 2                              # one rotated query token

    def step(q_len=1, cap=128, n_self=64, n_parts=n, wsb=ws, pos0=131072, ptr=FAKE):
        return lib.pulsar_decode_step(A, 1, 8, 16384, FAKE, ptr, FAKE, q_len, FAKE, FAKE, FAKE, FAKE,
                                      cap, n_self, pos0, FAKE, FAKE, n_parts, FAKE, None, FAKE, wsb,
                                      None)

    assert step(n_parts=n + 1) == B.PULSAR_EINVAL
    assert step(n_self=128) == B.PULSAR_EINVAL            # no room for the new token
    assert step(cap=124, n_self=64) == B.PULSAR_EUNSUPPORTED
    assert step(wsb=ws - 1) == B.PULSAR_EWORKSPACE
    assert step(pos0=-1) == B.PULSAR_EINVAL
    assert step(ptr=FAKE_MIS) == B.PULSAR_EINVAL
