"""Pins of the host-side cost model against the figures the pages print."""
import pytest

from long_context_blockwise_max_amd import costs as C


def test_critical_host_ratio_matches_up_to_3_3x():
    """Abstract: Phase-1 per-GPU FLOPs up to 3.3x lower than Star Attention
    (Table 3 setting: four blocks, summaries of 512 tokens, 64-token sink).
    Per-host causal attention on the last host at 64K gives (2b)^2/(b+1600)^2."""
    r64 = C.critical_host_ratio_star_vs_pulsar(65536, 4, 512)
    assert r64 == pytest.approx(3.32, abs=0.005)
    # the saving grows with the per-host block (Section 4): 16K < 32K < 64K
    r16 = C.critical_host_ratio_star_vs_pulsar(16384, 4, 512)
    r32 = C.critical_host_ratio_star_vs_pulsar(32768, 4, 512)
    assert r16 < r32 < r64


def test_prefix_length_1600():
    assert C.prefix_len(3, 64, 32, 16) == 1600          # Section 4: 64 + 3 x 512
    assert C.prefix_len(0, 64, 32, 16) == 0


def test_row_flops_against_explicit_sum():
    # 2 blocks of 4 rows, sink 2, chunk 1, k 1, 1 head, d 1: block 0 rows see 1..4 keys,
    # block 1 has prefix 2 + 1 = 3 and rows see 4..7 keys
    want = 4 * (1 + 2 + 3 + 4 + 4 + 5 + 6 + 7)
    assert C.phase1_flops_rows(2, 4, 2, 1, 1, 1, 1) == want


def test_phase2_sizes():
    assert C.phase2_kv_bytes(1, 8, 16384, 8, 128) == 512 * 2 ** 20
    assert C.phase2_flops(1, 64, 131072, 32, 128) == pytest.approx(137.473e9, rel=1e-4)
