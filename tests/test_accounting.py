"""Operation counts against the chunking page's printed tables (no GPU)."""
import json
import os

from chunked_causal_linear_amd.accounting import Shape, Work

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunking_page_tables.json")
T = json.load(open(GOLDEN, encoding="utf-8"))


def test_state_vs_kv_cache_table():
    d = T["state_vs_kv_cache"]["d"]
    for L, state, kv in T["state_vs_kv_cache"]["rows"]:
        s = Shape(L, d, 64)
        assert s.state_elements() == state
        assert s.kv_cache_elements() == kv
    # short sequences keep a larger state than the KV cache; long ones the reverse
    assert Shape(16, 64, 1).state_elements() > Shape(16, 64, 1).kv_cache_elements()
    assert Shape(32, 64, 1).state_elements() == Shape(32, 64, 1).kv_cache_elements()
    assert Shape(33, 64, 1).state_elements() < Shape(33, 64, 1).kv_cache_elements()


def test_cost_split_table():
    L, d = T["cost_split"]["L"], T["cost_split"]["d"]
    rows = T["cost_split"]["rows"]
    for C, fixed, prop, total, area in rows:
        s = Shape(L, d, C)
        assert s.state_macs() == fixed
        assert s.score_macs() == prop
        assert s.macs() == total
        assert s.intra_memory() == area
        # the generalised counter agrees with the page's closed form
        assert Work(1, L, d, d, d, C).page_macs() == total
    assert len({r[1] for r in rows}) == 1  # the fixed part never moves
    by_c = {r[0]: r[2] for r in rows}
    assert by_c[1024] == 1024 * by_c[1]  # proportional part exactly 1024x at 1024x C
    spread = rows[-1][3] / rows[0][3]
    assert spread > T["cost_split"]["claims"]["ends_differ_more_than"]
    assert round(spread, 2) == 16.74
    assert Shape(L, d, L).is_full_attention() and not Shape(L, d, 64).is_full_attention()
    assert Shape(L, d, 1).is_linear() and not Shape(L, d, 2).is_linear()


def test_growth_table():
    d = T["growth"]["d"]
    prev = None
    for L, full, c64 in T["growth"]["rows"]:
        assert Shape(L, d, L).macs() == full
        assert Shape(L, d, 64).macs() == c64
        if prev:
            assert c64 == 2 * prev[1]  # fixed C: doubling L doubles the work
            assert 3.5 < full / prev[0] <= 4.0  # C = L: roughly x4 (the square term dominates)
        prev = (full, c64)


def test_generalised_counts():
    # ragged last chunk: sum of c^2 over chunks
    w = Work(1, 10, 4, 4, 4, 4)
    assert w.page_macs() == 2 * 10 * 16 + (4 * 4 + 4 * 4 + 2 * 2) * 8
    assert w.causal_useful_macs() == 2 * 10 * 16 + (10 + 10 + 3) * 8
    # d_k != d_v
    w = Work(3, 64, 64, 256, 64, 64, normalize=True, fmap="favor")
    assert w.page_macs() == 3 * (2 * 64 * 256 * 64 + 64 * 64 * (256 + 64) + 2 * 64 * 256 + 64 * 64)
    assert w.fmap_macs() == 3 * 2 * 64 * 256 * 64


def test_headline_bytes():
    w = Work(128, 8192, 128, 128, 128, 64)
    assert w.fused_bytes() == 128 * 8192 * (3 * 128 * 2 + 128 * 2)
    assert w.page_flops() == 2 * 128 * (2 * 8192 * 128 * 128 + 2 * 8192 * 64 * 128)
