"""CPU check of the persistent expert-wave kernel's static task order (8 per-XCD streams).

tests/native/sched_emu.cpp includes the same host+device schedule header the
kernel uses (combine_wave_level_amd/csrc/wave_sched.h) and checks, for the
given dispatch tables: every m-tile is dealt once and the XCDs hold the
same number of m-tiles to within one (whole-expert deals split an expert
only when an XCD fills up), every GEMM1 / GEMM2 tile and combine chunk has
exactly one ticket, every wait is on smaller tickets (no deadlock for any
grid), and a multi-threaded emulated run reaches every wait target.  The
schedule also equals the plain sequential greedy's, and the kernel's split
of the build over threads gives the same schedule.  Weight-streaming shapes
whose m-tiles do not divide evenly over the XCDs spread every m-tile's
output tiles over all of them instead.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "sched_emu.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BT = 128  # rows per m-tile of the expert GEMMs


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sched") / "sched_emu")
    r = subprocess.run([HIPCC, "-O2", "-std=c++17", "-pthread", SRC, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def _run(emu, counts, ready_counts, G, NT1, NT2, cb_parts=1, threads=2, seed=1, lag=1, whole=1):
    E_local = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    ready_off = np.concatenate([[0], np.cumsum(ready_counts)]).astype(int)
    assert len(ready_off) == E_local // G + 2
    inp = f"{E_local} {G} {BT} {NT1} {NT2} {cb_parts} {threads} {seed} {lag} {whole}\n"
    inp += " ".join(map(str, offsets)) + "\n" + " ".join(map(str, ready_off)) + "\n"
    r = subprocess.run([emu], input=inp, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    return r.stdout


def _tables_from_routing(idx, e_begin, E_local, G):
    m = oracle.dispatch(idx, e_begin, E_local, G)
    W = E_local // G
    ready = m["token_ready_wave"]
    ready_counts = [int((ready == s - 1).sum()) for s in range(W + 1)]
    return m["counts"], ready_counts


def test_tiny_layer_tables(emu):
    inp = make_inputs("tiny")
    l = oracle.router_logits(inp["x"], inp["Wg"])
    idx, _, _ = oracle.route(l, 2)
    counts, ready = _tables_from_routing(idx, 0, 8, 4)
    out = _run(emu, counts, ready, G=4, NT1=2 * 128 // 128, NT2=256 // 128)
    assert "W=2" in out


@pytest.mark.parametrize("G,lag,whole", [(1, 1, 1), (2, 4, 0), (4, 1, 1), (4, 4, 0), (16, 64, 1)])
def test_mid_layer_cut_tables(emu, G, lag, whole):
    inp = make_inputs("mid", T=300, weights=False)
    l = oracle.router_logits(oracle.decode_bf16(inp["x"]), oracle.decode_bf16(inp["Wg"]))
    idx, _, _ = oracle.route(l, 4)
    counts, ready = _tables_from_routing(idx, 0, 16, G)
    _run(emu, counts, ready, G=G, NT1=2 * 1024 // 128, NT2=4096 // 128, lag=lag, whole=whole)


def test_empty_experts_and_waves(emu):
    # experts 0-3 (wave 0) and 8-11 (wave 2) receive nothing
    counts = [0, 0, 0, 0, 300, 5, 0, 129, 0, 0, 0, 0, 1, 640, 2, 77]
    W = 4
    rng = np.random.default_rng(0)
    ready = list(rng.integers(0, 50, size=W + 1))
    _run(emu, counts, ready, G=4, NT1=4, NT2=8, threads=4, lag=3)


def test_many_waves_one_expert_each(emu):
    rng = np.random.default_rng(1)
    counts = list(rng.integers(0, 400, size=64))
    ready = list(rng.integers(0, 30, size=65))
    _run(emu, counts, ready, G=1, NT1=3, NT2=5, threads=5, seed=7, lag=11)


def test_without_fused_combine_and_single_expert(emu):
    _run(emu, [1000], [0, 7], G=1, NT1=16, NT2=56, cb_parts=0)
    _run(emu, [1], [3, 1], G=1, NT1=2, NT2=2, threads=1)


def test_all_tokens_without_local_pick(emu):
    _run(emu, [0, 0, 0, 0], [64, 0, 0], G=2, NT1=2, NT2=2)


def test_combine_split_into_column_parts(emu):
    # small batch: every combine chunk of tokens split into 14 column ranges
    rng = np.random.default_rng(3)
    counts = list(rng.integers(0, 40, size=32))
    ready = list(rng.integers(0, 20, size=9))
    out = _run(emu, counts, ready, G=4, NT1=32, NT2=112, cb_parts=14, threads=3, seed=5, whole=0)
    assert "W=8" in out


def test_many_mtiles_per_xcd(emu):
    # 64 experts of up to 40 m-tiles, one expert per wave: hundreds of
    # m-tiles per XCD, within the schedule's capacity
    rng = np.random.default_rng(11)
    counts = list(rng.integers(0, 40 * 128, size=64))
    ready = list(rng.integers(0, 50, size=65))
    _run(emu, counts, ready, G=1, NT1=2, NT2=3, threads=4, seed=9, lag=16)


def test_hot_expert_dealt_in_chunks(emu):
    # one expert holds most rows: it is split over the XCDs as they fill up
    counts = [30 * 128] + [128 * 2] * 15
    ready = [5, 40, 3, 9, 60]
    out = _run(emu, counts, ready, G=4, NT1=8, NT2=16, threads=3, seed=4, lag=4)
    # GEMM2 groups are capped by the lag (4 here)
    assert "max_group=4" in out


def test_gemm2_groups_span_an_experts_mtiles(emu):
    # experts of 1 to 12 m-tiles under the long lag: groups of up to 8 m-tiles
    rng = np.random.default_rng(31)
    counts = [int(c) for c in rng.integers(1, 12 * BT, size=16)]
    ready = [int(r) for r in rng.integers(0, 300, size=5)]
    out = _run(emu, counts, ready, G=4, NT1=8, NT2=16, threads=2, seed=8, lag=64)
    assert "max_group=8" in out


def test_lumpy_experts_and_a_hot_one_stay_balanced(emu):
    # the stress layer's shape: 64 experts of 5 to 7 m-tiles and one of 32
    # (greedy whole-expert deals alone left XCDs 8 m-tiles apart)
    rng = np.random.default_rng(12)
    counts = [int(c) for c in rng.integers(5 * BT - 60, 7 * BT, size=64)]
    counts[37] = 32 * BT
    ready = [int(r) for r in rng.integers(0, 900, size=17)]
    _run(emu, counts, ready, G=4, NT1=12, NT2=16, threads=2, seed=6, lag=64)


@pytest.mark.parametrize("counts,spread", [
    ([40, 0, 3, 17, 64, 0, 0, 9, 31, 2, 5, 64, 0, 1, 7, 12], True),     # 13 m-tiles: 13 % 8 != 0
    ([1] * 8 + [0] * 8, False),                                         # 8 m-tiles: dealt one per XCD
])
def test_small_batch_spread_and_dealt(emu, counts, spread):
    # decode-like: every expert at most one m-tile (BT = 128 rows)
    rng = np.random.default_rng(21)
    ready = [int(r) for r in rng.integers(0, 9, size=5)]
    for threads in (1, 3):
        out = _run(emu, counts, ready, G=4, NT1=32, NT2=56, cb_parts=14, threads=threads, seed=threads, lag=64,
                   whole=0)
        assert f"spread={int(spread)}" in out


def test_spread_needs_tiles_divisible_by_xcds(emu):
    # NT2 = 54 is not a multiple of 8: single m-tile dealing
    rng = np.random.default_rng(22)
    counts = list(rng.integers(0, 300, size=32))
    ready = list(rng.integers(0, 20, size=9))
    n_mt = sum((c + BT - 1) // BT for c in counts)
    assert n_mt % 8 != 0
    assert "spread=0" in _run(emu, counts, ready, G=4, NT1=32, NT2=54, cb_parts=3, threads=2, seed=3, lag=64, whole=0)
    # the same tables with NT2 = 56 spread, also with a lag shorter than the m-tile count
    assert "spread=1" in _run(emu, counts, ready, G=4, NT1=32, NT2=56, cb_parts=3, threads=2, seed=3, lag=5, whole=0)
