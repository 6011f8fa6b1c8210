"""CPU check of the phase kernels' tile order: tests/native/phase_order.cpp
includes the host+device functions the GEMM phase kernels (forward and
backward) call to map a workgroup's loop to tiles, and checks that every
(m-tile, n-tile) pair runs exactly once in both orders, that the XCD-affine
order gives run b % 8 to workgroup b in equal runs, and that the m-tiles of an
expert sharing an n-tile sit side by side in the list.  Cases: the routing of
the benchmark workloads (expert row counts from the oracle's dispatch of their
seeded inputs), empty and single experts, grids that are not a multiple of 8,
and random counts.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from workloads import bf16_value, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "phase_order.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("phase") / "phase_order")
    r = subprocess.run([HIPCC, "-O2", "-std=c++17", SRC, "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def _run(exe, cases):
    text = "".join(f"{BT} {NT} {grid} {len(c)} {' '.join(map(str, c))}\n" for BT, NT, grid, c in cases)
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("OK"), r.stdout + r.stderr
    assert int(r.stdout.split()[1]) == len(cases)


def _counts(name, T=None):
    inp = make_inputs(name, T=T, weights=False)
    wl = inp["workload"]
    x = bf16_value(inp["x"]).astype(np.float64)
    logits = oracle.router_logits(x, bf16_value(inp["Wg"]).astype(np.float64), inp["bias"])
    idx, _, _ = oracle.route(logits, wl.k)
    return [int(c) for c in oracle.dispatch(idx, wl.e_begin, wl.E_local, wl.G)["counts"]]


@pytest.mark.parametrize("name,T,NT1,NT2", [("mid", 4096, 8, 16), ("stress", 4096, 12, 16)])
def test_benchmark_routing(exe, name, T, NT1, NT2):
    c = _counts(name, T)
    _run(exe, [(256, nt, grid, c) for nt in (NT1, NT2) for grid in (256, 255, 8)])


def test_edge_cases(exe):
    _run(exe, [
        (256, 8, 256, [0, 0, 0]),            # nothing routed
        (256, 8, 256, [1]),                  # one row
        (256, 16, 256, [0, 700, 0, 0, 3]),   # empty experts between routed ones
        (128, 7, 1, [300, 5, 129]),          # one workgroup
        (256, 28, 256, [257] * 32),          # every expert one full m-tile and a one-row tail
        (256, 12, 256, [8103] + [1400] * 63),  # a hot expert
    ])


def test_random_counts(exe):
    rng = np.random.default_rng(7)
    cases = []
    for _ in range(400):
        E = int(rng.integers(1, 64))
        c = (rng.integers(0, 2000, E) * (rng.random(E) < 0.8)).tolist()
        cases.append((int(rng.choice([128, 256])), int(rng.integers(1, 30)),
                      int(rng.choice([256, 255, 248, 8, 7, 1, 512])), c))
    _run(exe, cases)
