"""CPU check of the clamps the GEMM kernels apply to what they read from the
workspace (moe_denoise_forward_amd/csrc/plan.h): per-expert pair counts are
clamped to the list capacity and fitted, in expert order, into the L*k rows of
the act / slot buffers, and row ids are clamped into their buffer.  Whatever the
counts (stale, negative, huge: a workspace left by another call, or counters a
failed call never cleared), every tile the kernels derive stays in bounds.

The header is compiled for the host with hipcc (no device code runs) and
driven with random and adversarial counts; the expected plan is computed here
from its definition."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpu", "plan_check.cpp")


@pytest.fixture(scope="module")
def plan_bin(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("plan") / "plan_check")
    subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", SRC, "-o", out],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return out


def _expected(raw, cap, total, ids):
    rows, first, s = [], [], 0
    for c in raw:
        c = min(max(c, 0), cap)
        f = min(s, total)
        first.append(f)
        rows.append(min(s + c, total) - f)
        s += c
    return first, rows, [min(max(v, 0), total - 1) for v in ids]


def _cases():
    rng = np.random.default_rng(0)
    cases = []
    # valid counts: the plan is the plain exclusive scan
    for E, L, k in [(8, 32, 2), (128, 256, 8), (256, 70, 32), (4, 16384, 2)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(L)])
        raw = np.bincount(idx.ravel(), minlength=E).tolist()
        cases.append((E, L, L * k, raw, rng.integers(0, L * k, 16).tolist(), True))
    # stale / garbage counts: negative, past the capacity, summing past the rows
    for _ in range(200):
        E = int(rng.integers(1, 257))
        L = int(rng.integers(1, 3000))
        k = int(rng.integers(1, min(E, 32) + 1))
        raw = rng.integers(-2 ** 31, 2 ** 31, E).tolist()
        if rng.random() < 0.5:
            raw = rng.integers(-5, 3 * L, E).tolist()
        ids = rng.integers(-2 ** 31, 2 ** 31, 8).tolist() + [-1, 0, L * k - 1, L * k, L * k + 5]
        cases.append((E, L, L * k, raw, ids, False))
    # all 0xFF bytes (a poisoned workspace) and all at the capacity
    cases.append((128, 256, 2048, [-1] * 128, [-1] * 4, False))
    cases.append((128, 256, 2048, [256] * 128, [2047, 2048], False))
    return cases


def test_plan_clamps(plan_bin):
    cases = _cases()
    text = "".join(f"{E} {L} {T} {len(ids)} " + " ".join(map(str, raw)) + " " +
                   " ".join(map(str, ids)) + "\n" for E, L, T, raw, ids, _ in cases)
    out = subprocess.run([plan_bin], input=text, stdout=subprocess.PIPE, text=True, check=True)
    lines = out.stdout.strip().split("\n")
    assert len(lines) == len(cases)
    for (E, L, T, raw, ids, valid), line in zip(cases, lines):
        vals = list(map(int, line.split()))
        first, rows = vals[0:2 * E:2], vals[1:2 * E:2]
        cid = vals[2 * E:]
        ef, er, eid = _expected(raw, L, T, ids)
        assert first == ef and rows == er and cid == eid
        # the bounds the kernels rely on
        assert all(r >= 0 for r in rows) and all(r <= L for r in rows)
        assert sum(rows) <= T
        assert all(f + r <= T for f, r in zip(first, rows))
        assert all(0 <= v < T for v in cid)
        if valid:  # a real routing is left unchanged
            assert rows == raw and first == list(np.cumsum([0] + raw[:-1]))
