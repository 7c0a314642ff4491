"""Host-side logic of bench.py (no GPU): the work counts behind its
algorithmic flop and byte figures, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n,c,k,force", [(4096, 64, 8, True), (5000, 64, 16, True),
                                         (2065, 16, 5, True), (3000, 32, 7, False)])
def test_descent_counts_match_the_oracle_trace(n, c, k, force):
    """Scored child rows / raw keys per level, as the oracle's descent visits
    them on random data (the counts do not depend on the data)."""
    rng = np.random.default_rng(n + k)
    keys = rng.standard_normal((n, 16))
    q = rng.standard_normal(16)
    levels = oracle.build_pyramid(keys, c)
    sizes = [len(x) for x in levels]
    per_t = bench.descent_counts(n, c, k, force)
    for t in [0, 1, c - 1, c, c * k - 1, c * k, n - 1] + [int(x) for x in rng.integers(0, n, 25)]:
        sel = oracle.select_pisa_row(q, keys, levels, t, c, k, True, force)
        for rec in sel.trace:
            want = 0
            if rec.scored:
                rank = [i for i in rec.candidates if i not in rec.forced]
                want = (sum(len(oracle.node_children(i, rec.level, sizes, c, n, 2)) for i in rank)
                        if rec.level >= 2 else sum(min(c, n - i * c) for i in rank))
            assert bench.descent_row_counts(n, c, k, t, force)[rec.level] == want, (t, rec.level)
            assert per_t[rec.level][t] == want, (t, rec.level)


def test_attended_keys_match_the_selected_tokens():
    n, c, k = 3000, 64, 6
    keys = np.random.default_rng(3).standard_normal((n, 8))
    levels = oracle.build_pyramid(keys, c)
    q = np.random.default_rng(4).standard_normal(8)
    got = bench.attended_keys(n, c, k)
    for t in [0, 63, 64, 383, 384, 2999, 1234]:
        leaves = oracle.select_pisa_row(q, keys, levels, t, c, k, True, True).leaves
        want = sum(min(c, t + 1 - b * c) for b in leaves if b * c <= t)
        assert got[t] == want, t


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "GPU" in (r.stdout + r.stderr)
