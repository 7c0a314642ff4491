"""Comparison of the HIP path's outputs with the CPU oracle (test helper).

Protocol (tolerances are those the workloads state):
  * selection: leaf sets bit-exact on every row whose smallest Top-K margin over
    all scored levels exceeds 1e-3 (near-ties excluded); ranking scores of
    those rows within 1e-4 + 1e-5 |s| (fp32 dot products and LSE against fp64);
    structural checks on every row (ascending, no duplicates, -1 only at the
    tail, forced blocks present, every entry eligible, size = min(K, #eligible));
  * attention: the oracle attends with the GPU's own index row (ties cannot
    contaminate it); fp32 rows max|diff| <= 1e-3 max|o_ref|; bf16 rows
    max|diff| <= 2e-2 against fp64 and, tighter, normwise <= 1e-2;
    row LSE within 1e-3.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle

MARGIN = 1e-3


@dataclass
class Tally:
    rows: int = 0
    compared: int = 0
    mismatches: list = field(default_factory=list)

    def frac(self):
        return self.compared / max(self.rows, 1)


def check_structure(row, t, block, topk, n_leaves, causal, force):
    """Structural validity of one ascending, -1 padded leaf row."""
    row = [int(x) for x in row]
    valid = [x for x in row if x >= 0]
    n_valid = len(valid)
    assert row[:n_valid] == valid, f"padding not at the tail: {row}"
    assert all(x == -1 for x in row[n_valid:]), row
    assert valid == sorted(set(valid)), f"not ascending/unique: {row}"
    eligible = (t // block + 1) if causal else n_leaves
    assert all(0 <= x < eligible for x in valid), f"ineligible entry in {row} (t={t})"
    assert n_valid == min(topk, eligible), f"size {n_valid} != min(K, {eligible}) at t={t}"
    if causal:
        cur = t // block
        forced = {cur} | ({0, cur - 1} - {-1} if force else set())
        assert forced <= set(valid), f"forced {forced} missing from {row} at t={t}"


def compare_selection(kind, gpu_idx, gpu_score, q_group, keys, levels, rows, block, topk,
                      causal, force, scale, tally: Tally, variant: str = "lse"):
    """gpu_idx / gpu_score: [N, K] arrays of one (b, kv head).  Returns tally."""
    n_leaves = len(levels[0])
    for t in rows:
        check_structure(gpu_idx[t], t, block, topk, n_leaves, causal, force)
        qh = q_group[:, t, :]
        if kind == "pisa":
            sel = oracle.select_pisa_row(qh, keys, levels, t, block, topk, causal, force, scale,
                                         variant=variant)
        else:
            sel = oracle.select_bsa_row(qh, levels, t, block, topk, causal, force, scale)
        tally.rows += 1
        if sel.min_margin <= MARGIN:
            continue
        tally.compared += 1
        want = oracle.padded(sel.leaves, topk)
        got = [int(x) for x in gpu_idx[t]]
        if got != want:
            tally.mismatches.append((t, got, want, sel.min_margin))
            continue
        if gpu_score is not None:
            for pos, leaf in enumerate(got):
                if leaf < 0:
                    assert gpu_score[t, pos] == -math.inf
                elif leaf in sel.scores:
                    s = sel.scores[leaf]
                    assert abs(gpu_score[t, pos] - s) <= 1e-4 + 1e-5 * abs(s), (t, leaf, gpu_score[t, pos], s)
                else:
                    assert gpu_score[t, pos] == math.inf, (t, leaf, gpu_score[t, pos])
    return tally


def compare_attention(gpu_out, gpu_lse, q_group, keys, values, idx_rows, rows, block, causal,
                      scale, fp32: bool):
    """gpu_out: [G, N, d]; gpu_lse: [G, N] or None; idx_rows: [N, K] (GPU's own)."""
    worst = 0.0
    for t in rows:
        leaves = [int(x) for x in idx_rows[t] if x >= 0]
        ref, ref_lse = oracle.attend_row(q_group[:, t, :], keys, values, leaves, t, block, causal,
                                         scale)
        got = gpu_out[:, t, :].astype(np.float64)
        diff = np.abs(got - ref)
        if fp32:
            rel = diff.max() / max(np.abs(ref).max(), 1e-30)
            assert rel <= 1e-3, (t, rel)
            worst = max(worst, rel)
        else:
            assert diff.max() <= 2e-2, (t, diff.max())
            nrm = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
            assert nrm <= 1e-2, (t, nrm)
            worst = max(worst, nrm)
        if gpu_lse is not None:
            assert np.max(np.abs(gpu_lse[:, t] - ref_lse)) <= 1e-3, (t, gpu_lse[:, t], ref_lse)
    return worst


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy()
