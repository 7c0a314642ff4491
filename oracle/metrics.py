"""Selection-quality diagnostics on the CPU — test infrastructure only.

Follows the selection-quality diagnostic of the PISA reading page (§7.2,
Figure 2 and Table 7): Recall@K of a selector's leaf set against a reference
set (forced blocks included), the attention mass the selected blocks retain,
and the ratio of that mass to the reference set's.  "Net recall" drops the
forced blocks from both sets, which the page's §8.3 notes is not reported.
Masses are shares of the full causal attention of each head, averaged over the
group's heads (the reference rule of §4.4).
"""
from __future__ import annotations

import math

import numpy as np

from .pisa_oracle import forced_nodes, logsumexp


def block_masses(q_heads, keys, t, block, scale=None):
    """Share of full causal attention mass of query t in each leaf block 0..t//C,
    averaged over the group's heads.  Returns an array of length t//C + 1."""
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    d = keys.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    c = t // block
    out = np.zeros(c + 1)
    for q in q_heads:
        z = scale * (keys[:t + 1] @ q)
        total = logsumexp(z)
        p = np.exp(z - total)
        for i in range(c + 1):
            out[i] += p[i * block:min((i + 1) * block, t + 1)].sum()
    return out / len(q_heads)


def selection_quality(selected, reference, q_heads, keys, t, block, topk,
                      force_first_prev=True, scale=None):
    """Recall@K, net recall, retained mass and mass ratio for one query row.

    selected / reference: iterables of leaf indices (padding -1 ignored).
    """
    sel = {int(i) for i in selected if i >= 0}
    ref = {int(i) for i in reference if i >= 0}
    forced = forced_nodes(t, 1, block, True, force_first_prev)
    mass = block_masses(q_heads, keys, t, block, scale)
    kept = float(sum(mass[i] for i in sel))
    kept_ref = float(sum(mass[i] for i in ref))
    free = max(topk - len(forced), 1)
    return {
        "recall": len(sel & ref) / topk,
        "net_recall": len((sel - forced) & (ref - forced)) / free,
        "retained_mass": kept,
        "mass_ratio": kept / kept_ref if kept_ref > 0 else 1.0,
    }
