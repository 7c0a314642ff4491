"""Selection quality on planted-needle inputs (needs an MI355X).

The selection-quality diagnostic of the PISA reading page (§7.2, Table 7)
needs a trained model and its prompts, which are not available; planted
needles stand in for them (see hierarchical_block_selection_amd.inputs).  For
PISA, its eq. (9) ablations PISA-1 and PISA-2, and the flat BSA selector (all
on the GPU), against the exhaustive reference
(the oracle's flat selection by the exact leaf LSE over raw keys, summed over
the group's heads, with the same forcing), on sampled rows:

* Recall@K with the forced blocks counted, and net recall without them;
* retained attention mass and its ratio to the reference set's mass;
* needle hit rate: how often the needle block is selected at its target row.

The test asserts the metrics' ranges, the reference and BSA finding the
needles, and guards the measured quality with margins: PISA's recall, mass
ratio and needle hits at the N(0,1/d) scale, and with N(0,1) entries the
ordering of Table 7 (PISA above PISA-1, PISA-2 not below it).  The measured
numbers are printed, and written as JSON to the path in the PISA_QUALITY_OUT
environment variable when it is set.
"""
import json
import math
import os
import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from hierarchical_block_selection_amd import (Problem, pisa_bsa_select, pisa_build_pyramid,
                                              pisa_select)
from hierarchical_block_selection_amd.inputs import WORKLOADS, prefill_inputs

pytestmark = pytest.mark.gpu


def _quality(cfg_name, heads, rows_per_head, seed_rows=0, recipe=None):
    cfg = WORKLOADS[cfg_name]
    recipe = recipe or cfg["recipe"]
    prob = Problem(cfg["batch"], cfg["heads_q"], cfg["heads_kv"], cfg["seq_len"], cfg["head_dim"],
                   block=cfg["block"], topk=cfg["topk"], dtype=cfg["dtype"])
    print(f"[case] quality {cfg_name} {recipe} heads={heads}", flush=True)
    inp = prefill_inputs(prob.batch, prob.heads_q, prob.heads_kv, prob.seq_len, prob.head_dim,
                         prob.dtype, seed=cfg["seed"], recipe=recipe,
                         n_needles=cfg["n_needles"], block=prob.block, device="cuda")
    pyr = pisa_build_pyramid(prob, inp.k)
    pidx, _ = pisa_select(prob, inp.q, inp.k, pyr, want_score=False)
    # the eq. (9) ablations PISA-1 (mean) and PISA-2 (mean + var/2)
    p1idx, _ = pisa_select(replace(prob, score="mean"), inp.q, inp.k, pyr, want_score=False)
    p2idx, _ = pisa_select(replace(prob, score="mean_var"), inp.q, inp.k, pyr, want_score=False)
    bidx, _ = pisa_bsa_select(prob, inp.q, pyr, want_score=False)
    torch.cuda.synchronize()
    C, K, G = prob.block, prob.topk, prob.group
    rng = np.random.default_rng(seed_rows)
    names = ("pisa", "pisa1", "pisa2", "bsa", "exhaustive")
    stats = {name: [] for name in names}
    hits = {name: 0 for name in names}
    n_needles = 0
    for h in heads:
        keys = inp.k[0, h].double().cpu().numpy()
        qg = inp.q[0, h * G:(h + 1) * G].double().cpu().numpy()
        needle_rows = {nd.target_row: nd.block for nd in inp.needles
                       if nd.batch == 0 and nd.kv_head == h}
        rows = sorted(set(needle_rows) | set(
            int(x) for x in rng.integers(K * C, prob.seq_len, rows_per_head)))
        got = {"pisa": pidx[0, h].cpu().numpy(), "pisa1": p1idx[0, h].cpu().numpy(),
               "pisa2": p2idx[0, h].cpu().numpy(), "bsa": bidx[0, h].cpu().numpy()}
        for t in rows:
            ref = oracle.select_exhaustive_row(qg[:, t], keys, t, C, K, True, True).leaves
            sets = {name: v[t] for name, v in got.items()}
            sets["exhaustive"] = ref
            for name, sel in sets.items():
                stats[name].append(oracle.selection_quality(sel, ref, qg[:, t], keys, t, C, K))
            if t in needle_rows:
                n_needles += 1
                for name, sel in sets.items():
                    hits[name] += int(needle_rows[t] in set(int(x) for x in sel))
    out = {"workload": cfg_name, "recipe": recipe, "rows": len(stats["pisa"]),
           "needle_rows": n_needles}
    for name in stats:
        arr = {k: float(np.mean([s[k] for s in stats[name]])) for k in stats[name][0]}
        arr["needle_hit_rate"] = hits[name] / max(n_needles, 1)
        out[name] = arr
    return out


def _report(res):
    print(json.dumps(res, indent=1), flush=True)
    path = os.environ.get("PISA_QUALITY_OUT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(res) + "\n")


def _check(res, needles_clear=True):
    for name in ("pisa", "pisa1", "pisa2", "bsa", "exhaustive"):
        m = res[name]
        for key in ("recall", "net_recall", "retained_mass", "mass_ratio", "needle_hit_rate"):
            assert 0.0 <= m[key] <= 1.0 + 1e-9 or key == "mass_ratio", (name, key, m[key])
    assert res["exhaustive"]["recall"] == pytest.approx(1.0)
    # A needle block's keys point along its target query: the exact reference
    # and the flat mean-summary selector both find it.
    if needles_clear:
        assert res["exhaustive"]["needle_hit_rate"] >= 0.9
        assert res["bsa"]["needle_hit_rate"] >= 0.9
    for name in ("pisa", "pisa1", "pisa2"):
        assert res[name]["recall"] > 0.0


def _guard_small_scale(res, min_recall):
    # measured: recall 0.77 (c2) / 0.59 (c3), mass ratio 0.9998 / 0.9996,
    # every needle found; the margins leave room for ties broken otherwise
    assert res["pisa"]["recall"] >= min_recall, res["pisa"]
    assert res["pisa"]["mass_ratio"] >= 0.999, res["pisa"]
    assert res["pisa"]["needle_hit_rate"] >= 0.9, res["pisa"]


def test_quality_needles_c2():
    res = _quality("c2", heads=range(0, 16, 2), rows_per_head=24)
    _report(res)
    _check(res)
    _guard_small_scale(res, 0.65)


def test_quality_needles_c3():
    res = _quality("c3", heads=range(0, 8, 2), rows_per_head=16, seed_rows=1)
    _report(res)
    _check(res)
    _guard_small_scale(res, 0.5)


def test_quality_needles_c2_unit_variance():
    """The same shape with N(0,1) entries: logits spread widely, so the LSE of
    a node's children and their mean part ways (the regime where eq. (9)'s
    truncations and eq. (7) differ)."""
    res = _quality("c2", heads=range(0, 16, 4), rows_per_head=24, seed_rows=2, recipe="unit")
    _report(res)
    # with N(0,1) noise the planted blocks no longer stand out from the
    # strongest random blocks, so the needles are not required
    _check(res, needles_clear=False)
    # Table 7's ordering (measured recall 0.653 / 0.639 / 0.570, mass ratio
    # 0.966 / 0.962 / 0.946 for PISA / PISA-2 / PISA-1)
    assert res["pisa"]["recall"] >= res["pisa1"]["recall"] + 0.03, res
    assert res["pisa2"]["recall"] >= res["pisa1"]["recall"], res
    assert res["pisa"]["mass_ratio"] >= res["pisa1"]["mass_ratio"], res
    assert res["pisa"]["mass_ratio"] >= 0.95, res["pisa"]
