"""Plant plausible mistakes in a copy of the oracle and check that the pins catch
each one (no GPU).  The real oracle is never modified: each mutant is the oracle's
source text with one edit, loaded as a separate in-memory module."""
import os
import sys
import types

import pytest

import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pisa_oracle.py")
METRICS_SRC = os.path.join(ROOT, "oracle", "metrics.py")

# (name, text to find, replacement) -- each must occur exactly once.
MUTATIONS = [
    ("lse_replaced_by_mean", "return logsumexp(z)", "return float(np.mean(z))"),
    ("scale_dropped", "z = scale * (child_vecs @ q)", "z = (child_vecs @ q)"),
    ("child_index_shifted", "range(branch * node, branch * node + branch)",
     "range(branch * node + 1, branch * node + branch + 1)"),
    ("leaf_span_off_by_one", "keys[i * block:min((i + 1) * block, n)].mean(axis=0)",
     "keys[i * block:min((i + 1) * block + 1, n)].mean(axis=0)"),
    ("future_drop_strict", "cands = [i for i in cands if i <= limit]",
     "cands = [i for i in cands if i < limit]"),
    ("ranking_sign_flipped", "key=lambda i: (-scores[i], i)", "key=lambda i: (scores[i], i)"),
    ("tie_break_reversed", "key=lambda i: (-scores[i], i)", "key=lambda i: (-scores[i], -i)"),
    ("prev_block_wrong", "f.add((c - 1) >> (level - 1))", "f.add((c - 2) >> (level - 1))"),
    ("first_block_not_forced", "        f.add(0)\n", ""),
    ("keep_all_strict", "if len(cands) <= topk:", "if len(cands) < topk:"),
    ("forced_not_charged",
     "best, margin = top_by_score(rankable, scores, topk - len(forced))\n            kept = sorted(forced) + best",
     "best, margin = top_by_score(rankable, scores, topk)\n            kept = sorted(forced) + best"),
    ("bsa_forced_not_charged",
     "best, margin = top_by_score(rankable, scores, topk - len(forced))\n    return RowSelection(",
     "best, margin = top_by_score(rankable, scores, topk)\n    return RowSelection("),
    ("attention_mask_off_by_one", "if (not causal) or j <= t]\n    kk, vv = keys[cols], values[cols]\n    outs",
     "if (not causal) or j < t]\n    kk, vv = keys[cols], values[cols]\n    outs"),
    ("gqa_heads_averaged", "        total += reduce_logits(z, variant)\n    return total",
     "        total += reduce_logits(z, variant)\n    return total / len(q_heads)"),
    ("softmax_unnormalised", "outs.append((p @ vv) / p.sum())", "outs.append(p @ vv)"),
    ("pyramid_parent_uses_sum", ".mean(axis=0)\n                                for i in range(m)]))",
     ".sum(axis=0)\n                                for i in range(m)]))"),
    ("pisa2_sample_variance", "np.mean(z) + 0.5 * np.var(z)", "np.mean(z) + 0.5 * np.var(z, ddof=1)"),
    ("bsa_scale_dropped", "lambda i: float(sum(scale * (leaf_sum[i] @ q) for q in q_heads))",
     "lambda i: float(sum((leaf_sum[i] @ q) for q in q_heads))"),
    ("grad_delta_dropped", "dz = p * (vv @ g - g @ out)", "dz = p * (vv @ g)"),
    ("grad_dk_scale_dropped", "dk += scale * np.outer(dz, q)", "dk += np.outer(dz, q)"),
    ("grad_dq_uses_values", "dq[h] = scale * (dz @ kk)", "dq[h] = scale * (dz @ vv)"),
    ("grad_dv_heads_not_summed", "dv += np.outer(p, g)", "dv = np.outer(p, g)"),
    ("grad_mask_off_by_one", "if (not causal) or j <= t]\n\n\ndef attend_row_grad",
     "if (not causal) or j < t]\n\n\ndef attend_row_grad"),
    ("grad_block_rows_dropped", "rows = np.nonzero((np.asarray(idx_rows) == blk).any(axis=1))[0]",
     "rows = np.nonzero((np.asarray(idx_rows) == blk).any(axis=1))[0][1:]"),
    ("mean_mass_of_log_masses", "np.mean([math.exp(leaf_lse(q, i) - tot)",
     "np.mean([(leaf_lse(q, i) - tot)"),
    ("mean_mass_noncausal_total", "totals = [logsumexp(scale * (keys[:last + 1] @ q)) for q in q_heads]",
     "totals = [logsumexp(scale * (keys @ q)) for q in q_heads]"),
]

# Planted mistakes in the selection-quality diagnostics (oracle/metrics.py).
METRICS_MUTATIONS = [
    ("masses_heads_summed", "return out / len(q_heads)", "return out"),
    ("masses_total_over_block_only", "total = logsumexp(z)", "total = logsumexp(z[t // block * block:])"),
    ("retained_renormalised_over_selection", '"retained_mass": kept,',
     '"retained_mass": kept / sum(mass[i] for i in sel),'),
    ("net_recall_keeps_forced", "len((sel - forced) & (ref - forced)) / free",
     "len(sel & ref) / free"),
    ("recall_drops_forced", '"recall": len(sel & ref) / topk', '"recall": len((sel - forced) & (ref - forced)) / topk'),
    ("mass_ratio_inverted", '"mass_ratio": kept / kept_ref', '"mass_ratio": kept_ref / kept'),
]


def load_mutant(name, find, repl, src=SRC):
    text = open(src).read()
    assert text.count(find) == 1, f"mutation {name}: pattern occurs {text.count(find)} times"
    mutated = text.replace(find, repl)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    mod.__file__ = src
    mod.__package__ = "oracle"  # metrics.py imports from the real oracle package
    sys.modules[mod.__name__] = mod  # dataclasses look the module up by name
    try:
        exec(compile(mutated, f"<mutant {name}>", "exec"), mod.__dict__)
    finally:
        sys.modules.pop(mod.__name__, None)
    return mod


@pytest.mark.parametrize("name,find,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, find, repl):
    mutant = load_mutant(name, find, repl)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # AssertionError or a crash both count as caught
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
            break
    assert caught, f"no pin caught the planted mistake {name}"


@pytest.mark.parametrize("name,find,repl", METRICS_MUTATIONS, ids=[m[0] for m in METRICS_MUTATIONS])
def test_metrics_mutation_is_caught(name, find, repl):
    mutant = load_mutant(name, find, repl, METRICS_SRC)
    caught = []
    for pin in oracle_pins.METRIC_PINS:
        try:
            pin(mutant)
        except Exception as exc:
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
            break
    assert caught, f"no pin caught the planted mistake {name}"
