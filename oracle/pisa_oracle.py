"""Plain, slow CPU oracle of PISA's forward path and of the block-sparse
attention's backward (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``hierarchical_block_selection_amd``) never imports it, and this module imports
nothing from the product path: the two share no code.

What is followed
----------------
"PISA reading page" below is the section-by-section close reading titled
"论文精读 · Block Sparse Attention with Log-Linear Complexity (PISA)" (Paper
Reading Collection, attention-kv-cache/pisa).  Citations name its section and
equation.  Where the page is silent the reading taken is stated at the spot.

* Key pyramid: level sizes eq. (3), summaries eq. (4) (§4.1).
* Coarse-to-fine descent: eq. (5) and the bounds of eq. (6) (§4.2); the
  "keep every candidate when there are at most K of them" rule (§03).
* Node scores: LSE over child summaries, exact LSE over raw keys at the leaf
  level, eq. (7) (§4.3); first/second-order truncations eq. (9) (§4.3).
* GQA: a node's score is the sum of the scores of the query heads sharing the
  KV head, eq. (11) (§4.4).
* Forced blocks and causality (§5.3): the first, previous and current leaf and
  their ancestors are always kept; nodes on the current path are kept without
  being ranked; attention masks future tokens inside the current block.
* BSA baseline: eq. (1) block scores over mean-pooled leaf summaries + Top-K
  (§02, Table 1 row 5).
* Block-sparse attention: eq. (2) (§02), with the causal mask of §5.3.
* Its backward with the block lists held fixed (§5.3): the softmax chain rule
  written out per row.

Readings taken where the page leaves a step open:

R1  Ragged tails: eq. (4) is applied literally (mean of the children that
    exist); the leaf LSE runs over the keys that exist.
R2  Top-K ties: higher score first, equal scores -> lower node index first.
R3  The "at most K candidates -> keep all" test counts candidates after future
    nodes are dropped; forced nodes count.
R4  Forced blocks take slots of the K budget; the ancestors of all forced
    leaves are forced at every level.
R5  In causal mode the node containing the current leaf is always kept and
    never ranked, also without the first/previous forcing.
R6  Attention over the selected blocks keeps only keys j <= t in causal mode.
R7  BSA sums the per-head eq. (1) scores over a GQA group, like eq. (11).
R8  Non-causal mode: no forced nodes, every node eligible.
R9  Output leaf lists are ascending and padded with -1 to K.
R10 Decode: the new query sits at t = cache_len - 1; its own key is already in
    the cache and in the pyramid.
R11 Var(z) in eq. (9) is the population variance (1/m), as the cumulant
    expansion of eq. (8) implies.
R12 (eq. (15) of §5.1 lost its right-hand side) bears on the kernel design
    only; nothing here uses it.
R13 Backward (§5.3): the leaf lists are inputs, not functions of Q and K; the
    gradients are those of eq. (2) over the fixed token set, so nothing reaches
    the pyramid or the scores.  dK and dV of a key sum over every query head
    of the group and every row whose list holds the key's block.

Parity unpinned: outcomes at exact or near ties (several answers are then
correct); the ragged-tail reading R1 in non-causal mode has no worked example
on the page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Pyramid (PISA reading page §4.1, eqs. (3) and (4))
# --------------------------------------------------------------------------


def pyramid_level_sizes(n_tokens: int, block: int, branch: int = 2) -> list[int]:
    """Level sizes M_1..M_L of eq. (3): M_1 = ceil(N/C), M_{l+1} = ceil(M_l/g).

    The list stops at the first level holding a single node (the root).
    ``sizes[0]`` is M_1 (level 1 = leaf blocks).
    """
    if n_tokens < 1 or block < 1 or branch < 2:
        raise ValueError("need N >= 1, C >= 1, g >= 2")
    sizes = [-(-n_tokens // block)]
    while sizes[-1] > 1:
        sizes.append(-(-sizes[-1] // branch))
    return sizes


def build_pyramid(keys: np.ndarray, block: int, branch: int = 2) -> list[np.ndarray]:
    """Mean-pooled key summaries of eq. (4) for one KV head.

    keys: [N, d].  Returns ``levels`` with ``levels[l-1]`` the [M_l, d] summaries
    of level l.  Level 1 averages the C raw keys of each leaf block (g_0 = C);
    level l+1 averages the (up to g) existing level-l children (reading R1).
    """
    keys = np.asarray(keys, dtype=np.float64)
    n = keys.shape[0]
    sizes = pyramid_level_sizes(n, block, branch)
    level1 = np.stack([keys[i * block:min((i + 1) * block, n)].mean(axis=0)
                       for i in range(sizes[0])])
    levels = [level1]
    for m in sizes[1:]:
        below = levels[-1]
        levels.append(np.stack([below[branch * i:min(branch * i + branch, len(below))].mean(axis=0)
                                for i in range(m)]))
    return levels


def node_children(node: int, level: int, sizes: list[int], block: int, n_tokens: int,
                  branch: int = 2) -> list[int]:
    """Ch(i) of eq. (4)/(5): level-(l-1) nodes under node i of level l.

    For l = 1 the children are the raw token positions of the leaf block.
    Only children that exist are returned (reading R1).
    """
    if level == 1:
        return list(range(node * block, min((node + 1) * block, n_tokens)))
    below = sizes[level - 2]
    return [r for r in range(branch * node, branch * node + branch) if r < below]


# --------------------------------------------------------------------------
# Scores (PISA reading page §4.3 eqs. (7)-(9), §4.4 eq. (11))
# --------------------------------------------------------------------------


def logsumexp(z: np.ndarray) -> float:
    """log(sum(exp(z))) computed as m + log(sum(exp(z - m)))."""
    m = float(np.max(z))
    return m + math.log(float(np.sum(np.exp(z - m))))


def reduce_logits(z: np.ndarray, variant: str) -> float:
    """Eq. (7) for variant "lse"; the eq. (9) truncations "mean" (PISA-1) and
    "mean_var" (PISA-2, population variance, reading R11)."""
    if variant == "lse":
        return logsumexp(z)
    if variant == "mean":
        return float(np.mean(z))
    if variant == "mean_var":
        return float(np.mean(z) + 0.5 * np.var(z))
    raise ValueError(variant)


def node_score(q_heads: np.ndarray, node: int, level: int, levels: list[np.ndarray],
               keys: np.ndarray, block: int, scale: float, branch: int = 2,
               variant: str = "lse") -> float:
    """u_i of eq. (11): sum over the group's query heads of eq. (7)'s score.

    q_heads: [G, d].  At level 1 the children are the raw keys of the leaf
    (exact LSE); above, the children are the level-(l-1) summaries.
    """
    sizes = [len(x) for x in levels]
    ch = node_children(node, level, sizes, block, keys.shape[0], branch)
    child_vecs = keys[ch] if level == 1 else levels[level - 2][ch]
    total = 0.0
    for q in q_heads:
        z = scale * (child_vecs @ q)
        total += reduce_logits(z, variant)
    return total


# --------------------------------------------------------------------------
# Forced / eligible nodes (PISA reading page §5.3)
# --------------------------------------------------------------------------


def forced_nodes(t: int, level: int, block: int, causal: bool, force_first_prev: bool) -> set[int]:
    """Nodes of ``level`` that are kept without ranking for query t.

    Causal: the node holding the current leaf c = t // C (reading R5); with
    the forcing policy also the nodes holding leaf 0 and leaf c-1 (R4).
    A level-l node i holds leaves [i*2^(l-1), (i+1)*2^(l-1)), so the node
    holding leaf x is x >> (l-1).
    """
    if not causal:
        return set()
    c = t // block
    f = {c >> (level - 1)}
    if force_first_prev:
        f.add(0)
        if c >= 1:
            f.add((c - 1) >> (level - 1))
    return f


def last_eligible_node(t: int, level: int, block: int) -> int:
    """Largest level-l node index that holds no key strictly after the current leaf."""
    return (t // block) >> (level - 1)


def top_by_score(cands: list[int], scores: dict[int, float], keep: int) -> tuple[list[int], float]:
    """Top-``keep`` of ``cands`` by descending score, ties to the lower index (R2).

    Returns the kept nodes and the margin between the last kept score and the
    first dropped score (+inf when the choice does not depend on scores).
    """
    order = sorted(cands, key=lambda i: (-scores[i], i))
    if keep <= 0 or keep >= len(order):
        return order[:max(keep, 0)], math.inf
    return order[:keep], scores[order[keep - 1]] - scores[order[keep]]


# --------------------------------------------------------------------------
# PISA descent (PISA reading page §4.2 eqs. (5),(6); §03; §5.3)
# --------------------------------------------------------------------------


@dataclass
class LevelTrace:
    level: int
    candidates: list[int]          # A^(l) after dropping future nodes
    forced: list[int]              # F (subset of candidates)
    scored: bool                   # False when #A <= K (all kept)
    kept: list[int]                # I^(l)
    scores: dict[int, float] = field(default_factory=dict)
    margin: float = math.inf


@dataclass
class RowSelection:
    leaves: list[int]              # final I^(1), ascending
    scores: dict[int, float]       # leaf -> ranking score (ranked leaves only)
    unranked: set[int]             # leaves kept without ranking
    min_margin: float              # min margin over every scored level
    trace: list[LevelTrace]


def select_pisa_row(q_heads, keys, levels, t, block, topk, causal=True,
                    force_first_prev=True, scale=None, branch=2, variant="lse") -> RowSelection:
    """Coarse-to-fine Top-K descent for query position t of one KV group.

    q_heads: [G, d] queries of the group's heads at position t; keys: [N, d];
    levels: output of ``build_pyramid``.

    From the root (A^(L) = {root}), level by level (eq. 5): drop nodes that lie
    entirely in the future (causal), keep every candidate if there are at most
    K (§03), otherwise keep the forced nodes plus the best K - #F of the others
    by eq. (11)'s summed eq. (7) score; the kept nodes' children form the next
    candidate set.  At level 1 the kept leaves are the answer.
    """
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    d = keys.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    n_tok = keys.shape[0]
    sizes = [len(x) for x in levels]
    n_levels = len(levels)
    cands = [0]
    trace = []
    min_margin = math.inf
    leaf_scores: dict[int, float] = {}
    unranked: set[int] = set()
    for level in range(n_levels, 0, -1):
        if causal:
            limit = last_eligible_node(t, level, block)
            cands = [i for i in cands if i <= limit]
        forced = forced_nodes(t, level, block, causal, force_first_prev) & set(cands)
        rec = LevelTrace(level=level, candidates=list(cands), forced=sorted(forced),
                         scored=False, kept=[])
        if len(cands) <= topk:
            kept = list(cands)
            if level == 1:
                unranked |= set(kept)
        else:
            if len(forced) > topk:
                raise ValueError("more forced nodes than the budget K")
            rankable = [i for i in cands if i not in forced]
            scores = {i: node_score(q_heads, i, level, levels, keys, block, scale, branch, variant)
                      for i in rankable}
            best, margin = top_by_score(rankable, scores, topk - len(forced))
            kept = sorted(forced) + best
            rec.scored, rec.scores, rec.margin = True, scores, margin
            min_margin = min(min_margin, margin)
            if level == 1:
                unranked |= forced
                leaf_scores = {i: scores[i] for i in best}
        rec.kept = sorted(kept)
        trace.append(rec)
        if level > 1:
            cands = [ch for i in sorted(kept)
                     for ch in node_children(i, level, sizes, block, n_tok, branch)]
        else:
            cands = sorted(kept)
    return RowSelection(leaves=sorted(cands), scores=leaf_scores, unranked=unranked,
                        min_margin=min_margin, trace=trace)


# --------------------------------------------------------------------------
# Flat selectors: BSA (eq. 1) and the exhaustive exact-LSE reference
# --------------------------------------------------------------------------


def _flat_select(t, n_leaves, block, topk, causal, force_first_prev, score_fn):
    if causal:
        eligible = list(range(0, min(t // block, n_leaves - 1) + 1))
    else:
        eligible = list(range(n_leaves))
    forced = forced_nodes(t, 1, block, causal, force_first_prev) & set(eligible)
    if len(eligible) <= topk:
        return RowSelection(leaves=eligible, scores={}, unranked=set(eligible),
                            min_margin=math.inf, trace=[])
    rankable = [i for i in eligible if i not in forced]
    scores = {i: score_fn(i) for i in rankable}
    best, margin = top_by_score(rankable, scores, topk - len(forced))
    return RowSelection(leaves=sorted(set(best) | forced), scores={i: scores[i] for i in best},
                        unranked=set(forced), min_margin=margin, trace=[])


def select_bsa_row(q_heads, levels, t, block, topk, causal=True, force_first_prev=True,
                   scale=None) -> RowSelection:
    """BSA: s_{t,i} = q_t . kbar_i / sqrt(d) over the leaf summaries (eq. 1), summed
    over the group's heads (reading R7), then forced blocks + Top-(K - #F).

    Uses the same forcing, causal and keep-all rules as the PISA descent.
    """
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    leaf_sum = levels[0]
    scale = 1.0 / math.sqrt(leaf_sum.shape[1]) if scale is None else scale
    return _flat_select(t, len(leaf_sum), block, topk, causal, force_first_prev,
                        lambda i: float(sum(scale * (leaf_sum[i] @ q) for q in q_heads)))


def select_exhaustive_row(q_heads, keys, t, block, topk, causal=True, force_first_prev=True,
                          scale=None, rule="sum_lse") -> RowSelection:
    """Flat selection scored by the exact leaf LSE over raw keys.

    rule "sum_lse": sum over heads of the exact leaf LSE (what PISA's leaf level
    computes, eq. (7) at l = 1 with eq. (11)).  rule "mean_mass": mean over heads
    of the block's share of full causal attention mass (the diagnostic reference
    the page describes in §4.4 for GQA); for one head both rank identically.
    """
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    n_tok, d = keys.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    n_leaves = -(-n_tok // block)
    last = t if causal else n_tok - 1

    def leaf_lse(q, i):
        return logsumexp(scale * (keys[i * block:min((i + 1) * block, n_tok)] @ q))

    if rule == "sum_lse":
        fn = lambda i: float(sum(leaf_lse(q, i) for q in q_heads))
    elif rule == "mean_mass":
        totals = [logsumexp(scale * (keys[:last + 1] @ q)) for q in q_heads]
        fn = lambda i: float(np.mean([math.exp(leaf_lse(q, i) - tot)
                                      for q, tot in zip(q_heads, totals)]))
    else:
        raise ValueError(rule)
    return _flat_select(t, n_leaves, block, topk, causal, force_first_prev, fn)


# --------------------------------------------------------------------------
# Block-sparse attention (PISA reading page §02 eq. (2); mask of §5.3)
# --------------------------------------------------------------------------


def attend_row(q_heads, keys, values, leaves, t, block, causal=True, scale=None):
    """Eq. (2) for each query head of the group at position t.

    The token set is the union of the selected leaf blocks, restricted to
    j <= t in causal mode (reading R6).  Returns (out [G, d], lse [G]) where
    lse is the natural-log normaliser log sum_j exp(scale q.k_j).
    """
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n_tok, d = keys.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cols = [j for i in sorted(x for x in leaves if x >= 0)
            for j in range(i * block, min((i + 1) * block, n_tok))
            if (not causal) or j <= t]
    kk, vv = keys[cols], values[cols]
    outs, lses = [], []
    for q in q_heads:
        z = scale * (kk @ q)
        m = float(np.max(z))
        p = np.exp(z - m)
        outs.append((p @ vv) / p.sum())
        lses.append(m + math.log(float(p.sum())))
    return np.stack(outs), np.array(lses)


# --------------------------------------------------------------------------
# Backward of the block-sparse attention (PISA reading page §5.3 "backward":
# the selected block indices are held fixed and gradients flow only through
# the attention entries they select; the forward is eq. (2) of §02)
# --------------------------------------------------------------------------


def attended_tokens(leaves, t, block, n_tok, causal=True):
    """Token positions attend_row uses for position t: the union of the listed
    leaf blocks (entries < 0 skipped, in list order sorted ascending), clipped
    to the sequence and to j <= t in causal mode (reading R6)."""
    return [j for i in sorted(x for x in leaves if x >= 0)
            for j in range(i * block, min((i + 1) * block, n_tok))
            if (not causal) or j <= t]


def attend_row_grad(q_heads, keys, values, leaves, t, block, dout, causal=True, scale=None):
    """Gradient of sum_h dout[h] . out[h] for the rows of attend_row at t.

    The token set J is fixed (reading R13).  Per head, with z_j = scale q.k_j,
    p = softmax(z) over J and out = sum_j p_j v_j, the chain rule through the
    softmax gives
        dv_j = p_j dout,
        dz_j = p_j (dout . v_j - dout . out),
        dq   = scale sum_j dz_j k_j,
        dk_j = scale dz_j q.
    Returns (cols, dq [G, d], dk [len(cols), d], dv [len(cols), d]); dk and dv
    are summed over the group's heads, which read the same keys and values.
    A row with no token gets zero gradients.
    """
    q_heads = np.atleast_2d(np.asarray(q_heads, dtype=np.float64))
    dout = np.atleast_2d(np.asarray(dout, dtype=np.float64))
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    n_tok, d = keys.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    cols = attended_tokens(leaves, t, block, n_tok, causal)
    dq = np.zeros_like(q_heads)
    dk = np.zeros((len(cols), d))
    dv = np.zeros((len(cols), d))
    if not cols:
        return cols, dq, dk, dv
    kk, vv = keys[cols], values[cols]
    for h, (q, g) in enumerate(zip(q_heads, dout)):
        z = scale * (kk @ q)
        p = np.exp(z - np.max(z))
        p /= p.sum()
        out = p @ vv
        dz = p * (vv @ g - g @ out)
        dq[h] = scale * (dz @ kk)
        dk += scale * np.outer(dz, q)
        dv += np.outer(p, g)
    return cols, dq, dk, dv


def attention_backward(q_group, keys, values, idx_rows, dout_group, block, causal=True,
                       scale=None):
    """Whole-head backward for one (batch, KV head) by summing attend_row_grad
    over every row.  q_group, dout_group: [G, N, d]; keys, values: [N, d];
    idx_rows: [N, K] leaf lists (entries < 0 or beyond the last block skipped).
    Returns dq [G, N, d], dk [N, d], dv [N, d]."""
    q_group = np.asarray(q_group, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    n_tok = keys.shape[0]
    dq = np.zeros_like(q_group)
    dk = np.zeros_like(keys)
    dv = np.zeros_like(keys)
    for t in range(n_tok):
        cols, gq, gk, gv = attend_row_grad(q_group[:, t], keys, values, idx_rows[t], t, block,
                                           np.asarray(dout_group)[:, t], causal, scale)
        dq[:, t] = gq
        if cols:
            np.add.at(dk, cols, gk)
            np.add.at(dv, cols, gv)
    return dq, dk, dv


def key_block_grad(q_group, keys, values, idx_rows, dout_group, blk, block, causal=True,
                   scale=None):
    """dk, dv of the keys of leaf block ``blk`` alone: the contributions of the
    rows whose list holds ``blk``, computed row by row.  Returns two
    [n_keys, d] arrays (n_keys = keys of the block inside the sequence)."""
    keys = np.asarray(keys, dtype=np.float64)
    n_tok, d = keys.shape
    lo, hi = blk * block, min((blk + 1) * block, n_tok)
    dk = np.zeros((hi - lo, d))
    dv = np.zeros((hi - lo, d))
    rows = np.nonzero((np.asarray(idx_rows) == blk).any(axis=1))[0]
    for t in rows:
        cols, _, gk, gv = attend_row_grad(np.asarray(q_group)[:, t], keys, values, idx_rows[t],
                                          int(t), block, np.asarray(dout_group)[:, t], causal,
                                          scale)
        for c, j in enumerate(cols):
            if lo <= j < hi:
                dk[j - lo] += gk[c]
                dv[j - lo] += gv[c]
    return dk, dv


# --------------------------------------------------------------------------
# Decode step (PISA reading page §5.1 "decode uses one fused stage", §5.3 cache)
# --------------------------------------------------------------------------


def decode_row(q_heads, k_cache, v_cache, cache_len, block, topk, causal=True,
               force_first_prev=True, scale=None, branch=2, variant="lse"):
    """One decode step for one (sequence, KV head): the new query at
    t = cache_len - 1 (reading R10) selects over the pyramid of the first
    cache_len keys and attends to the selected blocks.

    Returns (RowSelection, out [G, d], lse [G]).
    """
    n = int(cache_len)
    keys = np.asarray(k_cache, dtype=np.float64)[:n]
    vals = np.asarray(v_cache, dtype=np.float64)[:n]
    levels = build_pyramid(keys, block, branch)
    sel = select_pisa_row(q_heads, keys, levels, n - 1, block, topk, causal,
                          force_first_prev, scale, branch, variant)
    out, lse = attend_row(q_heads, keys, vals, sel.leaves, n - 1, block, causal, scale)
    return sel, out, lse


# --------------------------------------------------------------------------
# Convenience: whole-head drivers and padding (reading R9)
# --------------------------------------------------------------------------


def padded(leaves: list[int], topk: int) -> list[int]:
    """Ascending leaf list padded with -1 to K entries."""
    out = sorted(leaves)
    if len(out) > topk:
        raise ValueError("more than K leaves")
    return out + [-1] * (topk - len(out))


def select_rows(kind, q_group, keys, levels, rows, block, topk, causal=True,
                force_first_prev=True, scale=None):
    """Run a selector over several rows of one KV group.

    q_group: [G, N, d].  kind: "pisa" | "bsa" | "exhaustive".
    Returns a list of RowSelection, one per row.
    """
    out = []
    for t in rows:
        qh = q_group[:, t, :]
        if kind == "pisa":
            out.append(select_pisa_row(qh, keys, levels, t, block, topk, causal,
                                       force_first_prev, scale))
        elif kind == "bsa":
            out.append(select_bsa_row(qh, levels, t, block, topk, causal, force_first_prev, scale))
        elif kind == "exhaustive":
            out.append(select_exhaustive_row(qh, keys, t, block, topk, causal,
                                             force_first_prev, scale))
        else:
            raise ValueError(kind)
    return out
