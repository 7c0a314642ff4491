"""Pins that tie the CPU oracle to facts fixed by the PISA pages and by mathematics.

Each ``pin_*`` takes the oracle module as its argument and raises
AssertionError when the oracle disagrees.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle
with planted mistakes and checks that every mistake is caught.

Independent routes used here (none of them calls the oracle's own scoring):
  * values the pages print (the §5.2 tower tables under tests/golden/);
  * closed forms (means of raw-key spans, the eq. (8) cumulant expansion);
  * library special cases (scipy's logsumexp, torch's dense causal SDPA, a
    NumPy GEMM plus a lexsort for BSA);
  * a dense brute force on tiny inputs (S = scale Q K^T, node logits as block
    means of S, descent by boolean masks);
  * invariants (eq. (6) bounds, eq. (10) sandwich, GQA duplication, causality);
  * for the backward: central differences of a dense masked attention written
    here, torch autograd of the same, and softmax invariants.
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def read_tower(name):
    rows, extras = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line:
                continue
            if line.startswith("#"):
                parts = line[1:].split()
                if len(parts) == 2 and parts[1].isdigit():
                    extras[parts[0]] = int(parts[1])
                continue
            rows.append(tuple(int(x) for x in line.split()))
    return rows, extras


# ---------------------------------------------------------------- P1 towers
def pin_tower_tables(O):
    """§5.2's two tower tables: level count, tokens per block, candidate counts,
    scored flags, leaf raw keys scored and kept leaves, for one (non-causal) query."""
    for name, n, k in (("tower_pretrain_n4096_c64_k8.txt", 4096, 8),
                       ("tower_cpt_n16384_c64_k32.txt", 16384, 32)):
        rows, extras = read_tower(name)
        c, d = 64, 8
        r = rng(n)
        keys = r.standard_normal((n, d))
        q = r.standard_normal((1, d))
        levels = O.build_pyramid(keys, c)
        assert len(levels) == len(rows), (name, len(levels))
        sel = O.select_pisa_row(q, keys, levels, n - 1, c, k, causal=False,
                                force_first_prev=False)
        by_level = {tr.level: tr for tr in sel.trace}
        for level, tokens, cands, scored in rows:
            assert c * 2 ** (level - 1) == tokens
            tr = by_level[level]
            assert len(tr.candidates) == cands, (name, level, len(tr.candidates))
            assert tr.scored == bool(scored), (name, level)
        leaf = by_level[1]
        assert len(leaf.scores) * c == extras["leaf_raw_keys_scored"]
        assert len(sel.leaves) == extras["kept_leaves"]
    # c1's shape from the workloads: 32 leaf blocks, 6 levels.
    assert O.pyramid_level_sizes(2048, 64) == [32, 16, 8, 4, 2, 1]


# ---------------------------------------------------------------- P2 bounds
def pin_eq6_bounds(O):
    """#I^(l) <= K and #A^(l-1) <= g #I^(l) <= gK at every level and row (eq. 6)."""
    r = rng(2)
    n, c, d = 1024, 16, 8
    keys = r.standard_normal((n, d))
    qs = r.standard_normal((n, 2, d))
    levels = O.build_pyramid(keys, c)
    for k in (2, 3, 5):
        for causal, force in ((False, False), (True, False), (True, True)):
            if force and k < 3:
                continue
            for t in range(0, n, 37):
                sel = O.select_pisa_row(qs[t], keys, levels, t, c, k, causal, force)
                tr = sel.trace
                for i, rec in enumerate(tr):
                    assert len(rec.kept) <= k
                    if i + 1 < len(tr):
                        assert len(tr[i + 1].candidates) <= 2 * len(rec.kept) <= 2 * k
                eligible = (t // c + 1) if causal else n // c
                assert len(sel.leaves) == min(k, eligible)


# ---------------------------------------------------------------- P3 pyramid
def pin_pyramid_closed_form(O):
    """With equal groups every summary is the mean of the raw keys in its span
    (§4.1); with ragged tails eq. (4) averages the existing children (reading R1)."""
    r = rng(3)
    for n, c in ((1024, 16), (2048, 64), (512, 8)):
        keys = r.standard_normal((n, 5))
        levels = O.build_pyramid(keys, c)
        for level, summ in enumerate(levels, start=1):
            span = c * 2 ** (level - 1)
            assert summ.shape == (max(n // span, 1), 5)
            for i in range(summ.shape[0]):
                ref = keys[i * span:(i + 1) * span].mean(axis=0)
                assert np.max(np.abs(summ[i] - ref)) <= 1e-12
    # ragged: N = 5C + 3 -> leaves of sizes C,C,C,C,C,3; levels 6,3,2,1
    c = 4
    keys = r.standard_normal((5 * c + 3, 3))
    lv = O.build_pyramid(keys, c)
    assert [len(x) for x in lv] == [6, 3, 2, 1]
    leaf = [keys[i * c:min((i + 1) * c, len(keys))].mean(axis=0) for i in range(6)]
    l2 = [(leaf[0] + leaf[1]) / 2, (leaf[2] + leaf[3]) / 2, (leaf[4] + leaf[5]) / 2]
    l3 = [(l2[0] + l2[1]) / 2, l2[2]]
    l4 = [(l3[0] + l3[1]) / 2]
    for got, want in zip(lv, (leaf, l2, l3, l4)):
        assert np.max(np.abs(np.asarray(got) - np.asarray(want))) <= 1e-12


# ---------------------------------------------------------------- P4 leaf LSE
def pin_leaf_lse_is_logsumexp(O):
    """At level 1, eq. (7) is the exact LSE of the C scaled raw logits."""
    r = rng(4)
    n, c, d = 256, 16, 8
    keys = r.standard_normal((n, d)) * 2
    q = r.standard_normal((2, d))
    levels = O.build_pyramid(keys, c)
    scale = 0.37
    for leaf in (0, 3, 15):
        got = O.node_score(q, leaf, 1, levels, keys, c, scale)
        want = sum(scipy.special.logsumexp(scale * (keys[leaf * c:(leaf + 1) * c] @ qq)) for qq in q)
        assert abs(got - want) <= 1e-12
    # and the descent's recorded leaf scores are these values
    sel = O.select_pisa_row(q, keys, levels, n - 1, c, 5, causal=True, force_first_prev=True,
                            scale=scale)
    assert sel.scores
    for leaf, s in sel.scores.items():
        want = sum(scipy.special.logsumexp(scale * (keys[leaf * c:(leaf + 1) * c] @ qq)) for qq in q)
        assert abs(s - want) <= 1e-12


# ---------------------------------------------------------------- P5 Jensen
def pin_jensen_sandwich(O):
    """Eq. (10): mean of child logits <= score - log g <= log-mean-exp over the raw
    keys of the node; equality on the right when each child's keys are constant."""
    r = rng(5)
    n, c, d = 512, 8, 6
    keys = r.standard_normal((n, d))
    q = r.standard_normal(d)
    levels = O.build_pyramid(keys, c)
    scale = 1 / math.sqrt(d)
    for level in range(2, len(levels) + 1):
        span = c * 2 ** (level - 1)
        for i in range(len(levels[level - 1])):
            u = O.node_score(q[None], i, level, levels, keys, c, scale)
            ch = levels[level - 2][2 * i:2 * i + 2]
            m = scale * (ch @ q)
            raw = scale * (keys[i * span:(i + 1) * span] @ q)
            right = scipy.special.logsumexp(raw) - math.log(len(raw))
            assert m.mean() <= u - math.log(2) + 1e-12
            assert u - math.log(2) <= right + 1e-12
    # equality case: every raw key of a child equals that child's summary
    keys2 = np.repeat(r.standard_normal((n // c, d)), c, axis=0)
    lv2 = O.build_pyramid(keys2, c)
    u = O.node_score(q[None], 0, 2, lv2, keys2, c, scale)
    raw = scale * (keys2[:2 * c] @ q)
    assert abs((u - math.log(2)) - (scipy.special.logsumexp(raw) - math.log(2 * c))) <= 1e-12


# ---------------------------------------------------------------- P6 Taylor
def pin_taylor_expansion(O):
    """Eq. (8): LSE(z) = log m + mean + Var/2 + O(eps^3); the eps^3 term is the
    third central moment / 6.  Checks the "lse", "mean" and "mean_var" reductions."""
    r = rng(6)
    w = r.standard_normal(64) + r.standard_normal(64) ** 2
    wc = w - w.mean()
    k3 = float(np.mean(wc ** 3))
    for eps in (1e-2, 5e-3, 2.5e-3):
        z = eps * w
        lse = O.reduce_logits(z, "lse")
        pisa1 = O.reduce_logits(z, "mean")
        pisa2 = O.reduce_logits(z, "mean_var")
        assert abs(pisa1 - eps * w.mean()) <= 1e-15
        resid = lse - math.log(64) - pisa2
        assert abs(resid - eps ** 3 * k3 / 6) <= 2 * eps ** 4 * float(np.mean(wc ** 4)), (eps, resid)
        assert abs(pisa2 - pisa1 - 0.5 * eps ** 2 * float(np.mean(wc ** 2))) <= 1e-15


# ---------------------------------------------------------------- P7 no pruning
def pin_no_pruning_equals_exhaustive(O):
    """K >= M_2: no intermediate level prunes, so PISA = the flat exact-LSE Top-K.
    K >= M_1: every eligible block is kept."""
    r = rng(7)
    n, c, d = 2048, 64, 16
    keys = r.standard_normal((n, d))
    qs = r.standard_normal((n, 1, d))
    levels = O.build_pyramid(keys, c)
    compared = total = 0
    for k in (16, 32):
        for causal, force in ((True, True), (False, False)):
            for t in range(0, n, 97):
                a = O.select_pisa_row(qs[t], keys, levels, t, c, k, causal, force)
                b = O.select_exhaustive_row(qs[t], keys, t, c, k, causal, force)
                total += 1
                if min(a.min_margin, b.min_margin) > 1e-9:
                    compared += 1
                    assert a.leaves == b.leaves, (k, t)
                if k == 32:
                    assert a.leaves == list(range((t // c + 1) if causal else n // c))
    assert compared >= 0.9 * total


# ---------------------------------------------------------------- P8 dense attention
def pin_dense_attention_recovered(O):
    """K*C >= N: every block is selected and eq. (2) with the causal mask is dense
    causal softmax attention (torch SDPA in float64 on the CPU)."""
    r = rng(8)
    n, c, d, k = 256, 16, 8, 16
    q = r.standard_normal((2, n, d))
    keys = r.standard_normal((n, d))
    vals = r.standard_normal((n, d))
    levels = O.build_pyramid(keys, c)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(keys)[None, None].expand(1, 2, n, d),
        torch.from_numpy(vals)[None, None].expand(1, 2, n, d), is_causal=True)[0].numpy()
    for t in range(0, n, 7):
        sel = O.select_pisa_row(q[:, t], keys, levels, t, c, k, True, True)
        out, lse = O.attend_row(q[:, t], keys, vals, sel.leaves, t, c, True)
        assert np.max(np.abs(out - ref[:, t])) <= 1e-12
        z = (q[:, t] @ keys[:t + 1].T) / math.sqrt(d)
        assert np.max(np.abs(lse - scipy.special.logsumexp(z, axis=1))) <= 1e-12


# ---------------------------------------------------------------- P9 brute force
def brute_force_selection(s_row, n, c, k, t, causal, force):
    """Dense route: s_row [G, N] = scale q_h . k_j for every key.  Node logits are
    block means of s_row over each node's raw span (q . mean k = mean q . k),
    node scores are scipy logsumexp over child logits summed over heads, and the
    descent runs on boolean masks with np.lexsort.  Needs N = C * 2^m."""
    m1 = n // c
    n_levels = int(math.log2(m1)) + 1
    cur = t // c

    def logit(level, r_):
        span = c * 2 ** (level - 1)
        return s_row[:, r_ * span:(r_ + 1) * span].mean(axis=1)

    alive = np.array([True])
    scores_out = {}
    for level in range(n_levels, 0, -1):
        cand = np.flatnonzero(alive)
        if causal:
            cand = cand[cand <= cur >> (level - 1)]
        forced = set()
        if causal:
            forced = {cur >> (level - 1)}
            if force:
                forced |= {0}
                if cur >= 1:
                    forced |= {(cur - 1) >> (level - 1)}
        if len(cand) <= k:
            keep = cand
        else:
            rank = np.array([x for x in cand if x not in forced])
            if level == 1:
                sc = np.array([scipy.special.logsumexp(s_row[:, x * c:(x + 1) * c], axis=1).sum()
                               for x in rank])
            else:
                sc = np.array([scipy.special.logsumexp(
                    np.stack([logit(level - 1, 2 * x), logit(level - 1, 2 * x + 1)]), axis=0).sum()
                    for x in rank])
            order = np.lexsort((rank, -sc))[:k - len(forced & set(cand.tolist()))]
            keep = np.union1d(rank[order], np.array(sorted(forced & set(cand.tolist())), dtype=int))
            if level == 1:
                scores_out = {int(rank[o]): float(sc[o]) for o in order}
        if level > 1:
            nxt = np.zeros(m1 >> (level - 2), dtype=bool)
            for x in keep:
                nxt[2 * x] = True
                nxt[2 * x + 1] = True
            alive = nxt
        else:
            return sorted(int(x) for x in keep), scores_out


def pin_brute_force_tiny(O):
    """Tiny N, C in {8, 16}, K in 2..5, causal with/without forcing and non-causal:
    the oracle's leaf sets equal the dense brute force (near-ties excluded) and its
    leaf scores agree to 1e-12."""
    r = rng(9)
    for n, c in ((256, 8), (512, 16), (128, 8)):
        d, g = 6, 2
        keys = r.standard_normal((n, d))
        qs = r.standard_normal((g, n, d))
        scale = 1 / math.sqrt(d)
        dense = scale * np.einsum("gnd,md->gnm", qs, keys)
        levels = O.build_pyramid(keys, c)
        compared = total = 0
        for k in (2, 3, 4, 5):
            for causal, force in ((True, True), (True, False), (False, False)):
                if force and k < 3:
                    continue
                for t in range(0, n, 11):
                    sel = O.select_pisa_row(qs[:, t], keys, levels, t, c, k, causal, force)
                    want, want_scores = brute_force_selection(dense[:, t], n, c, k, t, causal, force)
                    total += 1
                    if sel.min_margin <= 1e-9:
                        continue
                    compared += 1
                    assert sel.leaves == want, (n, c, k, causal, force, t)
                    assert set(sel.scores) == set(want_scores)
                    for x, s in sel.scores.items():
                        assert abs(s - want_scores[x]) <= 1e-12
        assert compared >= 0.9 * total


# ---------------------------------------------------------------- P10 BSA
def pin_bsa_is_gemm_topk(O):
    """BSA scores are Q K1bar^T * scale (a NumPy GEMM); the Top-K is a lexsort
    (score descending, index ascending) after the forced blocks take their slots."""
    r = rng(10)
    n, c, d, k = 1024, 16, 8, 5
    keys = r.standard_normal((n, d))
    qs = r.standard_normal((n, d))
    scale = 0.29
    levels = O.build_pyramid(keys, c)
    kbar = np.stack([keys[i * c:(i + 1) * c].mean(axis=0) for i in range(n // c)])
    s = (qs @ kbar.T) * scale
    compared = total = 0
    for t in range(0, n, 13):
        cur = t // c
        sel = O.select_bsa_row(qs[t][None], levels, t, c, k, True, True, scale=scale)
        forced = {cur, 0} | ({cur - 1} if cur >= 1 else set())
        elig = np.arange(cur + 1)
        if len(elig) <= k:
            assert sel.leaves == list(elig)
            continue
        rank = np.array([x for x in elig if x not in forced])
        order = np.lexsort((rank, -s[t, rank]))[:k - len(forced)]
        want = sorted(set(rank[order].tolist()) | forced)
        total += 1
        if sel.min_margin > 1e-9:
            compared += 1
            assert sel.leaves == want, t
            for x, v in sel.scores.items():
                assert abs(v - s[t, x]) <= 1e-12
    assert compared >= 0.9 * total


# ---------------------------------------------------------------- P11 GQA duplication
def pin_gqa_duplication(O):
    """Eq. (11): G copies of one query give G times the node scores and the same
    leaf set as the single head."""
    r = rng(11)
    n, c, d, k = 1024, 16, 8, 4
    keys = r.standard_normal((n, d))
    qs = r.standard_normal((n, d))
    levels = O.build_pyramid(keys, c)
    for t in range(0, n, 29):
        one = O.select_pisa_row(qs[t][None], keys, levels, t, c, k, True, True)
        four = O.select_pisa_row(np.stack([qs[t]] * 4), keys, levels, t, c, k, True, True)
        assert one.leaves == four.leaves
        for x in one.scores:
            assert abs(four.scores[x] - 4 * one.scores[x]) <= 1e-11


# ---------------------------------------------------------------- P12 causality / decode
def pin_causality_and_decode(O):
    """Row t depends on no key or value after t (current path unranked, mask of §5.3),
    so a decode step at cache length n equals prefill row n-1."""
    r = rng(12)
    n, c, d, k = 1024, 16, 8, 4
    keys = r.standard_normal((n, d))
    vals = r.standard_normal((n, d))
    qs = r.standard_normal((n, 2, d))
    levels = O.build_pyramid(keys, c)
    for t in (0, 5, 15, 16, 100, 333, 511, 700, 1023):
        sel = O.select_pisa_row(qs[t], keys, levels, t, c, k, True, True)
        out, lse = O.attend_row(qs[t], keys, vals, sel.leaves, t, c, True)
        k2, v2 = keys.copy(), vals.copy()
        k2[t + 1:] = r.standard_normal(k2[t + 1:].shape) * 3
        v2[t + 1:] = r.standard_normal(v2[t + 1:].shape) * 3
        lv2 = O.build_pyramid(k2, c)
        sel2 = O.select_pisa_row(qs[t], k2, lv2, t, c, k, True, True)
        assert sel2.leaves == sel.leaves
        out2, lse2 = O.attend_row(qs[t], k2, v2, sel2.leaves, t, c, True)
        assert np.max(np.abs(out2 - out)) <= 1e-12 and np.max(np.abs(lse2 - lse)) <= 1e-12
        dsel, dout, dlse = O.decode_row(qs[t], keys, vals, t + 1, c, k)
        assert dsel.leaves == sel.leaves
        assert np.max(np.abs(dout - out)) <= 1e-12


# ---------------------------------------------------------------- P13 worked causal example
def pin_worked_causal_example(O):
    """Hand-derived from §5.3's rules on the N=2048, C=64 shape (32 leaves, 6 levels),
    query t=1000 (current leaf 15), K=4, forcing on:
      l6 {0}; l5 node 1 is future -> {0}; l4 {0,1} kept (<= K); l3 {0..3} kept;
      l2 {0..7}: forced {0,7}, ranks {1..6}, keeps 2;
      l1: forced {0,14,15}, five rankable children, keeps 1;
    attention sees leaf 15 only up to token 1000."""
    r = rng(13)
    n, c, d = 2048, 64, 8
    keys = r.standard_normal((n, d))
    vals = r.standard_normal((n, d))
    q = r.standard_normal((1, d))
    levels = O.build_pyramid(keys, c)
    sel = O.select_pisa_row(q, keys, levels, 1000, c, 4, True, True)
    tr = {x.level: x for x in sel.trace}
    assert tr[6].candidates == [0] and not tr[6].scored
    assert tr[5].candidates == [0] and not tr[5].scored
    assert tr[4].candidates == [0, 1] and not tr[4].scored
    assert tr[3].candidates == [0, 1, 2, 3] and not tr[3].scored
    assert tr[2].candidates == list(range(8)) and tr[2].scored
    assert tr[2].forced == [0, 7] and sorted(tr[2].scores) == [1, 2, 3, 4, 5, 6]
    a, b = sorted(set(tr[2].kept) - {0, 7})
    assert sorted(tr[1].candidates) == sorted([0, 1, 14, 15, 2 * a, 2 * a + 1, 2 * b, 2 * b + 1])
    assert tr[1].forced == [0, 14, 15] and len(tr[1].scores) == 5
    assert len(sel.leaves) == 4 and {0, 14, 15} <= set(sel.leaves)
    out, _ = O.attend_row(q, keys, vals, [15], 1000, c, True)
    z = (keys[960:1001] @ q[0]) / math.sqrt(d)
    p = np.exp(z - z.max())
    assert np.max(np.abs(out[0] - (p @ vals[960:1001]) / p.sum())) <= 1e-12


# ---------------------------------------------------------------- tie rule (reading R2)
def pin_tie_rule(O):
    """Exact ties: duplicated leaf blocks give bit-identical scores; the lower
    block index wins, for PISA's leaf level, BSA and the exhaustive reference."""
    r = rng(14)
    n, c, d = 512, 16, 4
    base = r.standard_normal((c, d))
    keys = r.standard_normal((n, d)) * 0.01
    # leaves 5 and 9 hold the same strong keys; only one free slot remains
    for leaf in (5, 9):
        keys[leaf * c:(leaf + 1) * c] = base
    q = base.mean(axis=0)[None] * 4
    levels = O.build_pyramid(keys, c)
    t = 30 * c + 3
    # K=4: forced {0, 29, 30} + one free slot, which must go to leaf 5, not 9
    bsa = O.select_bsa_row(q, levels, t, c, 4, True, True)
    assert bsa.leaves == [0, 5, 29, 30], bsa.leaves
    ex = O.select_exhaustive_row(q, keys, t, c, 4, True, True)
    assert ex.leaves == [0, 5, 29, 30], ex.leaves
    # PISA with K >= M_2 reaches the leaf level unpruned and breaks the tie the same way
    sel = O.select_pisa_row(q, keys, levels, t, c, 16, True, True)
    assert 5 in sel.leaves
    small = O.select_pisa_row(q, keys, levels, t, c, 4, True, True)
    assert small.leaves[1] in (5, 9)
    ts = O.top_by_score([9, 5, 7], {9: 1.0, 5: 1.0, 7: 0.5}, 1)
    assert ts[0] == [5] and ts[1] == 0.0


# ---------------------------------------------------------------- P15 backward
def random_lists(r, n, c, k, causal, junk=False):
    """Leaf lists of K entries per row: the forced blocks {0, c-1, c} (causal)
    plus distinct random others, -1 padded; with junk, also out-of-range
    entries and, in causal mode, a future block."""
    m1 = -(-n // c)
    out = np.full((n, k), -1, np.int64)
    for t in range(n):
        cur = t // c
        hi = cur if causal else m1 - 1
        base = sorted({0, max(cur - 1, 0), cur}) if causal else []
        rest = [int(x) for x in r.permutation(hi + 1) if int(x) not in base]
        row = (base + rest)[:k - (1 if junk else 0)]
        if junk:
            row.append(int(r.choice([-1, m1, m1 + 3] + ([cur + 1] if causal and cur + 1 < m1 else []))))
        out[t, :len(row)] = row
    return out


def dense_mask(lists, n, c, causal):
    """mask[t, j]: token j is attended by row t (its block is listed and, in
    causal mode, j <= t), built without the oracle."""
    mask = np.zeros((n, n), bool)
    blk = np.arange(n) // c
    for t in range(n):
        listed = [x for x in lists[t] if 0 <= x]
        mask[t] = np.isin(blk, listed)
        if causal:
            mask[t, t + 1:] = False
    return mask


def dense_loss_np(q, keys, vals, dout, mask, scale):
    """sum over heads and rows of dout . out for masked dense attention (rows
    with no token contribute nothing)."""
    total = 0.0
    for h in range(q.shape[0]):
        s = scale * q[h] @ keys.T
        s = np.where(mask, s, -np.inf)
        for t in range(q.shape[1]):
            if not mask[t].any():
                continue
            p = np.exp(s[t] - s[t].max())
            p /= p.sum()
            total += float(dout[h, t] @ (p @ vals))
    return total


def pin_attention_grad_finite_differences(O):
    """The backward is the derivative of the forward: central differences of a
    dense masked softmax attention written here (fp64, step 1e-6) against
    every entry of dq, dk and dv, causal and not, with junk list entries."""
    r = rng(21)
    n, c, d, k, g = 22, 4, 5, 3, 2
    for causal in (True, False):
        q = r.standard_normal((g, n, d))
        keys = r.standard_normal((n, d))
        vals = r.standard_normal((n, d))
        dout = r.standard_normal((g, n, d))
        lists = random_lists(r, n, c, k, causal, junk=True)
        scale = 0.7
        mask = dense_mask(lists, n, c, causal)
        dq, dk, dv = O.attention_backward(q, keys, vals, lists, dout, c, causal, scale)
        eps = 1e-6
        for name, arr, grad in (("q", q, dq), ("k", keys, dk), ("v", vals, dv)):
            num = np.zeros_like(arr)
            for ix in np.ndindex(arr.shape):
                old = arr[ix]
                arr[ix] = old + eps
                up = dense_loss_np(q, keys, vals, dout, mask, scale)
                arr[ix] = old - eps
                dn = dense_loss_np(q, keys, vals, dout, mask, scale)
                arr[ix] = old
                num[ix] = (up - dn) / (2 * eps)
            err = np.max(np.abs(num - grad))
            assert err <= 1e-6 * (1 + np.max(np.abs(num))), (name, causal, err)


def pin_attention_grad_autograd(O):
    """torch autograd (float64, CPU) of dense attention masked by the lists,
    with GQA heads sharing K/V, rows without tokens included (zero gradient)."""
    r = rng(22)
    n, c, d, k, g = 160, 16, 8, 4, 4
    for causal in (True, False):
        lists = random_lists(r, n, c, k, causal, junk=True)
        if not causal:
            lists[5] = -1  # a row with nothing to attend
        mask = torch.from_numpy(dense_mask(lists, n, c, causal))
        q = torch.from_numpy(r.standard_normal((g, n, d))).requires_grad_()
        kk = torch.from_numpy(r.standard_normal((n, d))).requires_grad_()
        vv = torch.from_numpy(r.standard_normal((n, d))).requires_grad_()
        dout = torch.from_numpy(r.standard_normal((g, n, d)))
        s = (q @ kk.T) / math.sqrt(d)
        s = s.masked_fill(~mask, -math.inf)
        live = mask.any(dim=1)
        p = torch.softmax(s.masked_fill(~live[:, None], 0.0), dim=-1) * live[:, None]
        out = p @ vv
        (out * dout).sum().backward()
        dq, dk, dv = O.attention_backward(q.detach().numpy(), kk.detach().numpy(),
                                          vv.detach().numpy(), lists, dout.numpy(), c, causal)
        for name, a, b in (("q", dq, q.grad), ("k", dk, kk.grad), ("v", dv, vv.grad)):
            assert np.max(np.abs(a - b.numpy())) <= 1e-11, (name, causal)
        if not causal:
            assert np.all(dq[:, 5] == 0.0)


def pin_attention_grad_invariants(O):
    """Facts fixed by the softmax: per row the dv contributions sum to the
    group's dout (the weights sum to one); sum_t dq_t.q_t = sum_j dk_j.k_j (both
    are scale * sum dz q.k); a row that sees one token gets dq = 0, dk = 0 and
    dv = dout; key_block_grad agrees with the whole-head sums."""
    r = rng(23)
    n, c, d, k, g = 96, 8, 6, 4, 2
    q = r.standard_normal((g, n, d))
    keys = r.standard_normal((n, d))
    vals = r.standard_normal((n, d))
    dout = r.standard_normal((g, n, d))
    lists = random_lists(r, n, c, k, True)
    for t in (0, 17, 95):
        cols, gq, gk, gv = O.attend_row_grad(q[:, t], keys, vals, lists[t], t, c, dout[:, t])
        assert np.allclose(gv.sum(axis=0), dout[:, t].sum(axis=0), atol=1e-12)
        assert np.allclose(np.sum(gq * q[:, t]), np.sum(gk * keys[cols]), atol=1e-12)
    cols, gq, gk, gv = O.attend_row_grad(q[:, 0], keys, vals, [0], 0, c, dout[:, 0])
    assert cols == [0] and np.all(np.abs(gq) < 1e-15) and np.all(np.abs(gk) < 1e-15)
    assert np.allclose(gv[0], dout[:, 0].sum(axis=0), atol=1e-15)
    dq, dk, dv = O.attention_backward(q, keys, vals, lists, dout, c, True)
    assert np.allclose(np.sum(dq * q), np.sum(dk * keys), atol=1e-10)
    assert np.allclose(dv.sum(axis=0), dout.sum(axis=(0, 1)), atol=1e-10)
    for blk in (0, 3, n // c - 1):
        bk, bv = O.key_block_grad(q, keys, vals, lists, dout, blk, c, True)
        assert np.allclose(bk, dk[blk * c:(blk + 1) * c], atol=1e-12)
        assert np.allclose(bv, dv[blk * c:(blk + 1) * c], atol=1e-12)


# ------------------------------------------- selection-quality diagnostics
def dense_block_masses(q_heads, keys, block, scale):
    """Leaf-block attention masses by a route independent of the oracle: each
    head's full causal softmax matrix (torch, float64), its columns summed per
    leaf block, then averaged over the heads.  q_heads [G, n, d], keys [n, d];
    returns [n, n_leaves] (row t is zero past t's leaf)."""
    q = torch.tensor(np.asarray(q_heads, dtype=np.float64))
    k = torch.tensor(np.asarray(keys, dtype=np.float64))
    n = k.shape[0]
    s = scale * torch.matmul(q, k.T)
    s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    p = torch.softmax(s, dim=-1)
    nb = -(-n // block)
    p = torch.nn.functional.pad(p, (0, nb * block - n))
    return p.reshape(p.shape[0], n, nb, block).sum(dim=-1).mean(dim=0).numpy()


def _quality_problem(seed=41, n=200, block=16, d=8, g=3):
    r = rng(seed)
    # heads of different norms, so that summing instead of averaging, or
    # weighting heads unevenly, changes the numbers
    q = r.standard_normal((g, n, d)) * np.array([0.5, 1.0, 2.0][:g])[:, None, None]
    keys = r.standard_normal((n, d))
    return q, keys, block, 1.0 / math.sqrt(d)


def pin_block_masses_dense(M):
    """§7.2's retained attention mass is a share of each head's full causal
    attention; for a GQA group the reference averages the heads (§4.4).
    block_masses must equal the dense route's row, and sum to one."""
    q, keys, block, scale = _quality_problem()
    dense = dense_block_masses(q, keys, block, scale)
    for t in (0, 15, 16, 77, 150, 199):
        c = t // block
        got = M.block_masses(q[:, t], keys, t, block, scale)
        assert got.shape == (c + 1,), (t, got.shape)
        assert np.max(np.abs(got - dense[t, :c + 1])) <= 1e-12, t
        assert abs(got.sum() - 1.0) <= 1e-12, t


def pin_selection_quality_hand_sets(M):
    """Recall@K counts the forced blocks (§7.2, Table 7 note), net recall drops
    them from both sets, retained mass is the selected blocks' share of the
    full causal mass (not renormalised over the selection) and the mass ratio
    divides by the reference set's share.  Hand-built sets with known counts."""
    q, keys, block, scale = _quality_problem()
    dense = dense_block_masses(q, keys, block, scale)
    t = 9 * block + 5                      # leaf c = 9: forced {0, 8, 9}
    sel = [0, 2, 4, 5, 8, 9, -1]
    ref = [0, 2, 3, 7, 8, 9]
    res = M.selection_quality(sel, ref, q[:, t], keys, t, block, 6, True, scale)
    assert res["recall"] == 4 / 6, res     # 0, 2, 8, 9 shared
    assert res["net_recall"] == 1 / 3, res  # only 2 of the 3 free slots
    kept = dense[t, [0, 2, 4, 5, 8, 9]].sum()
    kept_ref = dense[t, ref].sum()
    assert abs(res["retained_mass"] - kept) <= 1e-12, res
    assert abs(res["mass_ratio"] - kept / kept_ref) <= 1e-12, res
    # every eligible block selected: all of the mass, full recall
    everything = list(range(10))
    res = M.selection_quality(everything, everything, q[:, t], keys, t, block, 10, True, scale)
    assert abs(res["retained_mass"] - 1.0) <= 1e-12 and res["recall"] == 1.0, res
    assert res["net_recall"] == 1.0 and abs(res["mass_ratio"] - 1.0) <= 1e-12, res


def pin_exhaustive_mean_mass(O):
    """The mean-mass reference of §4.4 for a GQA group: forced blocks plus the
    best K - #F others by head-averaged block mass (dense route, lexsort with
    ties to the lower index).  With one head it ranks as the summed exact leaf
    LSE does (the mass is a monotone function of the leaf LSE)."""
    q, keys, block, scale = _quality_problem(seed=43)
    dense = dense_block_masses(q, keys, block, scale)
    k = 5
    for t in range(40, 200, 3):
        c = t // block
        forced = {0, c - 1, c}
        rank = [i for i in range(c + 1) if i not in forced]
        m = dense[t, rank]
        order = np.lexsort((np.asarray(rank), -m))
        want = sorted(forced | {rank[j] for j in order[:k - len(forced)]})
        got = O.select_exhaustive_row(q[:, t], keys, t, block, k, True, True, scale,
                                      rule="mean_mass").leaves
        assert got == want, (t, got, want)
        one = O.select_exhaustive_row(q[2:, t], keys, t, block, k, True, True, scale,
                                      rule="mean_mass").leaves
        lse = O.select_exhaustive_row(q[2:, t], keys, t, block, k, True, True, scale).leaves
        assert one == lse, (t, one, lse)


ALL_PINS = [
    pin_tower_tables, pin_eq6_bounds, pin_pyramid_closed_form, pin_leaf_lse_is_logsumexp,
    pin_jensen_sandwich, pin_taylor_expansion, pin_no_pruning_equals_exhaustive,
    pin_dense_attention_recovered, pin_brute_force_tiny, pin_bsa_is_gemm_topk,
    pin_gqa_duplication, pin_causality_and_decode, pin_worked_causal_example, pin_tie_rule,
    pin_attention_grad_finite_differences, pin_attention_grad_autograd,
    pin_attention_grad_invariants, pin_exhaustive_mean_mass,
]

# Pins of the selection-quality diagnostics; they take the metrics module.
METRIC_PINS = [pin_block_masses_dense, pin_selection_quality_hand_sets]
