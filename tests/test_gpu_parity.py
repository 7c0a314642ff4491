"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Every call goes through the C ABI (the ctypes binding marshals arguments only).
Small shapes are compared on every row; the workload shapes (c1-c5) at their
full sizes, in the launch configuration the benchmark times, on sampled rows
and heads.  "unit" variants redraw the same shapes with N(0,1) entries so that
most rows clear the 1e-3 margin filter (at N(0,1/d) almost every row is a
near-tie and only structure and attention can be compared).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import parity
from hierarchical_block_selection_amd import (Problem, pisa_block_sparse_attn, pisa_bsa_select,
                                              pisa_build_pyramid, pisa_decode_step,
                                              pisa_pyramid_layout, pisa_select,
                                              pisa_workspace_bytes)
from hierarchical_block_selection_amd.inputs import (WORKLOADS, decode_inputs, prefill_inputs,
                                                     sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def problem_of(cfg, **over):
    kw = dict(batch=cfg["batch"], heads_q=cfg["heads_q"], heads_kv=cfg["heads_kv"],
              seq_len=cfg["seq_len"], head_dim=cfg["head_dim"], block=cfg["block"],
              topk=cfg["topk"], dtype=cfg["dtype"], causal=True, force_first_prev=True)
    kw.update(over)
    return Problem(**kw)


def levels_from_gpu_layout(pyr_head, n, c):
    offs = pisa_pyramid_layout(n, c)
    return [pyr_head[offs[i]:offs[i + 1]] for i in range(len(offs) - 1)]


def check_pyramid(pyr, k, prob, heads):
    """Every level of the GPU pyramid against the oracle (fp32 sums of <= C terms)."""
    for b, h in heads:
        keys = parity.to_np(k[b, h])
        want = oracle.build_pyramid(keys, prob.block)
        got = levels_from_gpu_layout(parity.to_np(pyr[b, h]), prob.seq_len, prob.block)
        assert len(got) == len(want)
        tol = 4e-6 * max(np.abs(keys).max(), 1e-30)
        for lg, lw in zip(got, want):
            assert lg.shape == lw.shape
            assert np.max(np.abs(lg - lw)) <= tol


def run_and_compare(cfg, recipe, heads, n_random, strategy="auto", check_bsa=True,
                    min_rows=None):
    prob = problem_of(cfg)
    announce(f"prefill N={prob.seq_len} H={prob.heads_q}/{prob.heads_kv} d={prob.head_dim} "
             f"K={prob.topk} {recipe} strategy={strategy}")
    inp = prefill_inputs(prob.batch, prob.heads_q, prob.heads_kv, prob.seq_len, prob.head_dim,
                         prob.dtype, seed=cfg["seed"], recipe=recipe,
                         n_needles=cfg["n_needles"], block=prob.block, device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr, strategy=strategy)
    if check_bsa:
        bidx, bscore = pisa_bsa_select(prob, inp.q, pyr)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    torch.cuda.synchronize()
    check_pyramid(pyr, inp.k, prob, heads[:2])
    rows = sample_rows(prob.seq_len, prob.block, prob.topk, n_random, cfg["seed"])
    g = prob.group
    fp32 = prob.dtype == torch.float32
    tallies = {"pisa": parity.Tally(), "bsa": parity.Tally()}
    for b, h in heads:
        keys = parity.to_np(inp.k[b, h])
        vals = parity.to_np(inp.v[b, h])
        qg = parity.to_np(inp.q[b, h * g:(h + 1) * g])
        levels = oracle.build_pyramid(keys, prob.block)
        parity.compare_selection("pisa", idx[b, h].cpu().numpy(), score[b, h].cpu().numpy(), qg,
                                 keys, levels, rows, prob.block, prob.topk, True, True,
                                 prob.logit_scale, tallies["pisa"])
        if check_bsa:
            parity.compare_selection("bsa", bidx[b, h].cpu().numpy(), bscore[b, h].cpu().numpy(),
                                     qg, keys, levels, rows, prob.block, prob.topk, True, True,
                                     prob.logit_scale, tallies["bsa"])
        parity.compare_attention(parity.to_np(out[b, h * g:(h + 1) * g]),
                                 lse[b, h * g:(h + 1) * g].cpu().numpy(), qg, keys, vals,
                                 idx[b, h].cpu().numpy(), rows, prob.block, True,
                                 prob.logit_scale, fp32)
    for name, tl in tallies.items():
        print(f"  {name}: compared {tl.compared}/{tl.rows} rows, mismatches {len(tl.mismatches)}",
              flush=True)
        assert not tl.mismatches, tl.mismatches[:3]
        if min_rows is not None and (name == "pisa" or check_bsa):
            assert tl.compared >= min_rows, (name, tl.compared, tl.rows)
    return tallies


HEADS = {"c1": [(0, 0), (0, 1)], "c2": [(0, 0), (0, 9), (0, 15)], "c3": [(0, 0), (0, 6)],
         "c4a": [(0, 0), (0, 3)], "c4b": [(0, 1), (0, 2)], "c4c": [(0, 0), (0, 3)]}


def test_c1_all_rows():
    cfg = WORKLOADS["c1"]
    prob = problem_of(cfg)
    announce("c1 all rows")
    inp = prefill_inputs(1, 2, 2, 2048, 64, torch.float32, seed=cfg["seed"], recipe="unit",
                         device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr)
    bidx, bscore = pisa_bsa_select(prob, inp.q, pyr)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    torch.cuda.synchronize()
    check_pyramid(pyr, inp.k, prob, [(0, 0), (0, 1)])
    rows = list(range(2048))
    for h in range(2):
        keys, vals = parity.to_np(inp.k[0, h]), parity.to_np(inp.v[0, h])
        qg = parity.to_np(inp.q[0, h:h + 1])
        levels = oracle.build_pyramid(keys, 64)
        tp = parity.compare_selection("pisa", idx[0, h].cpu().numpy(), score[0, h].cpu().numpy(),
                                      qg, keys, levels, rows, 64, 4, True, True, prob.logit_scale,
                                      parity.Tally())
        tb = parity.compare_selection("bsa", bidx[0, h].cpu().numpy(), bscore[0, h].cpu().numpy(),
                                      qg, keys, levels, rows, 64, 4, True, True, prob.logit_scale,
                                      parity.Tally())
        assert not tp.mismatches and not tb.mismatches, (tp.mismatches[:2], tb.mismatches[:2])
        assert tp.frac() > 0.9 and tb.frac() > 0.9
        parity.compare_attention(parity.to_np(out[0, h:h + 1]), lse[0, h:h + 1].cpu().numpy(), qg,
                                 keys, vals, idx[0, h].cpu().numpy(), rows, 64, True,
                                 prob.logit_scale, fp32=True)


@pytest.mark.parametrize("name", ["c2", "c3", "c4a", "c4b", "c4c"])
def test_workload_parity_unit_variant(name):
    """Workload shape with N(0,1) entries: a good share of rows clears the margin
    filter (fewer as the pyramid deepens: every scored level must clear it), so,
    with enough rows sampled, at least 100 rows per selector are compared bit
    for bit."""
    n_random = 192 if WORKLOADS[name]["seq_len"] <= 65536 else 480
    run_and_compare(WORKLOADS[name], "unit", HEADS[name], n_random=n_random, min_rows=100)


def test_mha_k8_sweep_shape():
    """The shape of the benchmark's K = 8 selection sweep (4 heads, one per KV
    head, d = 128) at 64K tokens, with N(0,1) entries: at least 100 rows per
    selector compared bit for bit past the margin."""
    cfg = dict(WORKLOADS["c4a"], seq_len=65536, topk=8, seed=4220)
    run_and_compare(cfg, "unit", [(0, 0), (0, 3)], n_random=192, min_rows=100)


@pytest.mark.parametrize("name", ["c2", "c3", "c4a", "c4b", "c4c"])
def test_workload_parity_as_configured(name):
    """Workload as configured (N(0,1/d), needles where stated): near-ties dominate,
    so structure and attention carry the check; exact sets where margins allow."""
    run_and_compare(WORKLOADS[name], WORKLOADS[name]["recipe"], HEADS[name], n_random=24)


EDGE = [
    # (N, C, d, K, Hq, Hkv, dtype, causal, force)
    (1, 64, 64, 4, 1, 1, torch.float32, True, True),
    (63, 64, 128, 4, 2, 2, torch.bfloat16, True, True),
    (100, 16, 64, 3, 2, 1, torch.float32, True, True),
    (1000, 32, 64, 5, 4, 2, torch.float32, True, True),
    (1000, 16, 128, 7, 2, 2, torch.bfloat16, True, False),
    (777, 16, 64, 4, 3, 3, torch.float32, False, False),
    (2048 + 17, 64, 128, 16, 16, 1, torch.bfloat16, True, True),
    (4096, 64, 64, 32, 4, 4, torch.float32, True, True),
    (3000, 64, 128, 8, 8, 2, torch.float32, False, False),
    (5000, 16, 128, 32, 2, 2, torch.bfloat16, True, True),
    # bf16, C=64: two-stage selection and the MFMA block attention path
    (5000, 64, 128, 8, 4, 2, torch.bfloat16, True, True),
    (4196, 64, 64, 32, 2, 2, torch.bfloat16, True, True),
    (3000, 64, 128, 5, 1, 1, torch.bfloat16, False, False),
    (1100, 64, 128, 4, 4, 1, torch.bfloat16, True, True),
    (8192, 64, 128, 16, 1, 1, torch.bfloat16, True, False),
    # two-stage selection with 8 and 16 query heads per KV head (the pages'
    # latency shape is G = 16, d = 64, K = 8)
    (6000, 64, 64, 8, 16, 1, torch.bfloat16, True, True),
    (5000, 64, 128, 16, 16, 2, torch.bfloat16, True, True),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"N{c[0]}_C{c[1]}_d{c[2]}_K{c[3]}_G{c[4]//c[5]}_"
                                            f"{'bf16' if c[6] == torch.bfloat16 else 'f32'}_"
                                            f"{'causal' if c[7] else 'full'}{'_force' if c[8] else ''}"
                                            for c in EDGE])
def test_edge_shapes_every_row(case):
    n, c, d, k, hq, hkv, dtype, causal, force = case
    prob = Problem(1, hq, hkv, n, d, block=c, topk=k, dtype=dtype, causal=causal,
                   force_first_prev=force)
    announce(f"edge {case}")
    inp = prefill_inputs(1, hq, hkv, n, d, dtype, seed=77 + n, recipe="unit", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr)
    bidx, bscore = pisa_bsa_select(prob, inp.q, pyr)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    torch.cuda.synchronize()
    check_pyramid(pyr, inp.k, prob, [(0, h) for h in range(hkv)])
    g = hq // hkv
    rows = list(range(n)) if n <= 1100 else list(range(0, n, 3)) + [n - 1]
    for h in range(hkv):
        keys, vals = parity.to_np(inp.k[0, h]), parity.to_np(inp.v[0, h])
        qg = parity.to_np(inp.q[0, h * g:(h + 1) * g])
        levels = oracle.build_pyramid(keys, c)
        for kind, ii, ss in (("pisa", idx, score), ("bsa", bidx, bscore)):
            tl = parity.compare_selection(kind, ii[0, h].cpu().numpy(), ss[0, h].cpu().numpy(), qg,
                                          keys, levels, rows, c, k, causal, force,
                                          prob.logit_scale, parity.Tally())
            assert not tl.mismatches, (kind, tl.mismatches[:3])
            assert tl.frac() > 0.6, (kind, tl.frac())
        parity.compare_attention(parity.to_np(out[0, h * g:(h + 1) * g]),
                                 lse[0, h * g:(h + 1) * g].cpu().numpy(), qg, keys, vals,
                                 idx[0, h].cpu().numpy(), rows, c, causal, prob.logit_scale,
                                 fp32=dtype == torch.float32)


BATCHED = [
    # (B, N, C, d, K, Hq, Hkv, dtype): several sequences per call on the paths
    # the workloads take (two-stage selection, block-centric attention, MFMA
    # BSA for bf16 at C = 64) and on the general ones
    (3, 6000, 64, 128, 16, 8, 2, torch.bfloat16),
    (2, 4096, 64, 64, 8, 2, 2, torch.bfloat16),
    (2, 2500, 32, 64, 6, 4, 4, torch.float32),
]


@pytest.mark.parametrize("case", BATCHED, ids=[f"B{c[0]}_N{c[1]}_C{c[2]}_d{c[3]}_K{c[4]}_"
                                               f"G{c[5] // c[6]}_"
                                               f"{'bf16' if c[7] == torch.bfloat16 else 'f32'}"
                                               for c in BATCHED])
def test_prefill_batches(case):
    """Prefill with several sequences per call: every (sequence, KV head)
    against the oracle on every eleventh row and the last (N(0,1) entries)."""
    bsz, n, c, d, k, hq, hkv, dtype = case
    prob = Problem(bsz, hq, hkv, n, d, block=c, topk=k, dtype=dtype)
    announce(f"prefill batch {case}")
    inp = prefill_inputs(bsz, hq, hkv, n, d, dtype, seed=9100 + n, recipe="unit", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr)
    bidx, bscore = pisa_bsa_select(prob, inp.q, pyr)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    torch.cuda.synchronize()
    check_pyramid(pyr, inp.k, prob, [(b, h) for b in range(bsz) for h in range(hkv)])
    g = hq // hkv
    rows = list(range(0, n, 11)) + [n - 1]
    for b in range(bsz):
        for h in range(hkv):
            keys, vals = parity.to_np(inp.k[b, h]), parity.to_np(inp.v[b, h])
            qg = parity.to_np(inp.q[b, h * g:(h + 1) * g])
            levels = oracle.build_pyramid(keys, c)
            for kind, ii, ss in (("pisa", idx, score), ("bsa", bidx, bscore)):
                tl = parity.compare_selection(kind, ii[b, h].cpu().numpy(), ss[b, h].cpu().numpy(),
                                              qg, keys, levels, rows, c, k, True, True,
                                              prob.logit_scale, parity.Tally())
                assert not tl.mismatches, (kind, b, h, tl.mismatches[:3])
                assert tl.frac() > 0.5, (kind, b, h, tl.frac())
            parity.compare_attention(parity.to_np(out[b, h * g:(h + 1) * g]),
                                     lse[b, h * g:(h + 1) * g].cpu().numpy(), qg, keys, vals,
                                     idx[b, h].cpu().numpy(), rows, c, True, prob.logit_scale,
                                     fp32=dtype == torch.float32)


@pytest.mark.parametrize("name", ["c2", "c4a"])
def test_workload_parity_fused_strategy(name):
    """The per-query fused selector on the workload shape (the default picks the
    two-stage selector for bf16)."""
    run_and_compare(WORKLOADS[name], "unit", HEADS[name], n_random=32, strategy="fused",
                    check_bsa=False, min_rows=20)


def test_selection_and_attention_deterministic():
    cfg = WORKLOADS["c4a"]
    prob = problem_of(cfg)
    announce("determinism c4a")
    inp = prefill_inputs(1, 4, 4, cfg["seq_len"], 128, torch.bfloat16, seed=9, device=DEV)
    pyr1 = pisa_build_pyramid(prob, inp.k)
    pyr2 = pisa_build_pyramid(prob, inp.k)
    i1, s1 = pisa_select(prob, inp.q, inp.k, pyr1)
    i2, s2 = pisa_select(prob, inp.q, inp.k, pyr2)
    b1, _ = pisa_bsa_select(prob, inp.q, pyr1)
    b2, _ = pisa_bsa_select(prob, inp.q, pyr2)
    o1, l1 = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, i1)
    o2, l2 = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, i2)
    torch.cuda.synchronize()
    assert torch.equal(pyr1, pyr2)
    assert torch.equal(i1, i2) and torch.equal(s1, s2) and torch.equal(b1, b2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def decode_compare(prob, inp, pyr, pairs, fp32=False, min_compared=None, min_count=None):
    idx, score, out, lse = pisa_decode_step(prob, inp.cache_len, inp.q, inp.k_cache, inp.v_cache,
                                            pyr)
    torch.cuda.synchronize()
    g = prob.group
    tally = parity.Tally()
    for b, h in pairs:
        n = int(inp.cache_len[b])
        keys = parity.to_np(inp.k_cache[b, h, :n])
        vals = parity.to_np(inp.v_cache[b, h, :n])
        qg = parity.to_np(inp.q[b, h * g:(h + 1) * g])
        force = prob.force_first_prev
        sel, ref, ref_lse = oracle.decode_row(qg, keys, vals, n, prob.block, prob.topk,
                                              force_first_prev=force, variant=prob.score)
        got = [int(x) for x in idx[b, h].cpu()]
        parity.check_structure(got, n - 1, prob.block, prob.topk, -(-n // prob.block), True, force)
        tally.rows += 1
        if sel.min_margin > parity.MARGIN:
            tally.compared += 1
            assert got == oracle.padded(sel.leaves, prob.topk), (b, h, got, sel.leaves)
        # attention against the oracle with the GPU's own selection
        leaves = [x for x in got if x >= 0]
        ref2, ref2_lse = oracle.attend_row(qg, keys, vals, leaves, n - 1, prob.block, True)
        o = parity.to_np(out[b, h * g:(h + 1) * g])
        d = np.abs(o - ref2)
        if fp32:
            assert d.max() <= 1e-3 * np.abs(ref2).max()
        else:
            assert d.max() <= 2e-2
            assert np.linalg.norm(o - ref2) <= 1e-2 * np.linalg.norm(ref2)
        assert np.max(np.abs(lse[b, h * g:(h + 1) * g].cpu().numpy() - ref2_lse)) <= 1e-3
    print(f"  decode: compared {tally.compared}/{tally.rows}", flush=True)
    if min_compared is not None:
        assert tally.frac() >= min_compared
    if min_count is not None:
        assert tally.compared >= min_count, (tally.compared, tally.rows)
    return idx, out


def test_decode_c5_sampled():
    cfg = WORKLOADS["c5"]
    prob = problem_of(cfg)
    announce("decode c5 B=32 cache=131072 GQA 32/8")
    inp = decode_inputs(32, 32, 8, cfg["seq_len"], 128, torch.bfloat16, seed=cfg["seed"],
                        device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k_cache)
    decode_compare(prob, inp, pyr, [(0, h) for h in range(8)] + [(17, h) for h in range(8)])


def test_decode_c5_unit_variance():
    """The decode workload at its full shape (32 sequences, 131072-token caches,
    32 query heads over 8 KV heads, d = 128, K = 16, 12 pyramid levels) with
    N(0,1) entries, so that the selection can be compared: 96 (sequence, KV
    head) units, bit-exact on every unit whose decision margins all exceed
    1e-3 (about a quarter of them at this length), at least 8 such units."""
    cfg = WORKLOADS["c5"]
    prob = problem_of(cfg)
    announce("decode c5 B=32 cache=131072 GQA 32/8 unit")
    inp = decode_inputs(32, 32, 8, cfg["seq_len"], 128, torch.bfloat16, seed=cfg["seed"],
                        recipe="unit", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k_cache)
    seqs = (0, 2, 5, 7, 10, 13, 16, 19, 22, 25, 28, 31)
    decode_compare(prob, inp, pyr, [(b, h) for b in seqs for h in range(8)], min_count=8)


@pytest.mark.parametrize("n,hq,d,k", [(262144 + 128, 2, 128, 16), (262144 + 128, 1, 128, 16),
                                      (262144 + 128, 16, 64, 8), (524288, 1, 128, 16),
                                      (524288, 8, 64, 16)])
def test_prefill_level2_beyond_dense_rows(n, hq, d, k):
    """Prefills past 256K tokens, where level 2 holds more rows than one
    window of the first selection stage (2048), so that its level-3 decision
    runs over several windows: 262272 tokens (level 2: 2049 rows, the second
    window one row) at 1, 2 and 16 query heads per KV head, and 524288
    (level 2: two full windows) at 1 and 8.  At 524288 BSA as well: 8192
    leaf blocks, so its Top-K takes the longer rows in two segments.  N(0,1)
    entries, 200 sampled rows (400 at 524288): selections bit-exact past the
    margin (at least 20 rows), attention within the bf16 bounds."""
    prob = Problem(1, hq, 1, n, d, block=64, topk=k, dtype=torch.bfloat16)
    announce(f"prefill N={n} G={hq} d={d} K={k} unit (level 2 beyond one window)")
    inp = prefill_inputs(1, hq, 1, n, d, torch.bfloat16, seed=7100 + hq, recipe="unit",
                         device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    with_bsa = -(-n // 64) % 4 == 0
    if with_bsa:
        bidx, bscore = pisa_bsa_select(prob, inp.q, pyr)
    torch.cuda.synchronize()
    check_pyramid(pyr, inp.k, prob, [(0, 0)])
    # deeper pyramids leave fewer rows past the margin at every level
    rows = sample_rows(n, 64, k, 200 if n < 500000 else 400, 7100)
    keys, vals = parity.to_np(inp.k[0, 0]), parity.to_np(inp.v[0, 0])
    qg = parity.to_np(inp.q[0, 0:hq])
    levels = oracle.build_pyramid(keys, 64)
    tl = parity.compare_selection("pisa", idx[0, 0].cpu().numpy(), score[0, 0].cpu().numpy(), qg,
                                  keys, levels, rows, 64, k, True, True, prob.logit_scale,
                                  parity.Tally())
    print(f"  pisa: compared {tl.compared}/{tl.rows} rows, mismatches {len(tl.mismatches)}",
          flush=True)
    assert not tl.mismatches, tl.mismatches[:3]
    assert tl.compared >= 20, (tl.compared, tl.rows)
    if with_bsa:
        tb = parity.compare_selection("bsa", bidx[0, 0].cpu().numpy(), bscore[0, 0].cpu().numpy(),
                                      qg, keys, levels, rows, 64, k, True, True,
                                      prob.logit_scale, parity.Tally())
        long_rows = sum(1 for r in rows if r // 64 >= 4096)
        print(f"  bsa: compared {tb.compared}/{tb.rows} rows ({long_rows} past 4096 leaves), "
              f"mismatches {len(tb.mismatches)}", flush=True)
        assert not tb.mismatches, tb.mismatches[:3]
        assert tb.compared >= 20 and long_rows >= 50, (tb.compared, long_rows)
    parity.compare_attention(parity.to_np(out[0, 0:hq]), lse[0, 0:hq].cpu().numpy(), qg, keys,
                             vals, idx[0, 0].cpu().numpy(), rows, 64, True, prob.logit_scale,
                             False)


@pytest.mark.parametrize("n,d,k", [(65536, 64, 8), (131072, 64, 8), (32768, 128, 16)])
def test_pages_latency_shape_g16(n, d, k):
    """16 query heads per KV head (the pages' latency shape: d = 64, K = 8)
    at lengths where each wave of the two-stage selector scores only the
    union of its 4 queries' kept parents: unit entries, sampled rows bit-exact
    past the margin, at least 60 rows compared."""
    cfg = dict(batch=1, heads_q=16, heads_kv=1, seq_len=n, head_dim=d, block=64, topk=k,
               dtype=torch.bfloat16, n_needles=0, seed=9100 + d + k)
    run_and_compare(cfg, "unit", [(0, 0)], n_random=160, min_rows=60)


def test_union_tile_windows():
    """The union tiles' window loop (16 query heads per KV head), which the
    default 8192-row windows reach only past 1M tokens: with 128-row windows
    (PISA_S1_TILE_ROWS) a 64K prefill scores its level-3 decision over 4
    windows and its level-4 decision over 2.  The selection must equal the
    one-window run bit for bit (each candidate's score does not depend on the
    tile it lands in) and the oracle past the margin."""
    import os
    n, d, k = 65536, 64, 8
    prob = Problem(1, 16, 1, n, d, block=64, topk=k, dtype=torch.bfloat16)
    announce(f"prefill N={n} G=16 d={d} K={k} unit, 128-row union-tile windows")
    inp = prefill_inputs(1, 16, 1, n, d, torch.bfloat16, seed=9300, recipe="unit", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx1, score1 = pisa_select(prob, inp.q, inp.k, pyr)
    saved = os.environ.get("PISA_S1_TILE_ROWS")
    os.environ["PISA_S1_TILE_ROWS"] = "128"
    try:
        idx2, score2 = pisa_select(prob, inp.q, inp.k, pyr)
        torch.cuda.synchronize()
    finally:
        if saved is None:
            del os.environ["PISA_S1_TILE_ROWS"]
        else:
            os.environ["PISA_S1_TILE_ROWS"] = saved
    assert torch.equal(idx1, idx2) and torch.equal(score1, score2)
    rows = sample_rows(n, 64, k, 120, 9300)
    keys = parity.to_np(inp.k[0, 0])
    qg = parity.to_np(inp.q[0])
    levels = oracle.build_pyramid(keys, 64)
    tl = parity.compare_selection("pisa", idx2[0, 0].cpu().numpy(), score2[0, 0].cpu().numpy(),
                                  qg, keys, levels, rows, 64, k, True, True, prob.logit_scale,
                                  parity.Tally())
    print(f"  pisa: compared {tl.compared}/{tl.rows} rows, mismatches {len(tl.mismatches)}",
          flush=True)
    assert not tl.mismatches, tl.mismatches[:3]
    assert tl.compared >= 40, (tl.compared, tl.rows)


def test_large_group_scores():
    """Peaked attention and large group-summed scores (queries N(0,64), keys
    N(0,1): group sums of several hundred nats over 16 query heads): the
    ranking must follow the scores, not the magnitude's rounding.  Prefill at
    16 query heads per KV head, d = 64, K = 8, every 13th row; decode at 8
    query heads per KV head, K = 16."""
    n = 16384
    prob = Problem(1, 16, 1, n, 64, block=64, topk=8, dtype=torch.bfloat16)
    announce(f"prefill N={n} G=16 d=64 K=8 wide_q")
    inp = prefill_inputs(1, 16, 1, n, 64, torch.bfloat16, seed=8100, recipe="wide_q", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, score = pisa_select(prob, inp.q, inp.k, pyr)
    torch.cuda.synchronize()
    keys = parity.to_np(inp.k[0, 0])
    qg = parity.to_np(inp.q[0])
    levels = oracle.build_pyramid(keys, 64)
    rows = list(range(0, n, 13)) + [n - 1]
    tl = parity.compare_selection("pisa", idx[0, 0].cpu().numpy(), score[0, 0].cpu().numpy(), qg,
                                  keys, levels, rows, 64, 8, True, True, prob.logit_scale,
                                  parity.Tally())
    print(f"  pisa: compared {tl.compared}/{tl.rows} rows, mismatches {len(tl.mismatches)}",
          flush=True)
    assert not tl.mismatches, tl.mismatches[:3]
    assert tl.frac() > 0.9, tl.frac()
    dprob = Problem(4, 16, 2, n, 128, block=64, topk=16, dtype=torch.bfloat16)
    announce("decode G=8 wide_q")
    dinp = decode_inputs(4, 16, 2, n, 128, torch.bfloat16, seed=8200, recipe="wide_q",
                         cache_len=[n, 12345, 9000, 4097], device=DEV)
    dpyr = pisa_build_pyramid(dprob, dinp.k_cache)
    decode_compare(dprob, dinp, dpyr, [(b, h) for b in range(4) for h in range(2)],
                   min_compared=0.75)


def test_decode_unit_variant_ragged_lengths():
    prob = Problem(4, 8, 2, 8192, 128, block=64, topk=16, dtype=torch.bfloat16)
    announce("decode ragged lengths unit")
    inp = decode_inputs(4, 8, 2, 8192, 128, torch.bfloat16, seed=31, recipe="unit",
                        cache_len=[1, 63, 3001, 8192], device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k_cache)
    decode_compare(prob, inp, pyr, [(b, h) for b in range(4) for h in range(2)], min_compared=0.5)


DECODE_SHAPES = [
    # (B, Hq, Hkv, capacity, d, K, force, cache lengths)
    (3, 8, 1, 8192, 128, 16, True, [1, 4000, 8192]),
    (2, 2, 2, 8192, 64, 8, False, [700, 8192]),
    (2, 4, 2, 6000, 128, 5, True, [65, 6000]),
    (2, 4, 4, 16384, 128, 16, True, [16384, 9999]),
    (2, 8, 2, 4096, 64, 16, True, [4096, 130]),
]


@pytest.mark.parametrize("case", DECODE_SHAPES, ids=[f"B{c[0]}_G{c[1]//c[2]}_d{c[4]}_K{c[5]}"
                                                     f"{'_force' if c[6] else ''}"
                                                     for c in DECODE_SHAPES])
def test_decode_group_sizes(case):
    """The bf16 workgroup decode for every group size it serves (1, 2, 4, 8),
    d = 64 and 128, budgets below 16 and with and without first/previous
    forcing, on ragged cache lengths."""
    bsz, hq, hkv, cap, d, k, force, lens = case
    prob = Problem(bsz, hq, hkv, cap, d, block=64, topk=k, dtype=torch.bfloat16,
                   force_first_prev=force)
    announce(f"decode {case}")
    inp = decode_inputs(bsz, hq, hkv, cap, d, torch.bfloat16, seed=41 + cap, recipe="unit",
                        cache_len=lens, device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k_cache)
    decode_compare(prob, inp, pyr, [(b, h) for b in range(bsz) for h in range(hkv)])


def test_decode_equals_prefill_row():
    """A decode step at cache length n gives the prefill row t = n - 1 bit for bit."""
    n_cap, lens = 4096, [4096, 2500]
    prob = Problem(2, 4, 1, n_cap, 64, block=64, topk=8, dtype=torch.float32)
    announce("decode == prefill row")
    inp = decode_inputs(2, 4, 1, n_cap, 64, torch.float32, seed=5, recipe="unit", cache_len=lens,
                        device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k_cache)
    didx, dscore, dout, dlse = pisa_decode_step(prob, inp.cache_len, inp.q, inp.k_cache,
                                                inp.v_cache, pyr)
    q_full = torch.zeros((2, 4, n_cap, 64), dtype=torch.float32, device=DEV)
    for b, n in enumerate(lens):
        q_full[b, :, n - 1] = inp.q[b]
    idx, score = pisa_select(prob, q_full, inp.k_cache, pyr)
    out, lse = pisa_block_sparse_attn(prob, q_full, inp.k_cache, inp.v_cache, idx)
    torch.cuda.synchronize()
    for b, n in enumerate(lens):
        assert torch.equal(didx[b], idx[b, :, n - 1])
        assert torch.equal(dscore[b], score[b, :, n - 1])
        assert torch.equal(dout[b], out[b, :, n - 1])
        assert torch.equal(dlse[b], lse[b, :, n - 1])


ARB = [
    # (N, d, K, Hq, Hkv, causal)
    (5000, 128, 16, 1, 1, True),
    (4133, 64, 8, 4, 2, True),
    (3000, 128, 12, 2, 1, False),
    (2500, 128, 16, 16, 1, True),
    (700, 128, 5, 8, 1, True),
]


def arbitrary_block_lists(n, hkv, k, causal, seed):
    """Caller-made lists: unsorted rows mixing the always-attended blocks
    (0, c - 1, c) with others, -1 and out-of-range entries, future blocks and
    empty rows."""
    rng = np.random.default_rng(seed)
    m1 = -(-n // 64)
    idx = np.full((1, hkv, n, k), -1, np.int32)
    for h in range(hkv):
        for t in range(n):
            c = t // 64
            hi = c if causal else m1 - 1
            kind = rng.integers(0, 10)
            if kind < 4:  # the forced blocks plus random others
                base = sorted({0, max(c - 1, 0), c})
                rest = [x for x in rng.permutation(hi + 1)[:k] if x not in base]
                row = (base + rest)[:k]
            elif kind < 7:  # random subset, forced blocks only by chance
                row = list(rng.permutation(hi + 1)[:rng.integers(1, k + 1)])
            elif kind < 9:  # random subset with junk and (causal) future blocks
                row = list(rng.permutation(hi + 1)[:rng.integers(1, k)])
                junk = [-1, -7, m1, m1 + 5] + ([min(c + 1 + int(rng.integers(0, 3)), m1 - 1)]
                                              if causal and c + 1 < m1 else [])
                row = (row + [int(x) for x in rng.choice(junk, size=k - len(row))])[:k]
                vals = [x for x in row if 0 <= x < m1]
                if len(vals) != len(set(vals)):  # keep valid entries distinct
                    seen, dedup = set(), []
                    for x in row:
                        if 0 <= x < m1 and x in seen:
                            x = -1
                        seen.add(x)
                        dedup.append(x)
                    row = dedup
            else:  # nothing attendable
                row = [-1] * (k - 1) + [m1]
            row = [int(x) for x in rng.permutation(np.array(row + [-1] * (k - len(row))))]
            idx[0, h, t] = row
    return idx


@pytest.mark.parametrize("case", ARB, ids=[f"N{c[0]}_d{c[1]}_K{c[2]}_G{c[3]//c[4]}_"
                                           f"{'causal' if c[5] else 'full'}" for c in ARB])
def test_attention_arbitrary_block_lists(case):
    """bf16 block attention (C = 64) on block lists made by the caller."""
    n, d, k, hq, hkv, causal = case
    prob = Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16, causal=causal,
                   force_first_prev=causal)
    announce(f"arbitrary lists {case}")
    inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=500 + n, recipe="unit",
                         device=DEV)
    idx_np = arbitrary_block_lists(n, hkv, k, causal, seed=n)
    idx = torch.from_numpy(idx_np).to(DEV)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    torch.cuda.synchronize()
    g = hq // hkv
    m1 = -(-n // 64)
    rows = list(range(0, n, 2)) + [n - 1]
    for h in range(hkv):
        keys, vals = parity.to_np(inp.k[0, h]), parity.to_np(inp.v[0, h])
        qg = parity.to_np(inp.q[0, h * g:(h + 1) * g])
        o = parity.to_np(out[0, h * g:(h + 1) * g])
        ls = lse[0, h * g:(h + 1) * g].cpu().numpy()
        full, empty = [], []
        for t in rows:
            leaves = [int(x) for x in idx_np[0, h, t] if 0 <= x < m1]
            live = [x for x in leaves if not causal or x * 64 <= t]
            (full if live else empty).append(t)
        for t in empty:
            assert np.all(o[:, t] == 0.0) and np.all(np.isneginf(ls[:, t])), t
        sub = np.where(idx_np[0, h] >= m1, -1, idx_np[0, h])
        parity.compare_attention(o, ls, qg, keys, vals, sub, full, 64, causal,
                                 prob.logit_scale, fp32=False)
        assert len(empty) > 0 and len(full) > len(rows) // 2


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_attention_nothing_attendable(causal):
    """Lists that name no block at all (-1, negative junk and indices past the
    last block) leave the block path with no (row, block) pair and so no
    partial anywhere: every row must come out as zeros with row_lse = -inf,
    here from a workspace whose bytes are all 0xff (NaN in bf16 and fp32), so
    that a merge which multiplied an unwritten partial by a zero weight would
    show up as NaN."""
    n, d, k, hq, hkv = 300, 128, 4, 4, 2
    prob = Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16, causal=causal,
                   force_first_prev=False)
    announce(f"nothing attendable causal={causal}")
    inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=530, recipe="unit", device=DEV)
    m1 = -(-n // 64)
    idx = torch.tensor([-1, m1, -5, m1 + 3], dtype=torch.int32).repeat(1, hkv, n, 1).to(DEV)
    ws = torch.full((pisa_workspace_bytes(prob, "attn"),), 255, dtype=torch.uint8, device=DEV)
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


SCORE_CASES = [
    # (score, N, C, d, K, Hq, Hkv, dtype)
    ("mean", 3000, 64, 128, 8, 2, 1, torch.bfloat16),
    ("mean_var", 3000, 64, 128, 8, 2, 1, torch.bfloat16),
    ("mean", 2500, 32, 64, 16, 4, 4, torch.float32),
    ("mean_var", 2065, 16, 64, 5, 4, 2, torch.float32),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[f"{c[0]}_N{c[1]}_C{c[2]}_d{c[3]}_K{c[4]}_"
                                                   f"G{c[5]//c[6]}" for c in SCORE_CASES])
def test_score_variants(case):
    """PISA-1 (mean) and PISA-2 (mean + var/2) candidate scores (eq. (9)) on
    the per-query selector, prefill rows and a decode step, against the
    oracle's same variant."""
    score, n, c, d, k, hq, hkv, dtype = case
    prob = Problem(1, hq, hkv, n, d, block=c, topk=k, dtype=dtype, score=score)
    announce(f"score variant {case}")
    inp = prefill_inputs(1, hq, hkv, n, d, dtype, seed=91 + n, recipe="unit", device=DEV)
    pyr = pisa_build_pyramid(prob, inp.k)
    idx, sc = pisa_select(prob, inp.q, inp.k, pyr)
    torch.cuda.synchronize()
    g = hq // hkv
    rows = list(range(0, n, 2)) + [n - 1]
    for h in range(hkv):
        keys = parity.to_np(inp.k[0, h])
        qg = parity.to_np(inp.q[0, h * g:(h + 1) * g])
        levels = oracle.build_pyramid(keys, c)
        tl = parity.compare_selection("pisa", idx[0, h].cpu().numpy(), sc[0, h].cpu().numpy(), qg,
                                      keys, levels, rows, c, k, True, True, prob.logit_scale,
                                      parity.Tally(), variant=score)
        print(f"  {score}: compared {tl.compared}/{tl.rows}", flush=True)
        assert not tl.mismatches, tl.mismatches[:3]
        assert tl.frac() > 0.6
    dprob = Problem(2, hq, hkv, n, d, block=c, topk=k, dtype=dtype, score=score)
    dinp = decode_inputs(2, hq, hkv, n, d, dtype, seed=93 + n, recipe="unit",
                         cache_len=[n, n // 2 + 7], device=DEV)
    dpyr = pisa_build_pyramid(dprob, dinp.k_cache)
    decode_compare(dprob, dinp, dpyr, [(b, h) for b in range(2) for h in range(hkv)])
