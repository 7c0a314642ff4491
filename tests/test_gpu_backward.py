"""Backward of the block-sparse attention (block lists held fixed): the HIP path
against the CPU oracle on the same seeded inputs (needs an MI355X).

The GPU runs the forward (pisa_block_sparse_attn) and feeds its out / row_lse
to pisa_block_sparse_attn_backward, as a training step does.  The oracle takes
only Q, K, V, the lists and dO and computes everything in fp64.

Tolerance (bf16).  The kernels round P and dS to bf16 before the MFMA
products, each block's dQ contribution to bf16, O (from the forward) and the
outputs to bf16; all sums are fp32.  A CPU emulation of exactly these
roundings against fp64 gives max|err| <= 6e-3 max|ref| and a normwise error of
<= 3e-3 on these shapes, so the test allows 2e-2 max|ref| and 1e-2 normwise
per tensor and KV head (the forward's bf16 bounds, taken relative).

Small shapes are compared on every row and every key; the 128K workload shape
on sampled query rows (dq) and sampled key blocks (dk, dv, each summed over
all rows that list the block), plus the identities sum_j dv_j = sum over rows
and heads of dO and sum_t dq_t . q_t = sum_j dk_j . k_j over the whole head.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import parity
from hierarchical_block_selection_amd import (Problem, pisa_block_sparse_attn,
                                              pisa_block_sparse_attn_backward)
from hierarchical_block_selection_amd.inputs import (WORKLOADS, block_lists, prefill_inputs,
                                                     sample_rows, seeded_normal)
from test_gpu_parity import DEV, announce, arbitrary_block_lists

pytestmark = pytest.mark.gpu

MAX_REL, NORM_REL = 2e-2, 1e-2
# fp32 inputs (general kernel, fp32 throughout): the forward's fp32 bound
MAX_REL_F32, NORM_REL_F32 = 1e-3, 1e-4


def close(name, got, ref, floor=0.0, max_rel=MAX_REL, norm_rel=NORM_REL):
    """Max and normwise error relative to the reference; ``floor`` stands in
    for max|ref| when the exact gradient vanishes (fp32 rounding of the
    dP - D difference then decides the result)."""
    err = np.abs(got - ref)
    scale = max(float(np.abs(ref).max()), floor, 1e-30)
    assert err.max() <= max_rel * scale, f"{name}: max err {err.max():.3e} vs {scale:.3e}"
    nr = max(float(np.linalg.norm(ref)), floor * math.sqrt(ref.size), 1e-30)
    assert np.linalg.norm(err) <= norm_rel * nr, f"{name}: normwise {np.linalg.norm(err) / nr:.3e}"


def rounding_floor(q, k, v, dout, scale):
    """2^-23-sized bound of the fp32 rounding in one gradient entry: d terms of
    the largest |dO| |v| |k| (or |q|) products."""
    d = q.shape[-1]
    big = max(float(q.abs().max()), float(k.abs().max()))
    return 1.2e-7 * d * float(dout.abs().max()) * float(v.abs().max()) * big * scale


def run_gpu(prob, inp, idx, dout):
    out, lse = pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx)
    dq, dk, dv = pisa_block_sparse_attn_backward(prob, inp.q, inp.k, inp.v, idx, out, lse, dout)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # (N, d, K, Hq, Hkv, causal, lists, dtype, C); bf16 with C = 64 and a
    # power-of-two group runs the MFMA kernel, everything else the general one
    (3000, 128, 8, 2, 1, True, "selector", "bf16", 64),     # ragged last block (56 keys), G = 2
    (4160, 64, 16, 4, 4, True, "selector", "bf16", 64),     # G = 1, d = 64, block 0 in 3 items
    (4160, 128, 16, 16, 1, True, "selector", "bf16", 64),   # G = 16: 128 pairs per item
    (1500, 64, 8, 8, 2, False, "selector", "bf16", 64),     # non-causal, G = 4, unselected blocks
    (2100, 128, 12, 4, 2, True, "arbitrary", "bf16", 64),   # unsorted, junk, future, empty rows
    (700, 64, 5, 2, 2, False, "arbitrary", "bf16", 64),
    (64, 128, 3, 8, 1, True, "selector", "bf16", 64),       # one block
    (1, 64, 3, 2, 1, True, "selector", "bf16", 64),         # one token
    # general kernel
    (2048, 64, 4, 2, 2, True, "selector", "fp32", 64),      # the fp32 workload shape; block 0 in 8 items
    (1000, 128, 5, 6, 2, False, "selector", "fp32", 16),    # C = 16, G = 3, non-causal, ragged
    (3000, 64, 8, 1, 1, True, "selector", "bf16", 32),      # bf16, C = 32
    (2500, 128, 16, 3, 1, True, "selector", "bf16", 64),    # bf16, C = 64, G = 3
    (1300, 64, 6, 4, 4, True, "arbitrary", "fp32", 64),     # caller-style lists on the general kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"N{c[0]}_d{c[1]}_K{c[2]}_G{c[3] // c[4]}_"
                                             f"{'causal' if c[5] else 'full'}_{c[6]}_{c[7]}_C{c[8]}"
                                             for c in CASES])
def test_backward_small(case):
    n, d, k, hq, hkv, causal, kind, dt, c = case
    announce(f"backward {case}")
    dtype = torch.float32 if dt == "fp32" else torch.bfloat16
    prob = Problem(1, hq, hkv, n, d, block=c, topk=k, dtype=dtype, causal=causal,
                   force_first_prev=causal and k >= 3)
    inp = prefill_inputs(1, hq, hkv, n, d, dtype, seed=900 + n, recipe="unit", device=DEV)
    dout = seeded_normal((1, hq, n, d), 905 + n, 1.0, dtype, DEV)
    if kind == "selector":
        idx = block_lists(1, hkv, n, c, k, seed=n, causal=causal, device=DEV)
    else:
        idx = torch.from_numpy(arbitrary_block_lists(n, hkv, k, causal, seed=n + 1)).to(DEV)
    dq, dk, dv = run_gpu(prob, inp, idx, dout)
    g = hq // hkv
    idx_np = idx.cpu().numpy()
    m1 = -(-n // c)
    fl = rounding_floor(inp.q, inp.k, inp.v, dout, prob.logit_scale)
    tol = (dict(max_rel=MAX_REL_F32, norm_rel=NORM_REL_F32) if dtype == torch.float32
           else dict(max_rel=MAX_REL, norm_rel=NORM_REL))
    for h in range(hkv):
        lists = np.where(idx_np[0, h] >= m1, -1, idx_np[0, h])
        rq, rk, rv = oracle.attention_backward(
            parity.to_np(inp.q[0, h * g:(h + 1) * g]), parity.to_np(inp.k[0, h]),
            parity.to_np(inp.v[0, h]), lists, parity.to_np(dout[0, h * g:(h + 1) * g]), c,
            causal, prob.logit_scale)
        close(f"dq h{h}", parity.to_np(dq[0, h * g:(h + 1) * g]), rq, fl, **tol)
        close(f"dk h{h}", parity.to_np(dk[0, h]), rk, fl, **tol)
        close(f"dv h{h}", parity.to_np(dv[0, h]), rv, **tol)
        # keys that no row attends get exact zeros
        seen = np.zeros(n, bool)
        for t in range(n):
            seen[oracle.attended_tokens(lists[t], t, c, n, causal)] = True
        assert np.all(parity.to_np(dk[0, h])[~seen] == 0) and np.all(parity.to_np(dv[0, h])[~seen] == 0)


BATCH_CASES = [
    # (B, N, d, K, Hq, Hkv, dtype, C)
    (2, 1700, 128, 8, 4, 2, "bf16", 64),   # MFMA kernel, batch index in every address
    (3, 900, 64, 6, 2, 2, "fp32", 32),     # general kernel
    (2, 2000, 64, 32, 16, 1, "bf16", 64),  # K = 32 (5 slot bits), G = 16
]


@pytest.mark.parametrize("case", BATCH_CASES, ids=[f"B{c[0]}_N{c[1]}_d{c[2]}_K{c[3]}_"
                                                   f"G{c[4] // c[5]}_{c[6]}_C{c[7]}"
                                                   for c in BATCH_CASES])
def test_backward_batches(case):
    """Several sequences at once: each (batch, KV head) against the oracle."""
    bsz, n, d, k, hq, hkv, dt, c = case
    announce(f"backward batch {case}")
    dtype = torch.float32 if dt == "fp32" else torch.bfloat16
    prob = Problem(bsz, hq, hkv, n, d, block=c, topk=k, dtype=dtype)
    inp = prefill_inputs(bsz, hq, hkv, n, d, dtype, seed=700 + n, recipe="unit", device=DEV)
    dout = seeded_normal((bsz, hq, n, d), 705 + n, 1.0, dtype, DEV)
    idx = block_lists(bsz, hkv, n, c, k, seed=n + 3, device=DEV)
    dq, dk, dv = run_gpu(prob, inp, idx, dout)
    g = hq // hkv
    idx_np = idx.cpu().numpy()
    fl = rounding_floor(inp.q, inp.k, inp.v, dout, prob.logit_scale)
    tol = (dict(max_rel=MAX_REL_F32, norm_rel=NORM_REL_F32) if dtype == torch.float32
           else dict(max_rel=MAX_REL, norm_rel=NORM_REL))
    for b in range(bsz):
        for h in range(hkv):
            rq, rk, rv = oracle.attention_backward(
                parity.to_np(inp.q[b, h * g:(h + 1) * g]), parity.to_np(inp.k[b, h]),
                parity.to_np(inp.v[b, h]), idx_np[b, h], parity.to_np(dout[b, h * g:(h + 1) * g]),
                c, True, prob.logit_scale)
            close(f"dq b{b} h{h}", parity.to_np(dq[b, h * g:(h + 1) * g]), rq, fl, **tol)
            close(f"dk b{b} h{h}", parity.to_np(dk[b, h]), rk, fl, **tol)
            close(f"dv b{b} h{h}", parity.to_np(dv[b, h]), rv, **tol)


def test_backward_is_deterministic():
    """Same inputs twice: bitwise identical gradients (no floating-point atomics)."""
    n, d, k, hq, hkv = 4160, 128, 16, 8, 2
    announce("backward determinism")
    prob = Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16)
    inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=31, device=DEV)
    dout = seeded_normal((1, hq, n, d), 32, 1.0 / math.sqrt(d), torch.bfloat16, DEV)
    idx = block_lists(1, hkv, n, 64, k, seed=33, device=DEV)
    a = run_gpu(prob, inp, idx, dout)
    b = run_gpu(prob, inp, idx, dout)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_workload_128k():
    """The 128K prefill shape (B=1, 4 heads, d=128, K=16, causal) in the launch
    configuration the benchmark times, lists shaped like a selector's."""
    cfg = WORKLOADS["c4b"]
    n, d, k, hq, hkv = cfg["seq_len"], cfg["head_dim"], cfg["topk"], cfg["heads_q"], cfg["heads_kv"]
    announce(f"backward 128K {n} {d} {k} {hq}/{hkv}")
    prob = Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16)
    inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=cfg["seed"], recipe=cfg["recipe"],
                         device=DEV)
    dout = seeded_normal((1, hq, n, d), cfg["seed"] + 5, 1.0 / math.sqrt(d), torch.bfloat16, DEV)
    idx = block_lists(1, hkv, n, 64, k, seed=cfg["seed"] + 6, device=DEV)
    dq, dk, dv = run_gpu(prob, inp, idx, dout)
    idx_np = idx.cpu().numpy()
    m1 = n // 64
    rows = sample_rows(n, 64, k, 24, seed=7)
    for h in (0, hkv - 1):
        keys, vals = parity.to_np(inp.k[0, h]), parity.to_np(inp.v[0, h])
        qg = parity.to_np(inp.q[0, h:h + 1])
        dog = parity.to_np(dout[0, h:h + 1])
        gq = parity.to_np(dq[0, h:h + 1])
        ref = np.stack([oracle.attend_row_grad(qg[:, t], keys, vals, idx_np[0, h, t], t, 64,
                                               dog[:, t], True, prob.logit_scale)[1][0]
                        for t in rows])
        close(f"dq rows h{h}", gq[0, rows], ref)
        gk, gv = parity.to_np(dk[0, h]), parity.to_np(dv[0, h])
        for blk in (1, 9, m1 // 2, m1 - 2, m1 - 1):
            rk, rv = oracle.key_block_grad(qg, keys, vals, idx_np[0, h], dog, blk, 64, True,
                                           prob.logit_scale)
            close(f"dk block {blk} h{h}", gk[blk * 64:(blk + 1) * 64], rk)
            close(f"dv block {blk} h{h}", gv[blk * 64:(blk + 1) * 64], rv)
        # identities over the whole head (every row attends its own block)
        sdv, sdo = gv.sum(axis=0), dog.sum(axis=(0, 1))
        assert np.linalg.norm(sdv - sdo) <= 1e-2 * np.linalg.norm(sdo)
        per_row = np.sum(gq[0] * qg[0], axis=1)
        lhs, rhs = per_row.sum(), np.sum(gk * keys)
        assert abs(lhs - rhs) <= 1e-2 * np.abs(per_row).sum(), (lhs, rhs)
