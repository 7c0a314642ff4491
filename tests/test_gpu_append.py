"""Pyramid cache upkeep for decode, pisa_pyramid_append (needs an MI355X).

The rows on the path of token n - 1 must equal, bit for bit, the rows that
pisa_build_pyramid writes for a sequence of n tokens (same arithmetic), and
the oracle's pyramid over the first n keys within fp32 rounding; rows off the
path must not change.  A sequence of appends followed by a decode step must
give exactly the decode step of a pyramid built over the whole cache, because
a decode step never ranks a node on the current path.
"""
import numpy as np
import pytest
import torch

import oracle
import parity
from hierarchical_block_selection_amd import (Problem, pisa_build_pyramid, pisa_decode_step,
                                              pisa_pyramid_append, pisa_pyramid_layout)
from hierarchical_block_selection_amd.inputs import decode_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # (dtype, d, C)
    (torch.bfloat16, 128, 64),
    (torch.bfloat16, 64, 16),
    (torch.float32, 128, 32),
    (torch.float32, 64, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{'bf16' if c[0] == torch.bfloat16 else 'f32'}"
                                             f"_d{c[1]}_C{c[2]}" for c in CASES])
def test_append_matches_prefix_pyramid(case):
    dtype, d, c = case
    cap, hkv = 4096, 2
    lens = [1, c - 1, c, c + 1, 2000, 3 * c + 5, cap]
    bsz = len(lens)
    print(f"[case] append {case}", flush=True)
    prob = Problem(bsz, hkv, hkv, cap, d, block=c, topk=8, dtype=dtype)
    inp = decode_inputs(bsz, hkv, hkv, cap, d, dtype, seed=61 + c + d, recipe="unit",
                        cache_len=lens, device=DEV)
    base = pisa_build_pyramid(prob, inp.k_cache)
    pyr = base.clone()
    pisa_pyramid_append(prob, inp.cache_len, inp.k_cache, pyr)
    torch.cuda.synchronize()
    offs = pisa_pyramid_layout(cap, c)
    n_levels = len(offs) - 1
    for b, n in enumerate(lens):
        pn = Problem(1, hkv, hkv, n, d, block=c, topk=8, dtype=dtype)
        ref = pisa_build_pyramid(pn, inp.k_cache[b:b + 1, :, :n].contiguous())
        torch.cuda.synchronize()
        offs_n = pisa_pyramid_layout(n, c)
        leaf = (n - 1) // c
        path = set()
        for h in range(hkv):
            keys = parity.to_np(inp.k_cache[b, h, :n])
            want = oracle.build_pyramid(keys, c)
            tol = 4e-6 * max(np.abs(keys).max(), 1e-30)
            for lvl in range(n_levels):
                node = leaf >> lvl
                row = offs[lvl] + node
                path.add(row)
                # above the n-token pyramid's root the path nodes equal that root
                lvl_n = min(lvl, len(offs_n) - 2)
                row_n = offs_n[lvl_n] + (leaf >> lvl_n)
                assert torch.equal(pyr[b, h, row], ref[0, h, row_n]), (b, h, lvl)
                got = parity.to_np(pyr[b, h, row])
                assert np.max(np.abs(got - want[lvl_n][leaf >> lvl_n])) <= tol, (b, h, lvl)
        others = [r for r in range(offs[-1]) if r not in path]
        assert torch.equal(pyr[b][:, others], base[b][:, others]), b


def test_append_sequence_then_decode():
    """70 single-token appends (crossing leaf and level-2 boundaries) from two
    starting lengths, then one decode step."""
    cap, bsz, hq, hkv, d, c, k = 8192, 2, 8, 2, 128, 64, 16
    start = [1000, 4090]
    print("[case] append sequence + decode", flush=True)
    prob = Problem(bsz, hq, hkv, cap, d, block=c, topk=k, dtype=torch.bfloat16)
    inp = decode_inputs(bsz, hq, hkv, cap, d, torch.bfloat16, seed=71, recipe="unit",
                        cache_len=start, device=DEV)
    full = pisa_build_pyramid(prob, inp.k_cache)
    pyr = full.clone()
    lens = torch.tensor(start, dtype=torch.int32, device=DEV)
    for _ in range(70):
        lens += 1
        pisa_pyramid_append(prob, lens, inp.k_cache, pyr)
    torch.cuda.synchronize()
    offs = pisa_pyramid_layout(cap, c)
    for b in range(bsz):
        n = int(lens[b])
        pn = Problem(1, hkv, hkv, n, d, block=c, topk=k, dtype=torch.bfloat16)
        ref = pisa_build_pyramid(pn, inp.k_cache[b:b + 1, :, :n].contiguous())
        torch.cuda.synchronize()
        offs_n = pisa_pyramid_layout(n, c)
        # every row of the n-token pyramid sits at the same node index in the
        # capacity layout
        for lvl in range(len(offs_n) - 1):
            m = offs_n[lvl + 1] - offs_n[lvl]
            assert torch.equal(pyr[b, :, offs[lvl]:offs[lvl] + m],
                               ref[0, :, offs_n[lvl]:offs_n[lvl] + m]), (b, lvl)
    r1 = pisa_decode_step(prob, lens, inp.q, inp.k_cache, inp.v_cache, pyr)
    r2 = pisa_decode_step(prob, lens, inp.q, inp.k_cache, inp.v_cache, full)
    torch.cuda.synchronize()
    for a, bb in zip(r1, r2):
        assert torch.equal(a, bb)
