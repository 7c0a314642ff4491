"""pisa_select_noalloc against pisa_select (needs an MI355X).

The entry point for callers that cannot allocate runs the same kernels on the
library's fixed device scratch instead of a caller workspace, so its outputs
must equal pisa_select's bit for bit.  Two calls in a row, the second on a
smaller problem of another shape (the scratch keeps the first call's contents),
then the first problem again."""
import pytest
import torch

from hierarchical_block_selection_amd import (Problem, pisa_build_pyramid, pisa_select,
                                              pisa_select_noalloc, pisa_workspace_bytes)
from hierarchical_block_selection_amd._lib import PISA_NOALLOC_SCRATCH_BYTES
from hierarchical_block_selection_amd.inputs import prefill_inputs

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Hq, Hkv, N, d, K, seed)
    (1, 4, 4, 16384, 128, 16, 8301),
    (1, 8, 2, 8192, 64, 8, 8302),
]


def _run(case):
    b, hq, hkv, n, d, k, seed = case
    prob = Problem(b, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16)
    assert 0 < pisa_workspace_bytes(prob, "select") <= PISA_NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc select B={b} H={hq}/{hkv} N={n} d={d} K={k}", flush=True)
    inp = prefill_inputs(b, hq, hkv, n, d, torch.bfloat16, seed=seed, recipe="unit",
                         device="cuda")
    pyr = pisa_build_pyramid(prob, inp.k)
    ref_idx, ref_score = pisa_select(prob, inp.q, inp.k, pyr)
    got_idx, got_score = pisa_select_noalloc(prob, inp.q, inp.k, pyr)
    torch.cuda.synchronize()
    assert torch.equal(got_idx, ref_idx)
    assert torch.equal(got_score, ref_score)
    assert int((got_idx >= 0).sum()) > 0


def test_noalloc_select_equals_select_twice_then_smaller():
    _run(CASES[0])
    _run(CASES[1])
    _run(CASES[0])
