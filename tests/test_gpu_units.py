"""(batch, KV head) units are independent: calls over slices of the KV heads
give bit for bit what one call over all heads gives (needs an MI355X).

This is what lets the work split across devices with no communication: a
device given a subset of the KV heads (and their query heads) computes exactly
its share of the full result.  Checked for the pyramid, the selection, the
attention and its backward, on the fast (bf16) paths.
"""
import math

import pytest
import torch

from hierarchical_block_selection_amd import (Problem, pisa_block_sparse_attn,
                                              pisa_block_sparse_attn_backward,
                                              pisa_build_pyramid, pisa_select)
from hierarchical_block_selection_amd.inputs import prefill_inputs, seeded_normal
from test_gpu_parity import DEV, announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_kv_head_slices_match_one_call(hq, hkv):
    n, d, k = 6000, 128, 16
    announce(f"kv head slices hq={hq} hkv={hkv}")
    g = hq // hkv
    full = Problem(1, hq, hkv, n, d, block=64, topk=k, dtype=torch.bfloat16)
    inp = prefill_inputs(1, hq, hkv, n, d, torch.bfloat16, seed=77, device=DEV)
    dout = seeded_normal((1, hq, n, d), 78, 1.0 / math.sqrt(d), torch.bfloat16, DEV)
    pyr = pisa_build_pyramid(full, inp.k)
    idx, _ = pisa_select(full, inp.q, inp.k, pyr)
    out, lse = pisa_block_sparse_attn(full, inp.q, inp.k, inp.v, idx)
    dq, dk, dv = pisa_block_sparse_attn_backward(full, inp.q, inp.k, inp.v, idx, out, lse, dout)
    torch.cuda.synchronize()
    one = Problem(1, g, 1, n, d, block=64, topk=k, dtype=torch.bfloat16)
    for h in range(hkv):
        qs = inp.q[:, h * g:(h + 1) * g].contiguous()
        ks = inp.k[:, h:h + 1].contiguous()
        vs = inp.v[:, h:h + 1].contiguous()
        p1 = pisa_build_pyramid(one, ks)
        i1, _ = pisa_select(one, qs, ks, p1)
        o1, l1 = pisa_block_sparse_attn(one, qs, ks, vs, i1)
        g1 = pisa_block_sparse_attn_backward(one, qs, ks, vs, i1, o1, l1,
                                             dout[:, h * g:(h + 1) * g].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(p1, pyr[:, h:h + 1])
        assert torch.equal(i1, idx[:, h:h + 1])
        assert torch.equal(o1.view(torch.int16), out[:, h * g:(h + 1) * g].view(torch.int16))
        assert torch.equal(l1, lse[:, h * g:(h + 1) * g])
        assert torch.equal(g1[0].view(torch.int16), dq[:, h * g:(h + 1) * g].view(torch.int16))
        assert torch.equal(g1[1].view(torch.int16), dk[:, h:h + 1].view(torch.int16))
        assert torch.equal(g1[2].view(torch.int16), dv[:, h:h + 1].view(torch.int16))
