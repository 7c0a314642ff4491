"""The library's launch sequences under HIP graph capture (needs an MI355X).

A caller that captures a prefill (pyramid, two-stage selection, block-sparse
attention) or a decode step (pyramid upkeep for the appended token, then the
step) into a graph and replays it must get what the eager calls give, bit for
bit: the library allocates nothing, clears its workspaces with its own kernels
and never waits on the host.  Each graph is replayed several times, with
eager work and synchronisations between the replays; before every prefill
replay its outputs are overwritten, and the decode graph reads new cache
lengths at every replay, as a serving loop would."""
import pytest
import torch

from hierarchical_block_selection_amd import (Problem, pisa_block_sparse_attn, pisa_build_pyramid,
                                              pisa_decode_step, pisa_pyramid_append,
                                              pisa_pyramid_layout, pisa_select,
                                              pisa_workspace_bytes)
from hierarchical_block_selection_amd.inputs import decode_inputs, prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    """torch's capture recipe: one warm-up call on a side stream, then the
    captured call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_graph_replays_equal_eager():
    n, h, d, k = 16384, 4, 128, 16
    prob = Problem(1, h, h, n, d, block=64, topk=k, dtype=torch.bfloat16)
    print(f"[case] prefill graph N={n} H={h} d={d} K={k}", flush=True)
    inp = prefill_inputs(1, h, h, n, d, torch.bfloat16, seed=8401, recipe="unit", device=DEV)
    rows = pisa_pyramid_layout(n, 64)[-1]
    pyr = torch.empty((1, h, rows, d), dtype=torch.float32, device=DEV)
    idx = torch.empty((1, h, n, k), dtype=torch.int32, device=DEV)
    score = torch.empty((1, h, n, k), dtype=torch.float32, device=DEV)
    out = torch.empty_like(inp.q)
    lse = torch.empty((1, h, n), dtype=torch.float32, device=DEV)
    ws_sel = torch.empty(pisa_workspace_bytes(prob, "select"), dtype=torch.uint8, device=DEV)
    ws_att = torch.empty(pisa_workspace_bytes(prob, "attn"), dtype=torch.uint8, device=DEV)

    def run():
        pisa_build_pyramid(prob, inp.k, pyr)
        pisa_select(prob, inp.q, inp.k, pyr, idx, score, strategy="two_stage", workspace=ws_sel)
        pisa_block_sparse_attn(prob, inp.q, inp.k, inp.v, idx, out, lse, workspace=ws_att)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (pyr, idx, score, out, lse)]
    g = _capture(run)
    for rep in range(3):
        pyr.fill_(float("nan"))
        idx.fill_(-7)
        score.fill_(float("nan"))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws_sel.fill_(0xA5)
        ws_att.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("pyramid", "block_idx", "block_score", "out", "row_lse"),
                                   (pyr, idx, score, out, lse), ref):
            assert torch.equal(got, want), (rep, name)
        # eager work between replays, on buffers of its own
        i2, _ = pisa_select(prob, inp.q, inp.k, ref[0])
        torch.cuda.synchronize()
        assert torch.equal(i2, ref[1])


def test_decode_graph_replays_follow_cache_lengths():
    cap, bsz, hq, hkv, d, k = 8192, 2, 8, 2, 128, 16
    start = [1000, 4090]
    prob = Problem(bsz, hq, hkv, cap, d, block=64, topk=k, dtype=torch.bfloat16)
    print(f"[case] decode graph B={bsz} H={hq}/{hkv} cap={cap} d={d} K={k}", flush=True)
    inp = decode_inputs(bsz, hq, hkv, cap, d, torch.bfloat16, seed=8402, recipe="unit",
                        cache_len=start, device=DEV)
    assert pisa_workspace_bytes(prob, "decode") == 0
    full = pisa_build_pyramid(prob, inp.k_cache)
    torch.cuda.synchronize()
    state = {}
    for side in ("graph", "eager"):
        state[side] = dict(
            pyr=full.clone(), lens=torch.tensor(start, dtype=torch.int32, device=DEV),
            idx=torch.empty((bsz, hkv, k), dtype=torch.int32, device=DEV),
            score=torch.empty((bsz, hkv, k), dtype=torch.float32, device=DEV),
            out=torch.empty_like(inp.q),
            lse=torch.empty((bsz, hq), dtype=torch.float32, device=DEV))

    def step(s):
        pisa_pyramid_append(prob, s["lens"], inp.k_cache, s["pyr"])
        pisa_decode_step(prob, s["lens"], inp.q, inp.k_cache, inp.v_cache, s["pyr"], s["idx"],
                         s["score"], s["out"], s["lse"])

    g = _capture(lambda: step(state["graph"]))
    step(state["eager"])  # the same history as the graph side's warm-up call
    torch.cuda.synchronize()
    for rep in range(4):
        for s in state.values():
            s["lens"] += 1 + 37 * rep  # crosses leaf boundaries on later replays
        torch.cuda.synchronize()
        g.replay()
        step(state["eager"])
        torch.cuda.synchronize()
        for key in ("pyr", "idx", "score", "out", "lse"):
            assert torch.equal(state["graph"][key], state["eager"][key]), (rep, key)
    assert int((state["graph"]["idx"] >= 0).sum()) > 0
