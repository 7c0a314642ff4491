"""Seeded synthetic inputs for PISA workloads.

This module holds no part of the selection or attention arithmetic; it only
draws tensors.  Both the HIP path's tests/benchmarks and the CPU oracle take
their inputs from here.

Shapes follow the library's layout: Q [B, Hq, N, d], K/V [B, Hkv, N, d];
decode: q [B, Hq, d], caches [B, Hkv, capacity, d], cache_len [B].

Value recipes:
  * "inv_sqrt_d": i.i.d. N(0, 1/d) entries (random long-context prefill);
  * "unit":       i.i.d. N(0, 1) entries (larger logit spread, fewer near-ties);
  * "wide_q":     queries N(0, 64), keys and values N(0, 1): logits of standard
                  deviation 8, peaked attention and large group-summed scores.
Planted needles (per KV head): ``n_needles`` distinct leaf blocks b drawn from
[1, M_1 - 3]; for each a target row r from [(b + 2) C, N); the block's keys are
replaced by alpha * q_r / |q_r| + fresh noise of the recipe's scale, where q_r
is the first query head of the group at row r.

Seeds: tensor seeds are seed+0 (Q), seed+1 (K), seed+2 (V), seed+3 (needle
positions, CPU generator), seed+4 (needle noise).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


def _sigma(recipe: str, head_dim: int) -> float:
    """Standard deviation of the keys and values (and of the queries unless
    _sigma_q says otherwise)."""
    if recipe == "inv_sqrt_d":
        return 1.0 / math.sqrt(head_dim)
    if recipe in ("unit", "wide_q"):
        return 1.0
    raise ValueError(f"unknown value recipe {recipe!r}")


def _sigma_q(recipe: str, head_dim: int) -> float:
    return 8.0 if recipe == "wide_q" else _sigma(recipe, head_dim)


def seeded_normal(shape, seed: int, sigma: float, dtype: torch.dtype, device) -> torch.Tensor:
    """N(0, sigma^2) tensor drawn in fp32 from a generator seeded with ``seed``,
    then cast.  Large tensors are drawn slice by slice along dim 0 from the
    same generator, so the values do not depend on available memory."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        x = torch.randn(shape[1:], generator=gen, dtype=torch.float32, device=device)
        out[b] = (x * sigma).to(dtype)
    return out


@dataclass
class Needle:
    batch: int
    kv_head: int
    block: int
    target_row: int


@dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    needles: list = field(default_factory=list)


def prefill_inputs(batch, heads_q, heads_kv, seq_len, head_dim, dtype=torch.bfloat16,
                   seed=0, recipe="inv_sqrt_d", n_needles=0, alpha=4.0, block=64,
                   device="cpu") -> PrefillInputs:
    sigma = _sigma(recipe, head_dim)
    q = seeded_normal((batch, heads_q, seq_len, head_dim), seed + 0, _sigma_q(recipe, head_dim),
                      dtype, device)
    k = seeded_normal((batch, heads_kv, seq_len, head_dim), seed + 1, sigma, dtype, device)
    v = seeded_normal((batch, heads_kv, seq_len, head_dim), seed + 2, sigma, dtype, device)
    needles = []
    if n_needles:
        n_leaves = -(-seq_len // block)
        if n_leaves - 3 < n_needles:
            raise ValueError("sequence too short for the requested needles")
        pos_gen = torch.Generator().manual_seed(seed + 3)
        noise_gen = torch.Generator(device=device).manual_seed(seed + 4)
        group = heads_q // heads_kv
        for b in range(batch):
            for h in range(heads_kv):
                blocks = (torch.randperm(n_leaves - 3, generator=pos_gen)[:n_needles] + 1).tolist()
                for blk in blocks:
                    lo = (blk + 2) * block
                    r = int(torch.randint(lo, seq_len, (1,), generator=pos_gen))
                    qr = q[b, h * group, r].to(torch.float32)
                    u = qr / qr.norm()
                    rows = min(block, seq_len - blk * block)
                    noise = torch.randn((rows, head_dim), generator=noise_gen,
                                        dtype=torch.float32, device=device) * sigma
                    k[b, h, blk * block:blk * block + rows] = (alpha * u + noise).to(dtype)
                    needles.append(Needle(b, h, blk, r))
    return PrefillInputs(q, k, v, needles)


@dataclass
class DecodeInputs:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    cache_len: torch.Tensor


def decode_inputs(batch, heads_q, heads_kv, capacity, head_dim, dtype=torch.bfloat16,
                  seed=0, recipe="inv_sqrt_d", cache_len=None, device="cpu") -> DecodeInputs:
    """One new query token per sequence plus a filled KV cache.

    ``cache_len``: None (every sequence full), an int, or a list of B ints.
    """
    sigma = _sigma(recipe, head_dim)
    q = seeded_normal((batch, heads_q, head_dim), seed + 0, _sigma_q(recipe, head_dim), dtype,
                      device)
    kc = seeded_normal((batch, heads_kv, capacity, head_dim), seed + 1, sigma, dtype, device)
    vc = seeded_normal((batch, heads_kv, capacity, head_dim), seed + 2, sigma, dtype, device)
    if cache_len is None:
        lens = [capacity] * batch
    elif isinstance(cache_len, int):
        lens = [cache_len] * batch
    else:
        lens = list(cache_len)
    if len(lens) != batch or min(lens) < 1 or max(lens) > capacity:
        raise ValueError("cache_len must hold B values in [1, capacity]")
    return DecodeInputs(q, kc, vc, torch.tensor(lens, dtype=torch.int32, device=device))


def block_lists(batch, heads_kv, seq_len, block, topk, seed, causal=True, device="cpu"):
    """Leaf lists shaped like a selector's output, for the attention and its
    backward when the lists are an input: [B, Hkv, N, K] int32, each row
    ascending and padded with -1.  Causal: row t (leaf c = t // C) holds the
    blocks 0, c - 1 and c plus distinct blocks drawn uniformly from [0, c];
    otherwise K distinct blocks from all leaves.  Each row draws 2K candidates
    and keeps the first distinct ones, so a row may hold fewer than
    min(K, eligible) blocks when draws collide."""
    import numpy as np

    n_leaves = -(-seq_len // block)
    rows = batch * heads_kv * seq_len
    rng = np.random.default_rng(seed)
    t = np.tile(np.arange(seq_len), batch * heads_kv)
    cur = t // block
    hi = cur if causal else np.full_like(cur, n_leaves - 1)
    draws = (rng.random((rows, 2 * topk)) * (hi[:, None] + 1)).astype(np.int64)
    if causal:
        forced = np.stack([np.zeros_like(cur), np.maximum(cur - 1, 0), cur], axis=1)
        vals = np.concatenate([forced, draws], axis=1)
    else:
        vals = draws
    width = vals.shape[1]
    pri = np.broadcast_to(np.arange(width), vals.shape)
    order = np.lexsort((pri, vals), axis=1)
    sv = np.take_along_axis(vals, order, axis=1)
    sp = np.take_along_axis(pri, order, axis=1).copy()
    dup = np.zeros_like(sv, dtype=bool)
    dup[:, 1:] = sv[:, 1:] == sv[:, :-1]
    big = width + 1
    sp[dup] = big
    keep = np.argsort(sp, axis=1, kind="stable")[:, :topk]
    kv = np.take_along_axis(sv, keep, axis=1)
    kp = np.take_along_axis(sp, keep, axis=1)
    kv = np.where(kp == big, np.iinfo(np.int64).max, kv)
    kv.sort(axis=1)
    kv[kv == np.iinfo(np.int64).max] = -1
    if kv.shape[1] < topk:
        kv = np.concatenate([kv, np.full((rows, topk - kv.shape[1]), -1)], axis=1)
    out = torch.from_numpy(kv.astype(np.int32)).reshape(batch, heads_kv, seq_len, topk)
    return out.to(device)


# Workload shapes of the five configurations: prefill c1-c4 (c4 sweeps N) and
# the decode step c5.  Sizes only; inputs come from prefill_inputs /
# decode_inputs with the given seed and recipe.
WORKLOADS = {
    "c1": dict(kind="prefill", batch=1, heads_q=2, heads_kv=2, seq_len=2048, head_dim=64,
               block=64, topk=4, dtype=torch.float32, recipe="unit", n_needles=0, seed=1000),
    "c2": dict(kind="prefill", batch=1, heads_q=16, heads_kv=16, seq_len=16384, head_dim=128,
               block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=8,
               seed=2000),
    "c3": dict(kind="prefill", batch=1, heads_q=8, heads_kv=8, seq_len=65536, head_dim=128,
               block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=8,
               seed=3000),
    "c4a": dict(kind="prefill", batch=1, heads_q=4, heads_kv=4, seq_len=32768, head_dim=128,
                block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=0,
                seed=4000),
    "c4b": dict(kind="prefill", batch=1, heads_q=4, heads_kv=4, seq_len=131072, head_dim=128,
                block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=0,
                seed=4010),
    "c4c": dict(kind="prefill", batch=1, heads_q=4, heads_kv=4, seq_len=262144, head_dim=128,
                block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=0,
                seed=4020),
    "c5": dict(kind="decode", batch=32, heads_q=32, heads_kv=8, seq_len=131072, head_dim=128,
               block=64, topk=16, dtype=torch.bfloat16, recipe="inv_sqrt_d", n_needles=0,
               seed=5000),
}


def sample_rows(seq_len: int, block: int, topk: int, n_random: int, seed: int) -> list[int]:
    """Query rows for sampled checks: block edges near the start, around the
    budget boundary K*C, the last rows, plus seeded random rows."""
    fixed = {0, 1, block - 1, block, 2 * block - 1, 2 * block, 3 * block + 5,
             topk * block - 1, topk * block, topk * block + 1, 2 * topk * block + 7,
             seq_len // 2, seq_len - block, seq_len - 2, seq_len - 1}
    gen = torch.Generator().manual_seed(seed)
    rand = torch.randint(0, seq_len, (n_random,), generator=gen).tolist()
    return sorted(r for r in fixed | set(rand) if 0 <= r < seq_len)
