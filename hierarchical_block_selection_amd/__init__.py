"""PISA on MI355X (gfx950): Python binding of libpisa's C ABI.

Every function here only marshals arguments (tensor pointers, sizes, the
current HIP stream) into the C entry point of the same name; all computation
runs in the library's HIP kernels.  PyTorch provides device memory and streams.
There is no CPU fallback: without the built library every call raises.

Entry points (see include/pisa.h for layouts and semantics):
  pisa_build_pyramid, pisa_select, pisa_select_noalloc, pisa_bsa_select,
  pisa_block_sparse_attn, pisa_block_sparse_attn_backward, pisa_pyramid_append,
  pisa_decode_step, plus pisa_pyramid_layout and pisa_workspace_bytes.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import PisaError  # noqa: F401

__all__ = [
    "Problem", "PisaError", "pisa_pyramid_layout", "pisa_workspace_bytes", "pisa_build_pyramid",
    "pisa_select", "pisa_select_noalloc", "pisa_bsa_select", "pisa_block_sparse_attn",
    "pisa_block_sparse_attn_backward", "pisa_pyramid_append", "pisa_decode_step",
    "pisa_profile_enable", "pisa_profile_report",
]

_DTYPES = {torch.float32: _lib.PISA_F32, torch.bfloat16: _lib.PISA_BF16}
_STRATEGIES = {"auto": _lib.PISA_SELECT_AUTO, "fused": _lib.PISA_SELECT_FUSED,
               "two_stage": _lib.PISA_SELECT_TWO_STAGE}
_SCORES = {"lse": 0, "mean": _lib.PISA_SCORE_MEAN, "mean_var": _lib.PISA_SCORE_MEAN_VAR}
_OPS = {"pyramid": _lib.PISA_OP_PYRAMID, "select": _lib.PISA_OP_SELECT, "bsa": _lib.PISA_OP_BSA,
        "attn": _lib.PISA_OP_ATTN, "decode": _lib.PISA_OP_DECODE,
        "attn_bwd": _lib.PISA_OP_ATTN_BWD}


@dataclass
class Problem:
    """Problem sizes and policy (the C struct pisa_problem)."""
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    block: int = 64
    topk: int = 16
    branch: int = 2
    causal: bool = True
    force_first_prev: bool = True
    dtype: torch.dtype = torch.bfloat16
    scale: float = 0.0  # <= 0 -> 1/sqrt(head_dim)
    score: str = "lse"  # "lse" (eq. 7), "mean" (PISA-1) or "mean_var" (PISA-2)

    def to_c(self) -> _lib.PisaProblem:
        if self.dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {self.dtype}")
        if self.score not in _SCORES:
            raise ValueError(f"unknown score {self.score!r}")
        flags = (_lib.PISA_CAUSAL if self.causal else 0) | (
            _lib.PISA_FORCE_FIRST_PREV if self.force_first_prev else 0) | _SCORES[self.score]
        return _lib.PisaProblem(self.batch, self.heads_q, self.heads_kv, self.seq_len,
                                self.head_dim, self.block, self.topk, self.branch, flags,
                                _DTYPES[self.dtype], float(self.scale))

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def logit_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)


def pisa_pyramid_layout(seq_len: int, block: int, branch: int = 2) -> list[int]:
    """Row offsets of every pyramid level plus the total row count R (last entry)."""
    lib = _lib.load()
    offs = (ctypes.c_int64 * (_lib.PISA_MAX_LEVELS + 1))()
    n = ctypes.c_int32()
    _lib.check("pisa_pyramid_layout",
               lib.pisa_pyramid_layout(seq_len, block, branch, ctypes.byref(n), offs,
                                       _lib.PISA_MAX_LEVELS + 1))
    return [int(offs[i]) for i in range(n.value + 1)]


def pisa_workspace_bytes(problem: Problem, op: str) -> int:
    lib = _lib.load()
    c = problem.to_c()
    out = ctypes.c_size_t()
    _lib.check("pisa_workspace_bytes", lib.pisa_workspace_bytes(ctypes.byref(c), _OPS[op], ctypes.byref(out)))
    return out.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _workspace(problem, op, workspace, device):
    need = pisa_workspace_bytes(problem, op)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace, workspace.numel() * workspace.element_size()


def pyramid_rows(problem: Problem) -> int:
    return pisa_pyramid_layout(problem.seq_len, problem.block, problem.branch)[-1]


def pisa_build_pyramid(problem: Problem, k, pyramid=None, stream=None):
    """[B, Hkv, N, d] keys -> [B, Hkv, R, d] float32 pyramid (all levels)."""
    p = problem
    _need(k, "k", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    rows = pyramid_rows(p)
    if pyramid is None:
        pyramid = torch.empty((p.batch, p.heads_kv, rows, p.head_dim), dtype=torch.float32,
                              device=k.device)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, rows, p.head_dim), torch.float32)
    c = p.to_c()
    _lib.check("pisa_build_pyramid", _lib.load().pisa_build_pyramid(
        ctypes.byref(c), _ptr(k), _ptr(pyramid), _stream(stream)))
    return pyramid


def pisa_select(problem: Problem, q, k, pyramid, block_idx=None, block_score=None,
                strategy: str = "auto", workspace=None, stream=None, want_score=True):
    """PISA Top-K selection -> (block_idx [B,Hkv,N,K] int32, block_score or None)."""
    p = problem
    _need(q, "q", (p.batch, p.heads_q, p.seq_len, p.head_dim), p.dtype)
    _need(k, "k", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, pyramid_rows(p), p.head_dim), torch.float32)
    shape = (p.batch, p.heads_kv, p.seq_len, p.topk)
    if block_idx is None:
        block_idx = torch.empty(shape, dtype=torch.int32, device=q.device)
    _need(block_idx, "block_idx", shape, torch.int32)
    if block_score is None and want_score:
        block_score = torch.empty(shape, dtype=torch.float32, device=q.device)
    if block_score is not None:
        _need(block_score, "block_score", shape, torch.float32)
    ws, ws_bytes = _workspace(p, "select", workspace, q.device)
    c = p.to_c()
    _lib.check("pisa_select", _lib.load().pisa_select(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(pyramid), _ptr(block_idx), _ptr(block_score),
        _STRATEGIES[strategy], _ptr(ws), ws_bytes, _stream(stream)))
    return block_idx, block_score


def pisa_select_noalloc(problem: Problem, q, k, pyramid, block_idx=None, block_score=None,
                        strategy: str = "auto", stream=None, want_score=True):
    """pisa_select without a workspace: the library's fixed device scratch
    (PISA_NOALLOC_SCRATCH_BYTES) serves the two-stage selector.  Outputs are
    allocated here when not given; the library call itself allocates nothing."""
    p = problem
    _need(q, "q", (p.batch, p.heads_q, p.seq_len, p.head_dim), p.dtype)
    _need(k, "k", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, pyramid_rows(p), p.head_dim), torch.float32)
    shape = (p.batch, p.heads_kv, p.seq_len, p.topk)
    if block_idx is None:
        block_idx = torch.empty(shape, dtype=torch.int32, device=q.device)
    _need(block_idx, "block_idx", shape, torch.int32)
    if block_score is None and want_score:
        block_score = torch.empty(shape, dtype=torch.float32, device=q.device)
    if block_score is not None:
        _need(block_score, "block_score", shape, torch.float32)
    c = p.to_c()
    _lib.check("pisa_select_noalloc", _lib.load().pisa_select_noalloc(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(pyramid), _ptr(block_idx), _ptr(block_score),
        _STRATEGIES[strategy], _stream(stream)))
    return block_idx, block_score


def pisa_bsa_select(problem: Problem, q, pyramid, block_idx=None, block_score=None,
                    workspace=None, stream=None, want_score=True):
    """BSA flat selection -> (block_idx, block_score or None)."""
    p = problem
    _need(q, "q", (p.batch, p.heads_q, p.seq_len, p.head_dim), p.dtype)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, pyramid_rows(p), p.head_dim), torch.float32)
    shape = (p.batch, p.heads_kv, p.seq_len, p.topk)
    if block_idx is None:
        block_idx = torch.empty(shape, dtype=torch.int32, device=q.device)
    _need(block_idx, "block_idx", shape, torch.int32)
    if block_score is None and want_score:
        block_score = torch.empty(shape, dtype=torch.float32, device=q.device)
    if block_score is not None:
        _need(block_score, "block_score", shape, torch.float32)
    ws, ws_bytes = _workspace(p, "bsa", workspace, q.device)
    c = p.to_c()
    _lib.check("pisa_bsa_select", _lib.load().pisa_bsa_select(
        ctypes.byref(c), _ptr(q), _ptr(pyramid), _ptr(block_idx), _ptr(block_score), _ptr(ws),
        ws_bytes, _stream(stream)))
    return block_idx, block_score


def pisa_block_sparse_attn(problem: Problem, q, k, v, block_idx, out=None, row_lse=None,
                           workspace=None, stream=None, want_lse=True):
    """Attention over the selected blocks -> (out [B,Hq,N,d], row_lse [B,Hq,N] or None)."""
    p = problem
    _need(q, "q", (p.batch, p.heads_q, p.seq_len, p.head_dim), p.dtype)
    _need(k, "k", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(v, "v", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(block_idx, "block_idx", (p.batch, p.heads_kv, p.seq_len, p.topk), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", tuple(q.shape), p.dtype)
    if row_lse is None and want_lse:
        row_lse = torch.empty((p.batch, p.heads_q, p.seq_len), dtype=torch.float32, device=q.device)
    if row_lse is not None:
        _need(row_lse, "row_lse", (p.batch, p.heads_q, p.seq_len), torch.float32)
    ws, ws_bytes = _workspace(p, "attn", workspace, q.device)
    c = p.to_c()
    _lib.check("pisa_block_sparse_attn", _lib.load().pisa_block_sparse_attn(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(row_lse),
        _ptr(ws), ws_bytes, _stream(stream)))
    return out, row_lse


def pisa_block_sparse_attn_backward(problem: Problem, q, k, v, block_idx, out, row_lse, dout,
                                    dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of the block-sparse attention with block_idx held fixed ->
    (dq [B,Hq,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]).  out and row_lse are the
    forward's outputs for these inputs."""
    p = problem
    _need(q, "q", (p.batch, p.heads_q, p.seq_len, p.head_dim), p.dtype)
    _need(k, "k", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(v, "v", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(block_idx, "block_idx", (p.batch, p.heads_kv, p.seq_len, p.topk), torch.int32)
    _need(out, "out", tuple(q.shape), p.dtype)
    _need(row_lse, "row_lse", (p.batch, p.heads_q, p.seq_len), torch.float32)
    _need(dout, "dout", tuple(q.shape), p.dtype)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", tuple(q.shape), p.dtype)
    _need(dk, "dk", tuple(k.shape), p.dtype)
    _need(dv, "dv", tuple(v.shape), p.dtype)
    ws, ws_bytes = _workspace(p, "attn_bwd", workspace, q.device)
    c = p.to_c()
    _lib.check("pisa_block_sparse_attn_backward", _lib.load().pisa_block_sparse_attn_backward(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(out), _ptr(row_lse),
        _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, _stream(stream)))
    return dq, dk, dv


def pisa_pyramid_append(problem: Problem, cache_len, k_cache, pyramid, stream=None):
    """Rewrite the pyramid rows on the path of token cache_len[b] - 1 (already in
    k_cache) to those of the pyramid over cache_len[b] tokens; in place."""
    p = problem
    _need(cache_len, "cache_len", (p.batch,), torch.int32)
    _need(k_cache, "k_cache", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, pyramid_rows(p), p.head_dim), torch.float32)
    c = p.to_c()
    _lib.check("pisa_pyramid_append", _lib.load().pisa_pyramid_append(
        ctypes.byref(c), _ptr(cache_len), _ptr(k_cache), _ptr(pyramid), _stream(stream)))
    return pyramid


def pisa_decode_step(problem: Problem, cache_len, q, k_cache, v_cache, pyramid, block_idx=None,
                     block_score=None, out=None, row_lse=None, workspace=None, stream=None):
    """One decode step -> (block_idx [B,Hkv,K], block_score, out [B,Hq,d], row_lse [B,Hq])."""
    p = problem
    _need(cache_len, "cache_len", (p.batch,), torch.int32)
    _need(q, "q", (p.batch, p.heads_q, p.head_dim), p.dtype)
    _need(k_cache, "k_cache", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(v_cache, "v_cache", (p.batch, p.heads_kv, p.seq_len, p.head_dim), p.dtype)
    _need(pyramid, "pyramid", (p.batch, p.heads_kv, pyramid_rows(p), p.head_dim), torch.float32)
    dev = q.device
    if block_idx is None:
        block_idx = torch.empty((p.batch, p.heads_kv, p.topk), dtype=torch.int32, device=dev)
    _need(block_idx, "block_idx", (p.batch, p.heads_kv, p.topk), torch.int32)
    if block_score is None:
        block_score = torch.empty((p.batch, p.heads_kv, p.topk), dtype=torch.float32, device=dev)
    _need(block_score, "block_score", (p.batch, p.heads_kv, p.topk), torch.float32)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", tuple(q.shape), p.dtype)
    if row_lse is None:
        row_lse = torch.empty((p.batch, p.heads_q), dtype=torch.float32, device=dev)
    _need(row_lse, "row_lse", (p.batch, p.heads_q), torch.float32)
    ws, ws_bytes = _workspace(p, "decode", workspace, dev)
    c = p.to_c()
    _lib.check("pisa_decode_step", _lib.load().pisa_decode_step(
        ctypes.byref(c), _ptr(cache_len), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pyramid),
        _ptr(block_idx), _ptr(block_score), _ptr(out), _ptr(row_lse), _ptr(ws), ws_bytes,
        _stream(stream)))
    return block_idx, block_score, out, row_lse


def pisa_profile_enable(enable: bool = True) -> None:
    """Start (or stop) recording HIP events around every library kernel launch."""
    _lib.check("pisa_profile_enable", _lib.load().pisa_profile_enable(1 if enable else 0))


def pisa_profile_report(max_kernels: int = 64) -> dict:
    """Wait for the recorded launches and return {kernel: (total_ms, launches)}."""
    lib = _lib.load()
    names = ctypes.create_string_buffer(8192)
    tot = (ctypes.c_float * max_kernels)()
    cnt = (ctypes.c_int32 * max_kernels)()
    n = ctypes.c_int32()
    _lib.check("pisa_profile_report",
               lib.pisa_profile_report(names, len(names), tot, cnt, max_kernels, ctypes.byref(n)))
    keys = names.value.decode().split("\n")[:min(n.value, max_kernels)]
    return {k: (float(tot[i]), int(cnt[i])) for i, k in enumerate(keys)}
