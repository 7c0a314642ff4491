"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/pisa.h declares, computes the pyramid layout, sizes workspaces, and
rejects every invalid argument before touching a device."""
import ctypes
import os
import re

import pytest

import oracle
from hierarchical_block_selection_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pisa.h")


def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libpisa.so not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(pisa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("pisa_build_pyramid", "pisa_select", "pisa_bsa_select",
                 "pisa_block_sparse_attn", "pisa_decode_step"):
        assert want in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in declared_functions():
        assert hasattr(L, name), name


@pytest.mark.parametrize("n,c", [(2048, 64), (16384, 64), (65536, 64), (131072, 64),
                                  (262144, 64), (1, 64), (63, 64), (65, 16), (5 * 4 + 3, 4)])
def test_pyramid_layout_matches_eq3(n, c):
    L = lib()
    levels = ctypes.c_int32()
    offs = (ctypes.c_int64 * 33)()
    assert L.pisa_pyramid_layout(n, c, 2, ctypes.byref(levels), offs, 33) == 0
    sizes = oracle.pyramid_level_sizes(n, c)
    assert levels.value == len(sizes)
    acc = 0
    for i, m in enumerate(sizes):
        assert offs[i] == acc
        acc += m
    assert offs[len(sizes)] == acc


def test_pyramid_layout_errors():
    L = lib()
    n = ctypes.c_int32()
    offs = (ctypes.c_int64 * 4)()
    assert L.pisa_pyramid_layout(0, 64, 2, ctypes.byref(n), None, 0) == _lib.PISA_ERR_INVALID
    assert L.pisa_pyramid_layout(100, 64, 3, ctypes.byref(n), None, 0) == _lib.PISA_ERR_INVALID
    # 2048/64 -> 6 levels needs 7 offsets
    assert L.pisa_pyramid_layout(2048, 64, 2, ctypes.byref(n), offs, 4) == _lib.PISA_ERR_INVALID


def problem(**kw):
    base = dict(batch=1, heads_q=4, heads_kv=4, seq_len=4096, head_dim=128, block=64, topk=16,
                branch=2, flags=_lib.PISA_CAUSAL | _lib.PISA_FORCE_FIRST_PREV,
                dtype=_lib.PISA_BF16, scale=0.0)
    base.update(kw)
    return _lib.PisaProblem(**base)


BAD = [
    (dict(batch=0), _lib.PISA_ERR_INVALID),
    (dict(heads_q=6, heads_kv=4), _lib.PISA_ERR_INVALID),
    (dict(seq_len=0), _lib.PISA_ERR_INVALID),
    (dict(topk=0), _lib.PISA_ERR_INVALID),
    (dict(dtype=7), _lib.PISA_ERR_INVALID),
    (dict(flags=_lib.PISA_FORCE_FIRST_PREV), _lib.PISA_ERR_INVALID),
    (dict(flags=16), _lib.PISA_ERR_INVALID),
    (dict(flags=_lib.PISA_CAUSAL | _lib.PISA_SCORE_MEAN | _lib.PISA_SCORE_MEAN_VAR),
     _lib.PISA_ERR_INVALID),
    (dict(scale=float("nan")), _lib.PISA_ERR_INVALID),
    (dict(branch=4), _lib.PISA_ERR_UNSUPPORTED),
    (dict(head_dim=96), _lib.PISA_ERR_UNSUPPORTED),
    (dict(block=128), _lib.PISA_ERR_UNSUPPORTED),
    (dict(topk=33), _lib.PISA_ERR_UNSUPPORTED),
    (dict(topk=2), _lib.PISA_ERR_UNSUPPORTED),
    (dict(heads_q=64, heads_kv=2), _lib.PISA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_invalid_problems_rejected_by_every_entry_point(kw, code):
    L = lib()
    p = problem(**kw)
    dummy = ctypes.create_string_buffer(64)
    ptr = ctypes.cast(dummy, ctypes.c_void_p)
    pp = ctypes.byref(p)
    assert L.pisa_build_pyramid(pp, ptr, ptr, None) == code
    assert L.pisa_select(pp, ptr, ptr, ptr, ptr, ptr, 0, ptr, 1 << 40, None) == code
    assert L.pisa_bsa_select(pp, ptr, ptr, ptr, ptr, ptr, 1 << 40, None) == code
    assert L.pisa_block_sparse_attn(pp, ptr, ptr, ptr, ptr, ptr, ptr, ptr, 1 << 40, None) == code
    assert L.pisa_decode_step(pp, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, 1 << 40,
                              None) == code
    assert L.pisa_pyramid_append(pp, ptr, ptr, ptr, None) == code
    assert L.pisa_block_sparse_attn_backward(pp, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                             ptr, 1 << 40, None) == code
    sz = ctypes.c_size_t()
    assert L.pisa_workspace_bytes(pp, 0, ctypes.byref(sz)) == code
    assert L.pisa_last_error()


def test_null_pointers_and_workspace_rejected():
    L = lib()
    p = problem()
    pp = ctypes.byref(p)
    ptr = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    assert L.pisa_build_pyramid(None, ptr, ptr, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_build_pyramid(pp, None, ptr, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_pyramid_append(pp, None, ptr, ptr, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_pyramid_append(pp, ptr, ptr, None, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_select(pp, None, ptr, ptr, ptr, None, 0, None, 0, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_select(pp, ptr, ptr, ptr, ptr, None, 9, None, 0, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_bsa_select(pp, ptr, ptr, None, None, ptr, 1 << 40, None) == _lib.PISA_ERR_INVALID
    # BSA always needs its score workspace
    sz = ctypes.c_size_t()
    assert L.pisa_workspace_bytes(pp, _lib.PISA_OP_BSA, ctypes.byref(sz)) == 0
    # fp32 scores for every (query, leaf) (+ slack for 16-byte row reads) + three
    # bf16 planes of the leaf summaries
    assert sz.value == 1 * 4 * 4096 * 64 * 4 + 256 + 3 * 1 * 4 * 64 * 128 * 2
    assert L.pisa_bsa_select(pp, ptr, ptr, ptr, None, ptr, sz.value - 1, None) == _lib.PISA_ERR_WORKSPACE
    assert L.pisa_bsa_select(pp, ptr, ptr, ptr, None, None, sz.value, None) == _lib.PISA_ERR_WORKSPACE
    assert L.pisa_block_sparse_attn(pp, ptr, ptr, None, ptr, ptr, None, None, 0, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_decode_step(pp, None, ptr, ptr, ptr, ptr, ptr, None, ptr, None, None, 0,
                              None) == _lib.PISA_ERR_INVALID
    nc = problem(flags=0)
    assert L.pisa_decode_step(ctypes.byref(nc), ptr, ptr, ptr, ptr, ptr, ptr, None, ptr, None,
                              None, 0, None) == _lib.PISA_ERR_INVALID
    # BSA past 4096 leaf blocks: the MFMA path only (bf16, power-of-two
    # group, a multiple of 4 leaf blocks), whose Top-K takes rows in segments
    big = problem(seq_len=64 * 4097)
    assert L.pisa_bsa_select(ctypes.byref(big), ptr, ptr, ptr, None, ptr, 1 << 60,
                             None) == _lib.PISA_ERR_UNSUPPORTED
    long_ok = problem(seq_len=64 * 4100)
    assert L.pisa_workspace_bytes(ctypes.byref(long_ok), _lib.PISA_OP_BSA, ctypes.byref(sz)) == 0
    assert sz.value >= 4 * 64 * 4100 * 4100 * 4
    long_f32 = problem(seq_len=64 * 4100, dtype=_lib.PISA_F32)
    assert L.pisa_workspace_bytes(ctypes.byref(long_f32), _lib.PISA_OP_BSA,
                                  ctypes.byref(sz)) == _lib.PISA_ERR_UNSUPPORTED
    assert L.pisa_workspace_bytes(pp, 99, ctypes.byref(sz)) == _lib.PISA_ERR_INVALID
    assert L.pisa_status_string(_lib.PISA_ERR_WORKSPACE) == b"workspace missing or too small"


def test_misaligned_pointers_rejected():
    """Tensors the kernels access with 16-byte vector loads and stores (Q, K, V,
    O, the pyramid, the caches, the gradients, the workspace) must be 16-byte
    aligned: every entry point refuses an address off that alignment before any
    device call (this runs without a GPU)."""
    L = lib()
    p = problem()
    pp = ctypes.byref(p)
    ok = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    bad = ctypes.c_void_p(4096 + 8)
    inv = _lib.PISA_ERR_INVALID

    def refused(rc):
        return rc == inv and b"aligned" in L.pisa_last_error()

    assert refused(L.pisa_build_pyramid(pp, bad, ok, None))
    assert refused(L.pisa_build_pyramid(pp, ok, bad, None))
    assert refused(L.pisa_select(pp, bad, ok, ok, ok, None, 0, None, 0, None))
    assert refused(L.pisa_select(pp, ok, ok, bad, ok, None, 0, None, 0, None))
    assert refused(L.pisa_select_noalloc(pp, ok, bad, ok, ok, None, 0, None))
    assert refused(L.pisa_bsa_select(pp, bad, ok, ok, None, ok, 1 << 40, None))
    assert refused(L.pisa_block_sparse_attn(pp, ok, ok, bad, ok, ok, None, ok, 1 << 40, None))
    assert refused(L.pisa_block_sparse_attn(pp, ok, ok, ok, ok, bad, None, ok, 1 << 40, None))
    assert refused(L.pisa_block_sparse_attn_backward(pp, ok, ok, ok, ok, ok, ok, ok, ok, bad, ok,
                                                     ok, 1 << 40, None))
    assert refused(L.pisa_pyramid_append(pp, ok, bad, ok, None))
    assert refused(L.pisa_decode_step(pp, ok, ok, ok, ok, bad, ok, None, ok, None, ok, 1 << 40,
                                      None))
    # the workspace too
    sz = ctypes.c_size_t()
    assert L.pisa_workspace_bytes(pp, _lib.PISA_OP_ATTN, ctypes.byref(sz)) == 0
    assert sz.value > 0
    assert refused(L.pisa_block_sparse_attn(pp, ok, ok, ok, ok, ok, None, bad, sz.value, None))
    # index and score arrays need only their elements' alignment
    assert L.pisa_bsa_select(pp, ok, ok, ctypes.c_void_p(4096 + 4), None, ok, 1,
                             None) == _lib.PISA_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    missing = str(tmp_path / "libpisa.so")
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            _lib.load(missing)
    finally:
        _lib._lib = saved


def test_score_variants_need_the_per_query_selector():
    """PISA-1 / PISA-2 scores run on the per-query selector; asking for the
    two-stage selector with them is refused before anything is launched."""
    L = lib()
    dummy = ctypes.create_string_buffer(64)
    ptr = ctypes.cast(dummy, ctypes.c_void_p)
    for bit in (_lib.PISA_SCORE_MEAN, _lib.PISA_SCORE_MEAN_VAR):
        p = problem(seq_len=131072, flags=_lib.PISA_CAUSAL | _lib.PISA_FORCE_FIRST_PREV | bit)
        assert L.pisa_select(ctypes.byref(p), ptr, ptr, ptr, ptr, None, _lib.PISA_SELECT_TWO_STAGE,
                             ptr, 1 << 40, None) == _lib.PISA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        from hierarchical_block_selection_amd import Problem
        Problem(1, 1, 1, 64, 64, score="max").to_c()


def test_backward_arguments():
    """The backward runs every shape the forward runs (bf16 C=64 power-of-two
    groups on MFMA, the rest on the general kernel) up to 8192 leaf blocks; it
    refuses more blocks, a missing row_lse or output, and a short workspace.
    Its workspace: the stable sort's maps, D, the dQ rows (bf16 on MFMA, fp32
    otherwise) and the fp32 per-item dk/dv partials."""
    L = lib()
    dummy = ctypes.create_string_buffer(64)
    ptr = ctypes.cast(dummy, ctypes.c_void_p)
    bwd = L.pisa_block_sparse_attn_backward
    sz = ctypes.c_size_t()
    for kw in (dict(dtype=_lib.PISA_F32), dict(block=32), dict(block=16, heads_q=6, heads_kv=2)):
        p = problem(**kw)
        assert L.pisa_workspace_bytes(ctypes.byref(p), _lib.PISA_OP_ATTN_BWD,
                                      ctypes.byref(sz)) == 0, kw
        assert sz.value > 0
    p = problem(seq_len=64 * 8192 + 1)
    assert bwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, 1 << 40,
               None) == _lib.PISA_ERR_UNSUPPORTED
    assert L.pisa_workspace_bytes(ctypes.byref(p), _lib.PISA_OP_ATTN_BWD,
                                  ctypes.byref(sz)) == _lib.PISA_ERR_UNSUPPORTED

    def a256(x):
        return (x + 255) // 256 * 256

    def want(g, hkv, n, k, c, d, per_item, dq_bytes):
        slots, m1 = hkv * n * k, hkv * -(-n // c)
        items = -(-slots // per_item) + m1
        chunks = -(-n // 128)  # row chunks of the stable sort
        return (a256(4 * m1) + a256(4 * (m1 + 1)) + a256(4 * m1) + a256(4 * (m1 + 1))
                + a256(4 * m1 * chunks) + a256(4 * slots) + a256(4 * slots)
                + a256(4 * g * hkv * n) + a256(dq_bytes * slots * g * d)
                + a256(4 * items * 2 * c * d))

    p = problem(heads_q=8, heads_kv=2, seq_len=3000, topk=8)
    pp = ctypes.byref(p)
    assert L.pisa_workspace_bytes(pp, _lib.PISA_OP_ATTN_BWD, ctypes.byref(sz)) == 0
    # MFMA path: 2048 columns per item = 512 pairs at G = 4, bf16 dQ rows
    assert sz.value == want(4, 2, 3000, 8, 64, 128, 512, 2)
    gp = problem(heads_q=6, heads_kv=2, seq_len=1000, topk=5, block=32, dtype=_lib.PISA_F32)
    assert L.pisa_workspace_bytes(ctypes.byref(gp), _lib.PISA_OP_ATTN_BWD, ctypes.byref(sz)) == 0
    # general path: 256 columns per item = 85 pairs at G = 3, fp32 dQ rows
    assert sz.value == want(3, 2, 1000, 5, 32, 128, 85, 4)
    assert L.pisa_workspace_bytes(pp, _lib.PISA_OP_ATTN_BWD, ctypes.byref(sz)) == 0
    args = [ptr] * 10
    for i in range(10):
        a = list(args)
        a[i] = None
        assert bwd(pp, *a, ptr, sz.value, None) == _lib.PISA_ERR_INVALID, i
    assert bwd(pp, *args, ptr, sz.value - 1, None) == _lib.PISA_ERR_WORKSPACE
    assert bwd(pp, *args, None, sz.value, None) == _lib.PISA_ERR_WORKSPACE


def test_noalloc_select_rejects_before_any_device_work():
    """pisa_select_noalloc validates on the host: null tensors, a bad strategy and
    a problem whose two-stage workspace exceeds the fixed scratch are rejected
    with no device call (this runs without a GPU)."""
    L = lib()
    big = problem(heads_q=8, heads_kv=8, seq_len=131072)
    need = ctypes.c_size_t()
    assert L.pisa_workspace_bytes(ctypes.byref(big), _lib.PISA_OP_SELECT, ctypes.byref(need)) == 0
    assert need.value > _lib.PISA_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    rc = L.pisa_select_noalloc(ctypes.byref(big), fake, fake, fake, fake, None,
                               _lib.PISA_SELECT_AUTO, None)
    assert rc == _lib.PISA_ERR_WORKSPACE
    assert b"scratch" in L.pisa_last_error()
    small = problem(seq_len=4096)
    assert L.pisa_select_noalloc(ctypes.byref(small), None, fake, fake, fake, None,
                                 _lib.PISA_SELECT_AUTO, None) == _lib.PISA_ERR_INVALID
    assert L.pisa_select_noalloc(ctypes.byref(small), fake, fake, fake, fake, None, 7,
                                 None) == _lib.PISA_ERR_INVALID
