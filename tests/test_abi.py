"""The C-ABI library loads, exports what include/losa.h declares, sizes its
buffers, and rejects bad arguments on the host before anything is enqueued
(no GPU needed: every call below fails validation before its first HIP call)."""
import ctypes

import pytest

from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W


@pytest.fixture(scope="module")
def lib():
    return L.load()


def shape_of(cfg, **kw):
    _, lens, T = W.prefix_layout(cfg.prefix_lens, cfg.page_size)
    args = dict(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead, n_kvhead=cfg.n_kvhead,
                head_dim=cfg.head_dim, budget_tokens=cfg.budget, n_active=cfg.n_active,
                max_prefix_len=int(max(lens)), dtype=cfg.dtype, kv_tokens=T)
    args.update(kw)
    return L.make_shape(**args)


CONFIGS = [W.tiny_f32(), W.gqa_16k(), W.long_64k(128, 4), W.long_64k(256, 8), W.ragged_batch(),
           W.trace_128k(0), W.trace_128k(20)]


def test_exports_every_header_symbol(lib):
    names = L.header_functions()
    assert set(names) >= {"losa_build_page_meta", "losa_step", "losa_dense_first_step",
                          "losa_status_string", "losa_page_meta_bytes", "losa_workspace_bytes",
                          "losa_union_capacity"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert L.status_string(L.LOSA_OK) == "ok"
    assert "workspace" in L.status_string(L.LOSA_ERR_WORKSPACE)
    assert L.status_string(99) == "unknown status"


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: c.name)
def test_sizes(cfg):
    sh = shape_of(cfg)
    _, lens, T = W.prefix_layout(cfg.prefix_lens, cfg.page_size)
    max_pages = (int(max(lens)) + 15) // 16
    cap = min(max_pages, cfg.group * cfg.n_active * (cfg.budget // 16))
    assert L.union_capacity(sh) == max(cap, 1)
    s_t = 2 if cfg.dtype == "bf16" else 4
    # metadata pages: the cache's pages or max_pages per sequence, whichever is more
    tiles = (max(T // 16, cfg.n_seq * max_pages) + 63) // 64
    # min/max pairs per (page, dimension), then one fp32 max |key| per page
    assert L.page_meta_bytes(sh) == cfg.n_kvhead * tiles * 64 * (2 * cfg.head_dim * 2 * s_t + 4)
    ws = L.workspace_bytes(sh)
    assert 0 < ws < 1 << 31


BAD_SHAPES = [
    (dict(n_qhead=6, n_kvhead=4), L.LOSA_ERR_INVALID_ARG),
    (dict(budget_tokens=40), L.LOSA_ERR_INVALID_ARG),
    (dict(budget_tokens=0), L.LOSA_ERR_INVALID_ARG),
    (dict(n_active=17), L.LOSA_ERR_INVALID_ARG),
    (dict(n_active=-1), L.LOSA_ERR_INVALID_ARG),
    (dict(head_dim=96), L.LOSA_ERR_UNSUPPORTED),
    (dict(page_size=32, budget_tokens=64), L.LOSA_ERR_UNSUPPORTED),
    (dict(dtype=7), L.LOSA_ERR_INVALID_ARG),
    (dict(flags=8), L.LOSA_ERR_INVALID_ARG),
    (dict(flags=1, n_qhead=32, n_kvhead=1, n_active=4), L.LOSA_ERR_UNSUPPORTED),
    (dict(max_prefix_len=2048), L.LOSA_ERR_INVALID_ARG),
    (dict(softmax_scale=-1.0), L.LOSA_ERR_INVALID_ARG),
    (dict(kv_tokens=1000), L.LOSA_ERR_INVALID_ARG),
    (dict(n_seq=0), L.LOSA_ERR_INVALID_ARG),
    (dict(block=65, n_active=4), L.LOSA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_SHAPES, ids=[str(k) for k, _ in BAD_SHAPES])
def test_bad_shape_rejected(lib, kw, status):
    sh = shape_of(W.tiny_f32(), **kw)
    assert L.workspace_bytes(sh) == 0 and L.page_meta_bytes(sh) == 0
    assert L.union_capacity(sh) == -1
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    r = lib.losa_step(ctypes.byref(sh), *([fake] * 13), None, fake, 1 << 30, None)
    assert r == status
    r = lib.losa_dense_first_step(ctypes.byref(sh), *([fake] * 11), None, fake, 1 << 30, None)
    assert r == status
    r = lib.losa_build_page_meta(ctypes.byref(sh), fake, fake, fake, None, fake, None)
    assert r == status
    r = lib.losa_update_page_meta(ctypes.byref(sh), fake, fake, fake, None, fake, 16, fake, None)
    assert r == status


def test_update_page_meta_checks(lib):
    """Block-commit update: null or misaligned pointers and a token bound outside
    0 .. max_prefix_len are rejected before anything is enqueued."""
    sh = shape_of(W.gqa_16k())
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    ok = [fake, fake, fake, None, fake]  # k_cache, kv_off, prefix_len, page_table, first_token
    for i in (0, 1, 2, 4):
        bad = list(ok)
        bad[i] = None
        assert lib.losa_update_page_meta(ctypes.byref(sh), *bad, 16, fake, None) == L.LOSA_ERR_INVALID_ARG
    assert lib.losa_update_page_meta(ctypes.byref(sh), *ok, 16, None, None) == L.LOSA_ERR_INVALID_ARG
    for i in (0, 1, 2, 3, 4):
        bad = list(ok)
        bad[i] = odd
        assert lib.losa_update_page_meta(ctypes.byref(sh), *bad, 16, fake, None) == \
            L.LOSA_ERR_INVALID_ARG
    assert lib.losa_update_page_meta(ctypes.byref(sh), *ok, -1, fake, None) == L.LOSA_ERR_INVALID_ARG
    assert lib.losa_update_page_meta(ctypes.byref(sh), *ok, sh.max_prefix_len + 1, fake,
                                     None) == L.LOSA_ERR_INVALID_ARG


def test_pointer_and_workspace_checks(lib):
    sh = shape_of(W.gqa_16k())
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    need = L.workspace_bytes(sh)
    # q_t q_prev k_blk v_blk k_cache v_cache page_meta kv_off prefix_len page_table op lp out
    args = [fake] * 9 + [None] + [fake] * 3
    KV_OFF, PREFIX_LEN, PAGE_TABLE, LP = 7, 8, 9, 11
    # null and misaligned tensors (a null page table is the contiguous layout)
    for i in range(13):
        bad = list(args)
        if i != PAGE_TABLE:
            bad[i] = None
            assert lib.losa_step(ctypes.byref(sh), *bad, None, fake, need, None) == L.LOSA_ERR_INVALID_ARG
        if i not in (KV_OFF, PREFIX_LEN, PAGE_TABLE, LP):  # int32 / fp32 arrays: 4-byte alignment
            bad[i] = odd
            assert lib.losa_step(ctypes.byref(sh), *bad, None, fake, need, None) == \
                L.LOSA_ERR_INVALID_ARG
    # a misaligned page table; a page table with a misaligned kv_off
    bad = list(args)
    bad[PAGE_TABLE] = odd
    assert lib.losa_step(ctypes.byref(sh), *bad, None, fake, need, None) == L.LOSA_ERR_INVALID_ARG
    bad = list(args)
    bad[PAGE_TABLE], bad[KV_OFF] = fake, odd
    assert lib.losa_step(ctypes.byref(sh), *bad, None, fake, need, None) == L.LOSA_ERR_INVALID_ARG
    assert lib.losa_step(ctypes.byref(sh), *args, None, None, need, None) == L.LOSA_ERR_INVALID_ARG
    # workspace one byte short
    assert lib.losa_step(ctypes.byref(sh), *args, None, fake, need - 1, None) == L.LOSA_ERR_WORKSPACE
    dense = [fake] * 7 + [None] + [fake] * 3
    assert lib.losa_dense_first_step(ctypes.byref(sh), *dense, None, fake, need - 1,
                                     None) == L.LOSA_ERR_WORKSPACE
    # debug union list shorter than the union capacity
    dbg = L.LosaDebug(None, None, None, fake, None, L.union_capacity(sh) - 1, None)
    assert lib.losa_step(ctypes.byref(sh), *args, ctypes.byref(dbg), fake, need, None) == \
        L.LOSA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    cfg = W.tiny_f32()
    sh = shape_of(cfg)
    t = torch.zeros(1 << 16)
    with pytest.raises(ValueError):
        L.losa_build_page_meta(sh, t, torch.zeros(1, dtype=torch.int32),
                               torch.zeros(1, dtype=torch.int32), torch.zeros(16, dtype=torch.uint8))


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The ragged batch's step needs more than the static scratch: LOSA_ERR_SCRATCH
    before any HIP call (the pointers below are never dereferenced)."""
    cfg = W.ragged_batch()
    sh = shape_of(cfg)
    p = ctypes.c_void_p(1 << 20)
    st = lib.losa_step_noalloc(ctypes.byref(sh), *([p] * 9), None, *([p] * 3), None, None)
    assert st == L.LOSA_ERR_SCRATCH, L.status_string(st)
    assert "static scratch" in L.status_string(L.LOSA_ERR_SCRATCH)
