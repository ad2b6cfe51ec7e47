"""Thin Python binding of liblosa.so (the C ABI in include/losa.h).

Functions carry the C entry points' names and arguments; they only marshal
torch tensors (device memory) and streams into pointers, check that every
tensor lives on the GPU with the dtype and size the layout needs (so no bad
pointer ever reaches a kernel), and raise ``LosaError`` on a non-zero status.
Every step of the computation runs in the HIP library; there is no fallback:
if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_void_p
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblosa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "losa.h")

(LOSA_OK, LOSA_ERR_INVALID_ARG, LOSA_ERR_UNSUPPORTED, LOSA_ERR_WORKSPACE, LOSA_ERR_HIP,
 LOSA_ERR_SCRATCH) = range(6)
LOSA_NOALLOC_SCRATCH_BYTES = 32 << 20
LOSA_F32, LOSA_BF16 = 0, 1
PAGE = 16


class LosaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class LosaShape(ctypes.Structure):
    _fields_ = [
        ("n_seq", c_int32), ("block", c_int32), ("n_qhead", c_int32), ("n_kvhead", c_int32),
        ("head_dim", c_int32), ("page_size", c_int32), ("budget_tokens", c_int32),
        ("n_active", c_int32), ("max_prefix_len", c_int32), ("dtype", c_int32),
        ("kv_tokens", c_int64), ("softmax_scale", c_float), ("flags", c_uint32),
    ]


class LosaDebug(ctypes.Structure):
    _fields_ = [
        ("locality", c_void_p), ("active", c_void_p), ("page_sel", c_void_p),
        ("union_idx", c_void_p), ("union_cnt", c_void_p), ("union_cap", c_int32),
        ("stage_events", POINTER(c_void_p)),
    ]


LOSA_STAGE_EVENTS = 6


_lib = None


def load(path: str = LIB_PATH):
    """Load liblosa.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m sparse_attention_block_amd.build")
    lib = ctypes.CDLL(path)
    S = POINTER(LosaShape)
    lib.losa_status_string.argtypes = [c_int]
    lib.losa_status_string.restype = ctypes.c_char_p
    lib.losa_page_meta_bytes.argtypes = [S]
    lib.losa_page_meta_bytes.restype = c_size_t
    lib.losa_workspace_bytes.argtypes = [S]
    lib.losa_workspace_bytes.restype = c_size_t
    lib.losa_union_capacity.argtypes = [S]
    lib.losa_union_capacity.restype = c_int32
    lib.losa_build_page_meta.argtypes = [S, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p]
    lib.losa_build_page_meta.restype = c_int
    lib.losa_update_page_meta.argtypes = [S, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_int32, c_void_p, c_void_p]
    lib.losa_update_page_meta.restype = c_int
    lib.losa_dense_first_step.argtypes = [S] + [c_void_p] * 11 + [POINTER(LosaDebug), c_void_p,
                                                                   c_size_t, c_void_p]
    lib.losa_dense_first_step.restype = c_int
    lib.losa_step.argtypes = [S] + [c_void_p] * 13 + [POINTER(LosaDebug), c_void_p, c_size_t,
                                                       c_void_p]
    lib.losa_step.restype = c_int
    lib.losa_step_noalloc.argtypes = [S] + [c_void_p] * 13 + [POINTER(LosaDebug), c_void_p]
    lib.losa_step_noalloc.restype = c_int
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/losa.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(losa_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load().losa_status_string(int(status)).decode()


def make_shape(*, n_seq, block, n_qhead, n_kvhead, head_dim, budget_tokens, n_active,
               max_prefix_len, dtype, kv_tokens, page_size=PAGE, softmax_scale=0.0,
               flags=0) -> LosaShape:
    dt = {"f32": LOSA_F32, "bf16": LOSA_BF16}.get(dtype, dtype)
    return LosaShape(n_seq, block, n_qhead, n_kvhead, head_dim, page_size, budget_tokens,
                     n_active, max_prefix_len, dt, kv_tokens, softmax_scale, flags)


def page_meta_bytes(shape: LosaShape) -> int:
    return int(load().losa_page_meta_bytes(ctypes.byref(shape)))


def workspace_bytes(shape: LosaShape) -> int:
    return int(load().losa_workspace_bytes(ctypes.byref(shape)))


def union_capacity(shape: LosaShape) -> int:
    return int(load().losa_union_capacity(ctypes.byref(shape)))


# ---------------------------------------------------------------------------
# argument checks (so that no bad pointer reaches a kernel)

def _torch_dtype(shape: LosaShape):
    return torch.bfloat16 if shape.dtype == LOSA_BF16 else torch.float32


def _check(t: Optional[torch.Tensor], name: str, dtype, numel: int, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return c_void_p(t.data_ptr())


def _stream(stream) -> c_void_p:
    """A torch stream, a raw hipStream_t handle (int), or None for torch's current stream."""
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _raise(status: int, what: str):
    if status != LOSA_OK:
        raise LosaError(status, what)


def _sizes(shape: LosaShape):
    S, B, Hq, Hk, d = shape.n_seq, shape.block, shape.n_qhead, shape.n_kvhead, shape.head_dim
    return dict(q=S * B * Hq * d, blk=S * B * Hk * d, cache=Hk * shape.kv_tokens * d,
                op=S * Hq * B * d, lp=S * Hq * B,
                pt=S * max(1, (shape.max_prefix_len + PAGE - 1) // PAGE))


def _layout(shape, kv_off, prefix_len, page_table):
    """kv_off (contiguous sequences) and prefix_len, or a page table (kv_off optional)."""
    n = _sizes(shape)
    return [_check(kv_off, "kv_off", torch.int32, shape.n_seq, optional=page_table is not None),
            _check(prefix_len, "prefix_len", torch.int32, shape.n_seq),
            _check(page_table, "page_table", torch.int32, n["pt"], optional=True)]


# ---------------------------------------------------------------------------
# entry points

def losa_build_page_meta(shape, k_cache, kv_off, prefix_len, page_meta, stream=None,
                         page_table=None):
    n = _sizes(shape)
    args = [
        _check(k_cache, "k_cache", _torch_dtype(shape), n["cache"]),
        *_layout(shape, kv_off, prefix_len, page_table),
        _check(page_meta, "page_meta", torch.uint8, page_meta_bytes(shape)),
    ]
    _raise(load().losa_build_page_meta(ctypes.byref(shape), *args, _stream(stream)),
           "losa_build_page_meta")


def losa_update_page_meta(shape, k_cache, kv_off, prefix_len, first_token, max_new_tokens,
                          page_meta, stream=None, page_table=None):
    n = _sizes(shape)
    args = [
        _check(k_cache, "k_cache", _torch_dtype(shape), n["cache"]),
        *_layout(shape, kv_off, prefix_len, page_table),
        _check(first_token, "first_token", torch.int32, shape.n_seq),
    ]
    meta = _check(page_meta, "page_meta", torch.uint8, page_meta_bytes(shape))
    _raise(load().losa_update_page_meta(ctypes.byref(shape), *args, int(max_new_tokens), meta,
                                        _stream(stream)), "losa_update_page_meta")


def losa_dense_first_step(shape, q_t, k_blk, v_blk, k_cache, v_cache, kv_off, prefix_len,
                          op_cache, lp_cache, out, workspace, debug=None, stream=None,
                          page_table=None):
    n, dt = _sizes(shape), _torch_dtype(shape)
    ws_need = workspace_bytes(shape)
    args = [
        _check(q_t, "q_t", dt, n["q"]), _check(k_blk, "k_blk", dt, n["blk"]),
        _check(v_blk, "v_blk", dt, n["blk"]), _check(k_cache, "k_cache", dt, n["cache"]),
        _check(v_cache, "v_cache", dt, n["cache"]),
        *_layout(shape, kv_off, prefix_len, page_table),
        _check(op_cache, "op_cache", torch.float32, n["op"]),
        _check(lp_cache, "lp_cache", torch.float32, n["lp"]),
        _check(out, "out", dt, n["q"]),
    ]
    dbg = ctypes.byref(debug.struct(shape)) if debug is not None else None
    ws = _check(workspace, "workspace", torch.uint8, ws_need)
    _raise(load().losa_dense_first_step(ctypes.byref(shape), *args, dbg, ws, workspace.numel(),
                                        _stream(stream)), "losa_dense_first_step")


@dataclass
class Debug:
    """Optional device outputs of losa_step (allocate with ``Debug.alloc``)."""

    locality: Optional[torch.Tensor] = None
    active: Optional[torch.Tensor] = None
    page_sel: Optional[torch.Tensor] = None
    union_idx: Optional[torch.Tensor] = None
    union_cnt: Optional[torch.Tensor] = None
    stage_events: Optional[list] = None   # LOSA_STAGE_EVENTS raw hipEvent_t handles (ints)

    @staticmethod
    def alloc(shape: LosaShape, device="cuda") -> "Debug":
        S, B, Hq, Hk, A = shape.n_seq, shape.block, shape.n_qhead, shape.n_kvhead, shape.n_active
        k = shape.budget_tokens // shape.page_size
        cap = max(1, union_capacity(shape))
        i32 = dict(dtype=torch.int32, device=device)
        return Debug(locality=torch.full((S, Hq, B), -1.0, dtype=torch.float32, device=device),
                     active=torch.full((S, Hq, max(A, 1)), -9, **i32),
                     page_sel=torch.full((S, Hq, max(A, 1), k), -9, **i32),
                     union_idx=torch.full((S, Hk, cap), -9, **i32),
                     union_cnt=torch.full((S, Hk), -9, **i32))

    def struct(self, shape: LosaShape) -> LosaDebug:
        S, B, Hq, Hk, A = shape.n_seq, shape.block, shape.n_qhead, shape.n_kvhead, shape.n_active
        k = shape.budget_tokens // shape.page_size
        cap = self.union_idx.shape[-1] if self.union_idx is not None else 0
        ev = None
        if self.stage_events is not None:
            if len(self.stage_events) != LOSA_STAGE_EVENTS:
                raise ValueError(f"stage_events needs {LOSA_STAGE_EVENTS} events")
            self._ev_array = (c_void_p * LOSA_STAGE_EVENTS)(*self.stage_events)
            ev = ctypes.cast(self._ev_array, POINTER(c_void_p))
        return LosaDebug(
            _check(self.locality, "debug.locality", torch.float32, S * Hq * B, True),
            _check(self.active, "debug.active", torch.int32, S * Hq * A, True),
            _check(self.page_sel, "debug.page_sel", torch.int32, S * Hq * A * k, True),
            _check(self.union_idx, "debug.union_idx", torch.int32, S * Hk * cap, True),
            _check(self.union_cnt, "debug.union_cnt", torch.int32, S * Hk, True),
            cap, ev)


def losa_step(shape, q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off, prefix_len,
              op_cache, lp_cache, out, workspace, debug: Optional[Debug] = None, stream=None,
              page_table=None):
    n, dt = _sizes(shape), _torch_dtype(shape)
    ws_need = workspace_bytes(shape)
    args = [
        _check(q_t, "q_t", dt, n["q"]), _check(q_prev, "q_prev", dt, n["q"]),
        _check(k_blk, "k_blk", dt, n["blk"]), _check(v_blk, "v_blk", dt, n["blk"]),
        _check(k_cache, "k_cache", dt, n["cache"]), _check(v_cache, "v_cache", dt, n["cache"]),
        _check(page_meta, "page_meta", torch.uint8, page_meta_bytes(shape)),
        *_layout(shape, kv_off, prefix_len, page_table),
        _check(op_cache, "op_cache", torch.float32, n["op"]),
        _check(lp_cache, "lp_cache", torch.float32, n["lp"]),
        _check(out, "out", dt, n["q"]),
    ]
    dbg = ctypes.byref(debug.struct(shape)) if debug is not None else None
    ws = _check(workspace, "workspace", torch.uint8, ws_need)
    _raise(load().losa_step(ctypes.byref(shape), *args, dbg, ws, workspace.numel(),
                            _stream(stream)), "losa_step")


def losa_step_noalloc(shape, q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off,
                      prefix_len, op_cache, lp_cache, out, debug: Optional[Debug] = None,
                      stream=None, page_table=None):
    """losa_step on the library's static per-GPU scratch (no workspace argument)."""
    n, dt = _sizes(shape), _torch_dtype(shape)
    args = [
        _check(q_t, "q_t", dt, n["q"]), _check(q_prev, "q_prev", dt, n["q"]),
        _check(k_blk, "k_blk", dt, n["blk"]), _check(v_blk, "v_blk", dt, n["blk"]),
        _check(k_cache, "k_cache", dt, n["cache"]), _check(v_cache, "v_cache", dt, n["cache"]),
        _check(page_meta, "page_meta", torch.uint8, page_meta_bytes(shape)),
        *_layout(shape, kv_off, prefix_len, page_table),
        _check(op_cache, "op_cache", torch.float32, n["op"]),
        _check(lp_cache, "lp_cache", torch.float32, n["lp"]),
        _check(out, "out", dt, n["q"]),
    ]
    dbg = ctypes.byref(debug.struct(shape)) if debug is not None else None
    _raise(load().losa_step_noalloc(ctypes.byref(shape), *args, dbg, _stream(stream)),
           "losa_step_noalloc")


# ---------------------------------------------------------------------------
# prepared calls: checks and marshalling done once, then a bare C call

class PreparedCall:
    """A call of one entry point with fixed, already checked arguments.

    ``set_events`` swaps the profiling events recorded between the library's
    launches (a list of LOSA_STAGE_EVENTS raw hipEvent_t handles, or None)."""

    def __init__(self, fn, head, dbg: LosaDebug, tail, what: str):
        self._fn, self._head, self._dbg, self._tail, self._what = fn, head, dbg, tail, what
        self._args = (*head, ctypes.byref(dbg), *tail)
        self._ev = None

    def set_events(self, events):
        if events is None:
            self._dbg.stage_events = None
            self._ev = None
        else:
            self._ev = (c_void_p * LOSA_STAGE_EVENTS)(*events)
            self._dbg.stage_events = ctypes.cast(self._ev, POINTER(c_void_p))

    def __call__(self):
        st = self._fn(*self._args)
        if st != LOSA_OK:
            raise LosaError(st, self._what)


def prepare_dense_first_step(shape, q_t, k_blk, v_blk, k_cache, v_cache, kv_off, prefix_len,
                             op_cache, lp_cache, out, workspace, stream=None,
                             page_table=None) -> PreparedCall:
    n, dt = _sizes(shape), _torch_dtype(shape)
    head = [ctypes.byref(shape),
            _check(q_t, "q_t", dt, n["q"]), _check(k_blk, "k_blk", dt, n["blk"]),
            _check(v_blk, "v_blk", dt, n["blk"]), _check(k_cache, "k_cache", dt, n["cache"]),
            _check(v_cache, "v_cache", dt, n["cache"]),
            *_layout(shape, kv_off, prefix_len, page_table),
            _check(op_cache, "op_cache", torch.float32, n["op"]),
            _check(lp_cache, "lp_cache", torch.float32, n["lp"]),
            _check(out, "out", dt, n["q"])]
    tail = [_check(workspace, "workspace", torch.uint8, workspace_bytes(shape)),
            c_size_t(workspace.numel()), _stream(stream)]
    keep = (q_t, k_blk, v_blk, k_cache, v_cache, kv_off, prefix_len, page_table, op_cache,
            lp_cache, out, workspace)
    call = PreparedCall(load().losa_dense_first_step, head, LosaDebug(), tail,
                        "losa_dense_first_step")
    call._keep = keep
    return call


def prepare_step(shape, q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off,
                 prefix_len, op_cache, lp_cache, out, workspace, stream=None,
                 page_table=None) -> PreparedCall:
    n, dt = _sizes(shape), _torch_dtype(shape)
    head = [ctypes.byref(shape),
            _check(q_t, "q_t", dt, n["q"]), _check(q_prev, "q_prev", dt, n["q"]),
            _check(k_blk, "k_blk", dt, n["blk"]), _check(v_blk, "v_blk", dt, n["blk"]),
            _check(k_cache, "k_cache", dt, n["cache"]), _check(v_cache, "v_cache", dt, n["cache"]),
            _check(page_meta, "page_meta", torch.uint8, page_meta_bytes(shape)),
            *_layout(shape, kv_off, prefix_len, page_table),
            _check(op_cache, "op_cache", torch.float32, n["op"]),
            _check(lp_cache, "lp_cache", torch.float32, n["lp"]),
            _check(out, "out", dt, n["q"])]
    tail = [_check(workspace, "workspace", torch.uint8, workspace_bytes(shape)),
            c_size_t(workspace.numel()), _stream(stream)]
    keep = (q_t, q_prev, k_blk, v_blk, k_cache, v_cache, page_meta, kv_off, prefix_len, page_table,
            op_cache, lp_cache, out, workspace)
    call = PreparedCall(load().losa_step, head, LosaDebug(), tail, "losa_step")
    call._keep = keep
    return call
