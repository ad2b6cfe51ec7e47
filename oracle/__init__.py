"""CPU oracle for LoSA's per-denoising-step attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``liblosa_oracle.so`` (plain C, built from
``losa_oracle.c`` by ``oracle/build.py``) with ctypes and numpy; it imports
nothing from the HIP library's package, and the HIP library imports nothing
from here.

Every function takes numpy arrays in the layouts described in
``losa_oracle.c`` plus a shape object: anything with the attributes
``n_seq, block, n_qhead, n_kvhead, head_dim, page_size, budget, n_active,
dtype`` (``"f32"`` or ``"bf16"``).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblosa_oracle.so")


class OracleShape(ctypes.Structure):
    _fields_ = [
        ("n_seq", c_int32), ("block", c_int32), ("n_qhead", c_int32), ("n_kvhead", c_int32),
        ("head_dim", c_int32), ("page_size", c_int32), ("budget_tokens", c_int32),
        ("n_active", c_int32), ("out_bf16", c_int32), ("union_cap", c_int32),
        ("kv_tokens", c_int64), ("softmax_scale", c_double), ("flags", c_int32),
        ("pad_", c_int32),
    ]


_F = POINTER(c_float)
_D = POINTER(c_double)
_I = POINTER(c_int32)
_S = POINTER(OracleShape)

_lib = None


def load(path: str = LIB_PATH):
    """Load (building first if absent) the oracle library."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_page_meta.argtypes = [_S, _F, _I, _I, _F, _F]
    lib.oracle_locality.argtypes = [_S, _F, _F, _F]
    lib.oracle_active_set.argtypes = [_S, _F, _I]
    lib.oracle_shared_active_set.argtypes = [_S, _F, _F, _I]
    lib.oracle_page_bound.argtypes = [_F, _F, _F, c_int]
    lib.oracle_page_bound.restype = c_float
    lib.oracle_select_pages.argtypes = [_S, _F, _F, _F, _I, _I, _I, _I, _I, _I, _F, c_int64]
    lib.oracle_step.argtypes = [_S, _F, _F, _F, _F, _F, _F, _F, _F, _I, _I, _D, _D, _F, _F, _I,
                                _I, _I, _I]
    lib.oracle_dense_first_step.argtypes = [_S, _F, _F, _F, _F, _F, _I, _I, _D, _D, _F]
    lib.oracle_naive_sparse_step.argtypes = [_S, _F, _F, _F, _F, _F, _F, _F, _I, _I, _D, _D, _F]
    lib.oracle_dense_row.argtypes = [_S, c_int, c_int, c_int, _F, _F, _F, _F, _F, _I, _I, _D, _D,
                                     _F]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _f(a):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(_F)


def _d(a):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(_D)


def _i(a):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(_I)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def make_shape(cfg, kv_tokens: int, union_cap: int = 0, n_active=None, budget=None,
               softmax_scale: float = 0.0) -> OracleShape:
    return OracleShape(
        cfg.n_seq, cfg.block, cfg.n_qhead, cfg.n_kvhead, cfg.head_dim, cfg.page_size,
        cfg.budget if budget is None else budget,
        cfg.n_active if n_active is None else n_active,
        1 if cfg.dtype == "bf16" else 0, union_cap, kv_tokens, softmax_scale,
        getattr(cfg, "flags", 0), 0)


class Oracle:
    """Stateful wrapper: one layer's prefix cache plus its (o_p, L_p) cache."""

    def __init__(self, cfg, kv_off, prefix_len, kv_tokens, k_cache, v_cache, lib=None,
                 softmax_scale: float = 0.0):
        self.lib = lib if lib is not None else load()
        self.cfg = cfg
        self.kv_off = _i32(kv_off)
        self.prefix_len = _i32(prefix_len)
        self.kv_tokens = int(kv_tokens)
        self.k_cache = _f32(k_cache)
        self.v_cache = _f32(v_cache)
        self.scale = softmax_scale
        P = cfg.page_size
        self.max_pages = int(max(1, max((int(L) + P - 1) // P for L in self.prefix_len)))
        self.kmin = None
        self.kmax = None
        nrow = cfg.n_seq * cfg.n_qhead * cfg.block
        self.op = np.zeros((cfg.n_seq, cfg.n_qhead, cfg.block, cfg.head_dim), np.float64)
        self.lp = np.full((cfg.n_seq, cfg.n_qhead, cfg.block), -np.inf, np.float64)
        assert self.op.size == nrow * cfg.head_dim

    def shape(self, union_cap=0, n_active=None, budget=None):
        return make_shape(self.cfg, self.kv_tokens, union_cap, n_active, budget, self.scale)

    @property
    def union_cap(self):
        c = self.cfg
        k = c.budget // c.page_size
        return int(min(self.max_pages, c.group * c.n_active * max(k, 1)))

    # --- building blocks -------------------------------------------------
    def page_meta(self):
        c = self.cfg
        TP = self.kv_tokens // c.page_size
        kmin = np.zeros((c.n_kvhead, TP, c.head_dim), np.float32)
        kmax = np.zeros((c.n_kvhead, TP, c.head_dim), np.float32)
        sh = self.shape()
        self.lib.oracle_page_meta(ctypes.byref(sh), _f(self.k_cache), _i(self.kv_off),
                                  _i(self.prefix_len), _f(kmin), _f(kmax))
        self.kmin, self.kmax = kmin, kmax
        return kmin, kmax

    def locality(self, q_t, q_prev):
        c = self.cfg
        out = np.zeros((c.n_seq, c.n_qhead, c.block), np.float32)
        sh = self.shape()
        self.lib.oracle_locality(ctypes.byref(sh), _f(_f32(q_t)), _f(_f32(q_prev)), _f(out))
        return out

    def active_set(self, score, n_active=None):
        c = self.cfg
        A = c.n_active if n_active is None else n_active
        out = np.zeros((c.n_seq, c.n_qhead, A), np.int32)
        sh = self.shape(n_active=A)
        self.lib.oracle_active_set(ctypes.byref(sh), _f(_f32(score)), _i(out))
        return out

    def select_pages(self, q_t, active, want_bounds=False):
        c = self.cfg
        if self.kmin is None:
            self.page_meta()
        A = active.shape[2]
        k = c.budget // c.page_size
        cap = self.max_pages
        page_sel = np.full((c.n_seq, c.n_qhead, A, max(k, 1)), -7, np.int32)
        uidx = np.full((c.n_seq, c.n_kvhead, cap), -1, np.int32)
        ucnt = np.zeros((c.n_seq, c.n_kvhead), np.int32)
        sh = self.shape(union_cap=cap, n_active=A)
        bounds = None
        bptr, bstride = None, 0
        if want_bounds:
            bounds = np.zeros((c.n_seq, c.n_kvhead, c.group * A, self.max_pages), np.float32)
            bptr, bstride = _f(bounds), self.max_pages
        self.lib.oracle_select_pages(ctypes.byref(sh), _f(_f32(q_t)), _f(self.kmin), _f(self.kmax),
                                     _i(self.kv_off), _i(self.prefix_len), _i(_i32(active)),
                                     _i(page_sel) if k > 0 else None, _i(uidx), _i(ucnt), bptr,
                                     bstride)
        return page_sel[..., :k], uidx, ucnt, bounds

    # --- whole steps ------------------------------------------------------
    def dense_first_step(self, q_t, k_blk, v_blk):
        c = self.cfg
        out = np.zeros((c.n_seq, c.block, c.n_qhead, c.head_dim), np.float32)
        sh = self.shape()
        self.lib.oracle_dense_first_step(ctypes.byref(sh), _f(_f32(q_t)), _f(_f32(k_blk)),
                                         _f(_f32(v_blk)), _f(self.k_cache), _f(self.v_cache),
                                         _i(self.kv_off), _i(self.prefix_len), _d(self.op),
                                         _d(self.lp), _f(out))
        return out

    def step(self, q_t, q_prev, k_blk, v_blk):
        """One LoSA step; updates the (o_p, L_p) cache; returns out and the debug indices."""
        c = self.cfg
        if self.kmin is None:
            self.page_meta()
        A = c.n_active
        k = c.budget // c.page_size
        cap = self.max_pages
        out = np.zeros((c.n_seq, c.block, c.n_qhead, c.head_dim), np.float32)
        loc = np.zeros((c.n_seq, c.n_qhead, c.block), np.float32)
        act = np.zeros((c.n_seq, c.n_qhead, max(A, 1)), np.int32)
        psel = np.full((c.n_seq, c.n_qhead, max(A, 1), max(k, 1)), -7, np.int32)
        uidx = np.full((c.n_seq, c.n_kvhead, cap), -1, np.int32)
        ucnt = np.zeros((c.n_seq, c.n_kvhead), np.int32)
        sh = self.shape(union_cap=cap)
        self.lib.oracle_step(ctypes.byref(sh), _f(_f32(q_t)), _f(_f32(q_prev)), _f(_f32(k_blk)),
                             _f(_f32(v_blk)), _f(self.k_cache), _f(self.v_cache), _f(self.kmin),
                             _f(self.kmax), _i(self.kv_off), _i(self.prefix_len), _d(self.op),
                             _d(self.lp), _f(out), _f(loc), _i(act), _i(psel), _i(uidx),
                             _i(ucnt))
        return dict(out=out, locality=loc, active=act[..., :A], page_sel=psel[..., :A, :k],
                    union_idx=uidx, union_cnt=ucnt)

    def dense_row(self, q_t, k_blk, v_blk, s, h, t):
        """One (sequence, head, token) row of the dense first step: (o_p, L_p, out row).
        Does not touch the (o_p, L_p) cache."""
        c = self.cfg
        op = np.zeros(c.head_dim, np.float64)
        lp = np.zeros(1, np.float64)
        out = np.zeros(c.head_dim, np.float32)
        sh = self.shape()
        self.lib.oracle_dense_row(ctypes.byref(sh), int(s), int(h), int(t), _f(_f32(q_t)),
                                  _f(_f32(k_blk)), _f(_f32(v_blk)), _f(self.k_cache),
                                  _f(self.v_cache), _i(self.kv_off), _i(self.prefix_len), _d(op),
                                  _d(lp), _f(out))
        return op, float(lp[0]), out

    def dense_rows(self, q_t, k_blk, v_blk, rows, threads=None):
        """oracle_dense_row for each (s, h, t) of ``rows``, on a pool of threads
        (ctypes releases the interpreter lock during each call, and every call
        reads shared inputs and writes only its own outputs).  Returns (o_p
        [n][d] float64, L_p [n] float64, out rows [n][d] float32); the cache is
        not touched."""
        q_t, k_blk, v_blk = _f32(q_t), _f32(k_blk), _f32(v_blk)
        with ThreadPoolExecutor(max_workers=threads or host_threads()) as ex:
            res = list(ex.map(lambda r: self.dense_row(q_t, k_blk, v_blk, *r), rows))
        return (np.stack([r[0] for r in res]), np.array([r[1] for r in res]),
                np.stack([r[2] for r in res]))

    def dense_first_step_threaded(self, q_t, k_blk, v_blk, threads=None):
        """dense_first_step computed row by row over a thread pool: the same
        per-row arithmetic (oracle_dense_row), so the same bits."""
        c = self.cfg
        rows = [(s, h, t) for s in range(c.n_seq) for h in range(c.n_qhead) for t in range(c.block)]
        op, lp, out_rows = self.dense_rows(q_t, k_blk, v_blk, rows, threads)
        out = np.zeros((c.n_seq, c.block, c.n_qhead, c.head_dim), np.float32)
        for i, (s, h, t) in enumerate(rows):
            self.op[s, h, t] = op[i]
            self.lp[s, h, t] = lp[i]
            out[s, t, h] = out_rows[i]
        return out

    def step_threaded(self, q_t, q_prev, k_blk, v_blk, threads=None):
        """step() as independent per-KV-head sub-problems on a pool of threads.

        A KV head's group of query heads, its pages, union, prefix attention,
        block attention and cache rows depend on no other KV head (the active
        sets are per query head), so oracle_step on each group alone -- shape
        with n_qhead = G, n_kvhead = 1 -- gives the same bits as one call over
        all heads.  Not for the shared active set, whose score sums over every
        query head."""
        c = self.cfg
        assert not (getattr(c, "flags", 0) & 2), "the shared active set spans all KV heads"
        if self.kmin is None:
            self.page_meta()
        G, Hk, A = c.group, c.n_kvhead, c.n_active
        k = c.budget // c.page_size
        q_t, q_prev, k_blk, v_blk = _f32(q_t), _f32(q_prev), _f32(k_blk), _f32(v_blk)
        sub_cfg = _SubShape(c, n_qhead=G, n_kvhead=1)

        def one(g):
            hs = slice(g * G, (g + 1) * G)
            sub = Oracle.__new__(Oracle)
            sub.lib, sub.cfg, sub.kv_off, sub.prefix_len = self.lib, sub_cfg, self.kv_off, self.prefix_len
            sub.kv_tokens, sub.scale, sub.max_pages = self.kv_tokens, self.scale, self.max_pages
            sub.k_cache, sub.v_cache = self.k_cache[g:g + 1], self.v_cache[g:g + 1]
            sub.kmin, sub.kmax = self.kmin[g:g + 1], self.kmax[g:g + 1]
            sub.op = np.ascontiguousarray(self.op[:, hs])
            sub.lp = np.ascontiguousarray(self.lp[:, hs])
            res = sub.step(np.ascontiguousarray(q_t[:, :, hs]), np.ascontiguousarray(q_prev[:, :, hs]),
                           np.ascontiguousarray(k_blk[:, :, g:g + 1]),
                           np.ascontiguousarray(v_blk[:, :, g:g + 1]))
            return g, res, sub.op, sub.lp

        with ThreadPoolExecutor(max_workers=min(Hk, threads or host_threads())) as ex:
            parts = list(ex.map(one, range(Hk)))
        out = np.zeros((c.n_seq, c.block, c.n_qhead, c.head_dim), np.float32)
        loc = np.zeros((c.n_seq, c.n_qhead, c.block), np.float32)
        act = np.zeros((c.n_seq, c.n_qhead, A), np.int32)
        psel = np.zeros((c.n_seq, c.n_qhead, A, k), np.int32)
        uidx = np.full((c.n_seq, Hk, self.max_pages), -1, np.int32)
        ucnt = np.zeros((c.n_seq, Hk), np.int32)
        for g, res, op, lp in parts:
            hs = slice(g * G, (g + 1) * G)
            out[:, :, hs] = res["out"]
            loc[:, hs] = res["locality"]
            act[:, hs] = res["active"]
            psel[:, hs] = res["page_sel"]
            uidx[:, g] = res["union_idx"][:, 0]
            ucnt[:, g] = res["union_cnt"][:, 0]
            self.op[:, hs] = op
            self.lp[:, hs] = lp
        return dict(out=out, locality=loc, active=act, page_sel=psel, union_idx=uidx,
                    union_cnt=ucnt)

    def naive_sparse_step(self, q_t, k_blk, v_blk):
        c = self.cfg
        if self.kmin is None:
            self.page_meta()
        out = np.zeros((c.n_seq, c.block, c.n_qhead, c.head_dim), np.float32)
        sh = self.shape()
        self.lib.oracle_naive_sparse_step(ctypes.byref(sh), _f(_f32(q_t)), _f(_f32(k_blk)),
                                          _f(_f32(v_blk)), _f(self.k_cache), _f(self.v_cache),
                                          _f(self.kmin), _f(self.kmax), _i(self.kv_off),
                                          _i(self.prefix_len), _d(self.op), _d(self.lp), _f(out))
        return out


class _SubShape:
    """The attributes make_shape reads, from a workload shape with some replaced."""

    def __init__(self, cfg, **kw):
        for a in ("n_seq", "block", "n_qhead", "n_kvhead", "head_dim", "page_size", "budget",
                  "n_active", "dtype"):
            setattr(self, a, kw.get(a, getattr(cfg, a)))
        self.flags = kw.get("flags", getattr(cfg, "flags", 0))

    @property
    def group(self):
        return self.n_qhead // self.n_kvhead


def host_threads() -> int:
    """Threads for the row-parallel oracle calls: the CPUs this process may run
    on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def page_bound(q, mn, mx, lib=None):
    """The oracle's bound for one query vector and one page's min/max vectors."""
    lib = lib if lib is not None else load()
    q, mn, mx = _f32(q), _f32(mn), _f32(mx)
    return float(lib.oracle_page_bound(_f(q), _f(mn), _f(mx), int(q.shape[0])))
