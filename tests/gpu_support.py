"""Shared helpers of the GPU parity tests: the HIP path (through the C ABI) and
the CPU oracle run side by side on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.layer import LayerState, to_device

# Output tolerances: bf16 outputs accumulated in fp32 against the double oracle
# (max relative 2e-2, absolute 1e-2); fp32 inputs: fp32 accumulation over at
# most a few thousand terms, errors ~1e-6 relative, bound set at 1e-4.
TOL = {"bf16": dict(rtol=2e-2, atol=1e-2), "f32": dict(rtol=1e-4, atol=1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    g = np.where(both_inf, 0.0, got)
    r = np.where(both_inf, 0.0, ref)
    tol = TOL[dtype]
    bad = ~(np.abs(g - r) <= tol["atol"] + tol["rtol"] * np.abs(r))
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        worst = float(np.nanmax(np.abs(g - r)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"first {idx}; max abs err {worst:.3g}")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


class Pair:
    """The HIP path and the oracle on one layer's inputs."""

    def __init__(self, lay: W.Layer, name: str):
        self.lay, self.cfg, self.name = lay, lay.cfg, name
        c = lay.cfg
        self.orc = Oracle(c, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
        say(f"[{name}] upload S={c.n_seq} L={list(c.prefix_lens)[:4]} B={c.block} "
            f"Hq={c.n_qhead} Hkv={c.n_kvhead} d={c.head_dim} budget={c.budget} A={c.n_active} {c.dtype}")
        self.gpu = LayerState.from_layer(lay)
        self.dev = lambda x: to_device(x, c.dtype)
        self.q = [self.dev(x) for x in lay.q]
        self.kb = [self.dev(x) for x in lay.k_blk]
        self.vb = [self.dev(x) for x in lay.v_blk]
        say(f"[{self.name}] build_page_meta")
        self.gpu.build_page_meta()
        torch.cuda.synchronize()
        self.orc.page_meta()

    def set_cache(self, op: np.ndarray, lp: np.ndarray):
        self.orc.op[...] = op.astype(np.float64)
        self.orc.lp[...] = lp.astype(np.float64)
        self.gpu.op_cache.copy_(torch.from_numpy(op).to(self.gpu.op_cache.device))
        self.gpu.lp_cache.copy_(torch.from_numpy(lp).to(self.gpu.lp_cache.device))

    def dense(self, step: int = 0, sample_rows=None):
        c = self.cfg
        say(f"[{self.name}] dense_first_step step={step}")
        out = self.gpu.dense_first_step(self.q[step], self.kb[step], self.vb[step])
        torch.cuda.synchronize()
        out, op, lp = host(out), host(self.gpu.op_cache), host(self.gpu.lp_cache)
        if sample_rows is None:
            ref = self.orc.dense_first_step(self.lay.q[step], self.lay.k_blk[step],
                                            self.lay.v_blk[step])
            assert_close(out, ref, c.dtype, f"{self.name} dense out")
            assert_close(op, self.orc.op, c.dtype, f"{self.name} dense o_p")
            assert_close(lp, self.orc.lp, c.dtype, f"{self.name} dense L_p")
        else:
            rng = np.random.default_rng(1234)
            for _ in range(sample_rows):
                s = int(rng.integers(c.n_seq))
                h = int(rng.integers(c.n_qhead))
                t = int(rng.integers(c.block))
                o_p, l_p, row = self.orc.dense_row(self.lay.q[step], self.lay.k_blk[step],
                                                   self.lay.v_blk[step], s, h, t)
                assert_close(out[s, t, h], row, c.dtype, f"{self.name} dense out {s},{h},{t}")
                assert_close(op[s, h, t], o_p, c.dtype, f"{self.name} dense o_p {s},{h},{t}")
                assert_close(lp[s, h, t], l_p, c.dtype, f"{self.name} dense L_p {s},{h},{t}")
        return out

    def sparse(self, step: int, check_values=True):
        c = self.cfg
        dbg = L.Debug.alloc(self.gpu.shape)
        say(f"[{self.name}] losa_step step={step}")
        out = self.gpu.step(self.q[step], self.q[step - 1], self.kb[step], self.vb[step],
                            debug=dbg)
        torch.cuda.synchronize()
        res = self.orc.step(self.lay.q[step], self.lay.q[step - 1], self.lay.k_blk[step],
                            self.lay.v_blk[step])
        A, k = c.n_active, c.budget // c.page_size
        # Indices: bit-exact.
        assert np.array_equal(host(dbg.locality), res["locality"]), f"{self.name} locality bits"
        assert np.array_equal(host(dbg.active)[..., :A], res["active"]), f"{self.name} active set"
        if A > 0:
            assert np.array_equal(host(dbg.page_sel), res["page_sel"]), f"{self.name} page_sel"
        ucnt = host(dbg.union_cnt)
        assert np.array_equal(ucnt, res["union_cnt"]), f"{self.name} union_cnt"
        uidx = host(dbg.union_idx)
        for s in range(c.n_seq):
            for g in range(c.n_kvhead):
                n = int(ucnt[s, g])
                assert np.array_equal(uidx[s, g, :n], res["union_idx"][s, g, :n]), \
                    f"{self.name} union {s},{g}"
        if check_values:
            assert_close(host(out), res["out"], c.dtype, f"{self.name} step {step} out")
            assert_close(host(self.gpu.op_cache), self.orc.op, c.dtype, f"{self.name} step {step} o_p")
            assert_close(host(self.gpu.lp_cache), self.orc.lp, c.dtype, f"{self.name} step {step} L_p")
        return dict(out=host(out), res=res, union_cnt=ucnt)
