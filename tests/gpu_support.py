"""Shared helpers of the GPU parity tests: the HIP path (through the C ABI) and
the CPU oracle run side by side on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from checks import TOL, check_lp, check_values
from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.layer import LayerState, to_device


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, dtype, what):
    """Values (last axis = one row) within the checks module's element and row bounds."""
    say("  " + check_values(got, ref, dtype, what))


def assert_lp(got, ref, dtype, what):
    say("  " + check_lp(got, ref, dtype, what))


def stratified_rows(cfg, per_group: int, seed: int):
    """Rows (s, h, t) of a dense step: per_group rows in every (sequence, KV
    head) group, each a random query head of the group and a random token,
    distinct within the group."""
    rng = np.random.default_rng(seed)
    rows = []
    for s in range(cfg.n_seq):
        for g in range(cfg.n_kvhead):
            picks = rng.choice(cfg.group * cfg.block, size=min(per_group, cfg.group * cfg.block),
                               replace=False)
            rows += [(s, g * cfg.group + int(x) // cfg.block, int(x) % cfg.block) for x in picks]
    return rows


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


class Pair:
    """The HIP path and the oracle on one layer's inputs.  With ``paged`` =
    (k_pool, v_pool, page_table) the GPU reads the prefix from a paged pool
    (workloads.paged_pool) while the oracle reads the layer's contiguous cache."""

    def __init__(self, lay: W.Layer, name: str, paged=None):
        self.lay, self.cfg, self.name = lay, lay.cfg, name
        c = lay.cfg
        self.orc = Oracle(c, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
        say(f"[{name}] upload S={c.n_seq} L={list(c.prefix_lens)[:4]} B={c.block} "
            f"Hq={c.n_qhead} Hkv={c.n_kvhead} d={c.head_dim} budget={c.budget} A={c.n_active} {c.dtype}"
            + (f" paged pool of {paged[0].shape[1] // c.page_size} pages" if paged else ""))
        if paged is None:
            self.gpu = LayerState.from_layer(lay)
        else:
            k_pool, v_pool, pt = paged
            self.gpu = LayerState(n_seq=c.n_seq, block=c.block, n_qhead=c.n_qhead,
                                  n_kvhead=c.n_kvhead, head_dim=c.head_dim, budget_tokens=c.budget,
                                  n_active=c.n_active, dtype=c.dtype,
                                  k_cache=to_device(k_pool, c.dtype), v_cache=to_device(v_pool, c.dtype),
                                  kv_off=lay.kv_off, prefix_len=lay.prefix_len,
                                  flags=getattr(c, "flags", 0), page_table=pt)
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

    def dense(self, step: int = 0, rows=None):
        """The dense first step on the GPU against the oracle: every row (rows
        None: the oracle's whole step, row-parallel over the host's cores), or
        the given (s, h, t) rows only."""
        c = self.cfg
        say(f"[{self.name}] dense_first_step step={step}")
        out = self.gpu.dense_first_step(self.q[step], self.kb[step], self.vb[step])
        torch.cuda.synchronize()
        out, op, lp = host(out), host(self.gpu.op_cache), host(self.gpu.lp_cache)
        args = (self.lay.q[step], self.lay.k_blk[step], self.lay.v_blk[step])
        if rows is None:
            ref = self.orc.dense_first_step_threaded(*args)
            assert_close(out, ref, c.dtype, f"{self.name} dense out")
            assert_close(op, self.orc.op, c.dtype, f"{self.name} dense o_p")
            assert_lp(lp, self.orc.lp, c.dtype, f"{self.name} dense L_p")
        else:
            o_p, l_p, o_rows = self.orc.dense_rows(*args, rows)
            idx = tuple(np.array(rows).T)
            s_, h_, t_ = idx
            say(f"  {len(rows)} rows over {len(set(zip(s_, h_ // c.group)))} (sequence, KV head) groups")
            assert_close(out[s_, t_, h_], o_rows, c.dtype, f"{self.name} dense out rows")
            assert_close(op[s_, h_, t_], o_p, c.dtype, f"{self.name} dense o_p rows")
            assert_lp(lp[s_, h_, t_], l_p, c.dtype, f"{self.name} dense L_p rows")
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
            assert_lp(host(self.gpu.lp_cache), self.orc.lp, c.dtype, f"{self.name} step {step} L_p")
        return dict(out=host(out), res=res, union_cnt=ucnt)
