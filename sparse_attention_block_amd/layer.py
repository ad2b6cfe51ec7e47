"""Caller-side plumbing: one attention layer's device buffers for LoSA steps.

Holds the prefix KV cache, its page metadata, the (o_p, L_p) cache and a
workspace as torch tensors on the GPU, and calls the library's entry points
(``binding``) on the current stream.  All arithmetic happens in liblosa.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as L


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """A float32 array whose values are representable in ``dtype`` -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


class LayerState:
    def __init__(self, *, n_seq, block, n_qhead, n_kvhead, head_dim, budget_tokens, n_active,
                 dtype, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_off, prefix_len,
                 max_prefix_len: Optional[int] = None, softmax_scale=0.0, flags=0,
                 device="cuda", page_table=None):
        self.device = device
        kv_off = torch.as_tensor(np.asarray(kv_off, np.int32)).to(device)
        prefix_len_t = torch.as_tensor(np.asarray(prefix_len, np.int32)).to(device)
        if max_prefix_len is None:
            max_prefix_len = int(np.max(np.asarray(prefix_len))) if len(prefix_len) else 0
        self.shape = L.make_shape(n_seq=n_seq, block=block, n_qhead=n_qhead, n_kvhead=n_kvhead,
                                  head_dim=head_dim, budget_tokens=budget_tokens,
                                  n_active=n_active, max_prefix_len=max_prefix_len, dtype=dtype,
                                  kv_tokens=k_cache.shape[1], softmax_scale=softmax_scale,
                                  flags=flags)
        self.dtype = dtype
        self.k_cache, self.v_cache = k_cache, v_cache
        self.kv_off, self.prefix_len = kv_off, prefix_len_t
        # paged KV pool: [n_seq][pages of the longest prefix] physical pages (or None)
        self.page_table = (None if page_table is None else
                           torch.as_tensor(np.asarray(page_table, np.int32)).contiguous().to(device))
        self.page_meta = torch.zeros(max(1, L.page_meta_bytes(self.shape)), dtype=torch.uint8,
                                     device=device)
        self.workspace = torch.zeros(max(1, L.workspace_bytes(self.shape)), dtype=torch.uint8,
                                     device=device)
        self.op_cache = torch.zeros((n_seq, n_qhead, block, head_dim), dtype=torch.float32,
                                    device=device)
        self.lp_cache = torch.full((n_seq, n_qhead, block), float("-inf"), dtype=torch.float32,
                                   device=device)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.out = torch.empty((n_seq, block, n_qhead, head_dim), dtype=tdt, device=device)

    @classmethod
    def from_layer(cls, lay, device="cuda", n_active=None, budget=None) -> "LayerState":
        c = lay.cfg
        return cls(n_seq=c.n_seq, block=c.block, n_qhead=c.n_qhead, n_kvhead=c.n_kvhead,
                   head_dim=c.head_dim, budget_tokens=c.budget if budget is None else budget,
                   n_active=c.n_active if n_active is None else n_active, dtype=c.dtype,
                   k_cache=to_device(lay.k_cache, c.dtype, device),
                   v_cache=to_device(lay.v_cache, c.dtype, device),
                   kv_off=lay.kv_off, prefix_len=lay.prefix_len,
                   flags=getattr(c, "flags", 0), device=device)

    def build_page_meta(self, stream=None):
        L.losa_build_page_meta(self.shape, self.k_cache, self.kv_off, self.prefix_len,
                               self.page_meta, stream, page_table=self.page_table)

    def update_page_meta(self, first_token, max_new_tokens: int, stream=None):
        """After a committed block: the new prefix lengths are already in
        self.prefix_len; first_token[s] is each sequence's first new token."""
        ft = torch.as_tensor(np.asarray(first_token, np.int32)).to(self.device)
        L.losa_update_page_meta(self.shape, self.k_cache, self.kv_off, self.prefix_len, ft,
                                max_new_tokens, self.page_meta, stream, page_table=self.page_table)

    def dense_first_step(self, q_t, k_blk, v_blk, out=None, debug: Optional[L.Debug] = None,
                         stream=None):
        out = self.out if out is None else out
        L.losa_dense_first_step(self.shape, q_t, k_blk, v_blk, self.k_cache, self.v_cache,
                                self.kv_off, self.prefix_len, self.op_cache, self.lp_cache, out,
                                self.workspace, debug, stream, page_table=self.page_table)
        return out

    def prepare_dense_first_step(self, q_t, k_blk, v_blk, out=None, stream=None):
        out = self.out if out is None else out
        return L.prepare_dense_first_step(self.shape, q_t, k_blk, v_blk, self.k_cache,
                                          self.v_cache, self.kv_off, self.prefix_len,
                                          self.op_cache, self.lp_cache, out, self.workspace,
                                          stream, page_table=self.page_table)

    def prepare_step(self, q_t, q_prev, k_blk, v_blk, out=None, stream=None):
        out = self.out if out is None else out
        return L.prepare_step(self.shape, q_t, q_prev, k_blk, v_blk, self.k_cache, self.v_cache,
                              self.page_meta, self.kv_off, self.prefix_len, self.op_cache,
                              self.lp_cache, out, self.workspace, stream,
                              page_table=self.page_table)

    def step(self, q_t, q_prev, k_blk, v_blk, debug: Optional[L.Debug] = None, out=None,
             stream=None):
        out = self.out if out is None else out
        L.losa_step(self.shape, q_t, q_prev, k_blk, v_blk, self.k_cache, self.v_cache,
                    self.page_meta, self.kv_off, self.prefix_len, self.op_cache, self.lp_cache,
                    out, self.workspace, debug, stream, page_table=self.page_table)
        return out
