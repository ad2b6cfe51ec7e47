"""Naive per-query sparse attention on the GPU: every block token active, each
attending only over the pages it selected itself (losa_step with n_active = B
and LOSA_FLAG_ROW_MASK), against the oracle's per-query step
(oracle_naive_sparse_step: each token's own top-k pages, no reuse).  This is the
comparator the pages set LoSA against (agifrontier tutorial, section on KV
inflation; gist.science pt summary, "1. O Problema"): its loads are the union of
all B tokens' pages.  Supported while G * B <= 64 rows per KV head."""
import numpy as np
import pytest
import torch

from gpu_support import Pair, assert_close, assert_lp, host, say
from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W

pytestmark = pytest.mark.gpu
ROW_MASK = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def naive_cfg(base):
    return base.replace(n_active=base.block, flags=ROW_MASK)


CASES = [
    ("naive_bf16_small", lambda: naive_cfg(W.small_case(
        500, dtype="bf16", head_dim=128, block=16, budget=64, prefix_lens=(2000, 700, 0),
        n_kvhead=2, n_qhead=8, needles=True, n_steps=2))),
    ("naive_f32_d64", lambda: naive_cfg(W.small_case(
        501, dtype="f32", head_dim=64, block=16, budget=48, prefix_lens=(1000,), n_kvhead=1,
        n_qhead=4, n_steps=2))),
    ("naive_16k", lambda: naive_cfg(W.gqa_16k())),
    ("naive_64k_b128", lambda: naive_cfg(W.long_64k(128, 4))),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_naive_per_query_step(name, make):
    cfg = make()
    lay = W.make_layer(cfg, n_steps=2)
    p = Pair(lay, name)
    op, lp = W.make_cache_state(cfg)
    p.set_cache(op, lp)
    r = p.sparse(1)  # against the oracle's LoSA step with every token active and row masks
    # and against the oracle's separate per-query sparse step
    naive = Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
    ref = naive.naive_sparse_step(lay.q[1], lay.k_blk[1], lay.v_blk[1])
    assert_close(r["out"], ref, cfg.dtype, f"{name} out vs naive per-query step")
    assert_close(host(p.gpu.op_cache), naive.op, cfg.dtype, f"{name} o_p vs naive")
    assert_lp(host(p.gpu.lp_cache), naive.lp, cfg.dtype, f"{name} L_p vs naive")
    say(f"  union pages per (seq, KV head): {r['union_cnt'].tolist()}")
