"""The oracle's thread-pool drivers give the same bits as its single calls.

dense_first_step_threaded runs oracle_dense_row per (sequence, head, token);
step_threaded runs oracle_step per KV head on that head's group of query heads.
Both exist only to spread the same arithmetic over the host's cores (the GPU
tests compare every dense row at the long-context sizes, and the benchmark
times the oracle on all cores beside one).
"""
import numpy as np
import pytest

from oracle import Oracle
from sparse_attention_block_amd import workloads as W


def _pair(cfg):
    lay = W.make_layer(cfg)
    mk = lambda: Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
    return lay, mk(), mk()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_threaded_matches_single_calls(dtype):
    cfg = W.small_case(700, n_qhead=8, n_kvhead=2, head_dim=64, block=16, n_active=3, budget=48,
                       dtype=dtype, prefix_lens=(700, 0, 333), n_steps=3, needles=True)
    lay, a, b = _pair(cfg)
    out_a = a.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    out_b = b.dense_first_step_threaded(lay.q[0], lay.k_blk[0], lay.v_blk[0], threads=4)
    assert np.array_equal(out_a, out_b)
    assert np.array_equal(a.op, b.op) and np.array_equal(a.lp, b.lp)
    for t in (1, 2):
        ra = a.step(lay.q[t], lay.q[t - 1], lay.k_blk[t], lay.v_blk[t])
        rb = b.step_threaded(lay.q[t], lay.q[t - 1], lay.k_blk[t], lay.v_blk[t], threads=3)
        for key in ("out", "locality", "active", "page_sel", "union_cnt"):
            assert np.array_equal(ra[key], rb[key]), key
        for s in range(cfg.n_seq):
            for g in range(cfg.n_kvhead):
                n = int(ra["union_cnt"][s, g])
                assert np.array_equal(ra["union_idx"][s, g, :n], rb["union_idx"][s, g, :n])
        assert np.array_equal(a.op, b.op) and np.array_equal(a.lp, b.lp)


def test_dense_rows_subset():
    cfg = W.small_case(701, n_qhead=4, n_kvhead=1, head_dim=64, prefix_lens=(500,), dtype="bf16")
    lay, a, _ = _pair(cfg)
    out = a.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    rows = [(0, 3, 5), (0, 0, 0), (0, 2, 15)]
    op, lp, o = a.dense_rows(lay.q[0], lay.k_blk[0], lay.v_blk[0], rows, threads=2)
    for i, (s, h, t) in enumerate(rows):
        assert np.array_equal(op[i], a.op[s, h, t]) and lp[i] == a.lp[s, h, t]
        assert np.array_equal(o[i], out[s, t, h])
