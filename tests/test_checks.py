"""The GPU parity checks reject the mistakes long context makes small.

Negative controls on the CPU: the oracle's own sparse step at the 64K
long-context shape, then the same prefix statistics recomputed (float64,
through torch's attention) with one union page left out -- the error a
kernel that skipped or mis-addressed one page of a ~110-page union would make.
The checks of tests/checks.py, which the GPU tests apply to the HIP path's
outputs, must reject both the log-normalisers and the prefix outputs.
"""
import numpy as np

from checks import LP_ATOL, TOL, check_lp, check_values, lp_errors, value_errors
from oracle import Oracle
from oracle_pins import sdpa64, union_tokens
from sparse_attention_block_amd import workloads as W


def test_checks_reject_one_dropped_union_page():
    cfg = W.long_64k(128, 4)
    lay = W.make_layer(cfg, n_steps=2)
    orc = Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
    op, lp = W.make_cache_state(cfg)
    orc.op[...] = op
    orc.lp[...] = lp
    res = orc.step_threaded(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    scale = 1.0 / np.sqrt(cfg.head_dim)
    G, A = cfg.group, cfg.n_active
    rows_lp = {"exact": [], "dropped": []}
    rows_op = {"exact": [], "dropped": []}
    ref_lp, ref_op = [], []
    for g in range(cfg.n_kvhead):
        union = res["union_idx"][0, g, :res["union_cnt"][0, g]].tolist()
        drop = union[len(union) // 2]
        kept = [p for p in union if p != drop]
        ka, va = union_tokens(lay, 0, g, union)
        kd, vd = union_tokens(lay, 0, g, kept)
        for j in range(G):
            h = g * G + j
            for t in res["active"][0, h]:
                q = lay.q[1][0, t, h]
                for tag, (k, v) in (("exact", (ka, va)), ("dropped", (kd, vd))):
                    o, l = sdpa64(q, k, v, scale)
                    rows_op[tag].append(o)
                    rows_lp[tag].append(l)
                ref_op.append(orc.op[0, h, t])
                ref_lp.append(orc.lp[0, h, t])
    ref_op, ref_lp = np.array(ref_op), np.array(ref_lp)
    n = len(ref_lp)
    # the exact recomputation passes with a wide margin ...
    check_lp(np.array(rows_lp["exact"]), ref_lp, "bf16", "exact L_p")
    check_values(np.array(rows_op["exact"]), ref_op, "bf16", "exact o_p")
    # ... one dropped page fails: most rows' L_p, and their o_p rows
    e_lp = lp_errors(np.array(rows_lp["dropped"]), ref_lp, "bf16")
    e_op = value_errors(np.array(rows_op["dropped"]), ref_op, "bf16")
    assert e_lp["n_bad"] >= n // 2, (e_lp["n_bad"], n, e_lp["max_abs"])
    assert e_op["n_bad_row"] >= n // 2, (e_op["n_bad_row"], n, e_op["max_row_rel"])


def test_tolerances_are_the_stated_ones():
    assert TOL["bf16"] == dict(rtol=2e-2, atol=1e-2)
    assert LP_ATOL["bf16"] == 4e-3 and LP_ATOL["f32"] == 1e-4
