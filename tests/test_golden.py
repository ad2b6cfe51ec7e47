"""The oracle on a hand-worked two-step example (tests/golden/hand_worked_d2.json).

The fixture's inputs are small enough that every index and every output has a
closed form, written in the fixture's derivation; the expected floats are
evaluated here from those closed forms, not from any implementation.
"""
import json
import math
import os

import numpy as np

from oracle import Oracle
from sparse_attention_block_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    with open(os.path.join(HERE, "golden", "hand_worked_d2.json")) as f:
        return json.load(f)


def _rle(runs):
    return np.array([v for v, n in runs for _ in range(n)], np.float32)


def test_hand_worked_two_step_trace():
    g = _load()
    sh = g["shape"]
    cfg = W.small_case(900, n_seq=1, block=sh["block"], n_qhead=1, n_kvhead=1,
                       head_dim=sh["head_dim"], page_size=sh["page_size"], budget=sh["budget"],
                       n_active=sh["n_active"], dtype=sh["dtype"], prefix_lens=(sh["prefix_len"],))
    k = _rle(g["prefix"]["keys"])[None]          # [1][32][2]
    v = _rle(g["prefix"]["values"])[None]
    orc = Oracle(cfg, [0], [sh["prefix_len"]], 32, k, v)

    def arr(x, heads=1):
        return np.array(x, np.float32).reshape(1, cfg.block, heads, cfg.head_dim)

    s1, s2 = g["step1"], g["step2"]
    orc.dense_first_step(arr(s1["q"]), arr(s1["k_blk"]), arr(s1["v_blk"]))
    res = orc.step(arr(s2["q"]), arr(s1["q"]), arr(s2["k_blk"]), arr(s2["v_blk"]))

    exp_ = g["expected"]
    assert res["active"][0, 0].tolist() == exp_["active_step2"]
    assert res["page_sel"][0, 0, 0].tolist() == exp_["page_sel_step2_token0"]
    assert res["union_idx"][0, 0, :res["union_cnt"][0, 0]].tolist() == exp_["union_step2"]
    _, _, _, bounds = orc.select_pages(arr(s2["q"]), np.array([[[0]]], np.int32), want_bounds=True)
    assert bounds[0, 0, 0, :2].tolist() == exp_["bound_step2_token0"]
    assert res["locality"][0, 0].tolist() == [0.5, 0.0]

    r2 = math.sqrt(2.0)
    sig = 1.0 / (1.0 + math.exp(1 / r2 - r2))
    lp0 = math.log(8 * math.exp(r2) + 8 * math.exp(1 / r2))
    assert np.allclose(orc.op[0, 0, 0], [sig, 1 - sig], rtol=0, atol=1e-14)
    assert abs(orc.lp[0, 0, 0] - lp0) < 1e-13
    # token 1 is stable: its step-1 (dense, uniform) statistics are reused
    assert np.allclose(orc.op[0, 0, 1], [2.75, 2.75], atol=1e-14)
    assert abs(orc.lp[0, 0, 1] - math.log(32)) < 1e-13

    def merged(lp, op):
        w = math.exp(lp)
        return (w * np.asarray(op) + 2 * np.array([1.0, 1.0])) / (w + 2)

    assert np.allclose(res["out"][0, 0, 0], merged(lp0, [sig, 1 - sig]), rtol=1e-6, atol=1e-7)
    assert np.allclose(res["out"][0, 1, 0], merged(math.log(32), [2.75, 2.75]), rtol=1e-6,
                       atol=1e-7)
