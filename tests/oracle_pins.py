"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes the loaded oracle library (so the mutation test
can run the same pins against deliberately broken builds) and raises
AssertionError when the oracle disagrees with:

* library routines that compute the same mathematics independently
  (torch's scaled-dot-product attention and logsumexp in float64, numpy's
  min/max/lexsort, scipy's linear-programming solver);
* closed forms (a merge of two softmaxes is one softmax over both key sets;
  a page whose keys are all equal bounds the score exactly);
* structure planted in the synthetic inputs (the drifting tokens are the
  active ones; needle pages rank high for the query that defines them);
* invariants (the page bound is at least every true score in the page).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import Oracle
from sparse_attention_block_amd import workloads as W


# ---------------------------------------------------------------------------
# float64 references built from library routines

def sdpa64(q, keys, vals, scale):
    """o and log-sum-exp of one query over key/value rows, via torch float64."""
    qt = torch.tensor(np.asarray(q, np.float64))[None, None, None, :]
    kt = torch.tensor(np.asarray(keys, np.float64))[None, None]
    vt = torch.tensor(np.asarray(vals, np.float64))[None, None]
    if kt.shape[2] == 0:
        return np.zeros(q.shape[-1]), -math.inf
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0]
    lse = torch.logsumexp((kt[0, 0] @ qt[0, 0, 0]) * scale, dim=0)
    return o.numpy(), float(lse)


def union_tokens(lay, s, g, pages):
    c = lay.cfg
    P, L, off = c.page_size, int(lay.prefix_len[s]), int(lay.kv_off[s])
    toks = [p * P + j for p in pages for j in range(P) if p * P + j < L]
    idx = off + np.asarray(toks, dtype=np.int64)
    return lay.k_cache[g, idx], lay.v_cache[g, idx]


def close(a, b, rtol, atol, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.abs(a - b) - (atol + rtol * np.abs(b))
    assert np.all(err <= 0), f"{what}: max excess {err.max():.3g}"


def new_oracle(lib, lay, scale=0.0):
    return Oracle(lay.cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache,
                  lib=lib, softmax_scale=scale)


# ---------------------------------------------------------------------------
# a0: page metadata

def pin_page_meta(lib):
    cfg = W.small_case(1, n_seq=3, n_qhead=4, n_kvhead=2, head_dim=64, prefix_lens=(40, 16, 1000))
    lay = W.make_layer(cfg, n_steps=1)
    # Padding past each prefix is zero; make it large so a leak would show.
    for s in range(cfg.n_seq):
        a = int(lay.kv_off[s]) + int(lay.prefix_len[s])
        b = int(lay.kv_off[s]) + (int(lay.prefix_len[s]) + 15) // 16 * 16
        lay.k_cache[:, a:b] = 100.0
    orc = new_oracle(lib, lay)
    kmin, kmax = orc.page_meta()
    P = cfg.page_size
    for s in range(cfg.n_seq):
        L, off = int(lay.prefix_len[s]), int(lay.kv_off[s])
        for p in range((L + P - 1) // P):
            gp = off // P + p
            keys = lay.k_cache[:, off + p * P: off + min((p + 1) * P, L)]
            assert np.array_equal(kmin[:, gp], keys.min(axis=1)), (s, p)
            assert np.array_equal(kmax[:, gp], keys.max(axis=1)), (s, p)


# ---------------------------------------------------------------------------
# a1-a2: locality score and active set

def pin_locality_value(lib):
    cfg = W.small_case(2, n_qhead=4, n_kvhead=1, head_dim=64, dtype="bf16")
    lay = W.make_layer(cfg, n_steps=2)
    orc = new_oracle(lib, lay)
    sc = orc.locality(lay.q[1], lay.q[0])
    ref = ((lay.q[1].astype(np.float64) - lay.q[0]) ** 2).mean(axis=-1)  # [s][t][h]
    close(sc, ref.transpose(0, 2, 1), 1e-5, 1e-30, "locality MSE")


def pin_locality_planted_drift(lib):
    for cid, (B, A, dtype, d) in enumerate([(16, 4, "f32", 64), (32, 8, "bf16", 128),
                                             (16, 2, "bf16", 128)]):
        cfg = W.small_case(10 + cid, n_qhead=8, n_kvhead=2, head_dim=d, block=B, n_active=A,
                           dtype=dtype, prefix_lens=(64,), n_steps=4)
        lay = W.make_layer(cfg)
        orc = new_oracle(lib, lay)
        for t in range(1, cfg.n_steps):
            act = orc.active_set(orc.locality(lay.q[t], lay.q[t - 1]))
            for h in range(cfg.n_qhead):
                assert np.array_equal(act[0, h], lay.drift_tokens[t][0]), (cid, t, h)


def pin_active_set_order_and_ties(lib):
    cfg = W.small_case(3, n_qhead=2, n_kvhead=1, block=8, n_active=3)
    lay = W.make_layer(cfg, n_steps=1, cache=False)
    orc = new_oracle(lib, lay)
    score = np.array([[[0.5, 2.0, 2.0, 0.1, 2.0, 3.0, 0.0, 0.5],
                       [1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0]]], np.float32)
    act = orc.active_set(score)
    # head 0: 3.0 at t5, then the 2.0 tie at t1, t2, t4 -> t1, t2 win; output ascending
    assert act[0, 0].tolist() == [1, 2, 5], act
    assert act[0, 1].tolist() == [0, 1, 2], act
    # brute force with a total order (score desc, token asc) on random ties
    rng = np.random.default_rng(5)
    for _ in range(50):
        sc = rng.integers(0, 4, size=(1, 2, 8)).astype(np.float32)
        for A in (0, 1, 3, 8):
            got = orc.active_set(sc, n_active=A)
            for h in range(2):
                order = np.lexsort((np.arange(8), -sc[0, h]))
                assert got[0, h].tolist() == sorted(order[:A].tolist())


# ---------------------------------------------------------------------------
# a3: page bound

def pin_page_bound_is_box_maximum(lib):
    """The bound equals max of q.x over the box [min, max] (scipy linprog) and is
    at least every key's score in the page."""
    from scipy.optimize import linprog
    import oracle as O
    rng = np.random.default_rng(7)
    for trial in range(40):
        d = 16 if trial % 2 else 8
        keys = W.round_bf16(rng.standard_normal((16, d)).astype(np.float32))
        q = W.round_bf16(rng.standard_normal(d).astype(np.float32))
        if trial % 5 == 0:
            q = np.abs(q)
        if trial % 7 == 0:
            q = -np.abs(q)
        mn, mx = keys.min(0), keys.max(0)
        U = O.page_bound(q, mn, mx, lib=lib)
        res = linprog(-q.astype(np.float64), bounds=list(zip(mn.astype(float), mx.astype(float))),
                      method="highs")
        assert res.status == 0
        lp_max = -res.fun
        assert abs(U - lp_max) <= 1e-5 * (1 + np.abs(q) @ np.maximum(np.abs(mn), np.abs(mx))), \
            (trial, U, lp_max)
        true_max = float((keys.astype(np.float64) @ q.astype(np.float64)).max())
        assert U >= true_max - 1e-5 * (1 + abs(true_max)), (trial, U, true_max)
    # a page of identical keys is bounded by exactly its score
    k = W.round_bf16(rng.standard_normal(32).astype(np.float32))
    q = W.round_bf16(rng.standard_normal(32).astype(np.float32))
    U = O.page_bound(q, k, k, lib=lib)
    assert abs(U - float(q.astype(np.float64) @ k)) <= 1e-5 * (np.abs(q) @ np.abs(k))


# ---------------------------------------------------------------------------
# a4-a5: top-k and union

def _tie_layer(cid, n_active=3, budget=48, prefix_lens=(200, 90)):
    cfg = W.small_case(cid, n_seq=len(prefix_lens), n_qhead=4, n_kvhead=2, head_dim=32,
                       budget=budget, n_active=n_active, dtype="bf16", prefix_lens=prefix_lens)
    lay = W.make_layer(cfg, n_steps=2)
    # Duplicate page 1 into pages 2 and 4 of every sequence: equal bounds -> ties.
    P = cfg.page_size
    for s in range(cfg.n_seq):
        off = int(lay.kv_off[s])
        src = lay.k_cache[:, off + P: off + 2 * P].copy()
        for p in (2, 4):
            if (p + 1) * P <= int(lay.prefix_len[s]):
                lay.k_cache[:, off + p * P: off + (p + 1) * P] = src
    return cfg, lay


def pin_topk_and_union(lib):
    for cid, (A, budget) in enumerate([(3, 48), (1, 16), (4, 64), (2, 512)]):
        cfg, lay = _tie_layer(20 + cid, A, budget)
        orc = new_oracle(lib, lay)
        orc.page_meta()
        act = orc.active_set(orc.locality(lay.q[1], lay.q[0]))
        psel, uidx, ucnt, bounds = orc.select_pages(lay.q[1], act, want_bounds=True)
        k, G, P = budget // cfg.page_size, cfg.group, cfg.page_size
        for s in range(cfg.n_seq):
            npg = (int(lay.prefix_len[s]) + P - 1) // P
            for g in range(cfg.n_kvhead):
                want_union = set()
                for r in range(G * A):
                    h, a = g * G + r // A, r % A
                    U = bounds[s, g, r, :npg]
                    order = np.lexsort((np.arange(npg), -U.astype(np.float64)))
                    want = sorted(order[:min(k, npg)].tolist())
                    got = [x for x in psel[s, h, a].tolist() if x >= 0]
                    assert got == want, (cid, s, g, r, got, want)
                    want_union |= set(want)
                    # the bounds are the oracle's per-page bounds for this row's query
                    t = int(act[s, h, a])
                    q = lay.q[1][s, t, h]
                    off = int(lay.kv_off[s]) // P
                    for p in (0, npg - 1):
                        mn, mx = orc.kmin[g, off + p], orc.kmax[g, off + p]
                        acc = np.float32(0)
                        for i in range(cfg.head_dim):
                            acc = np.float32(acc + np.float32(q[i] * (mx[i] if q[i] >= 0 else mn[i])))
                        assert acc == U[p], (p, acc, U[p])
                assert int(ucnt[s, g]) == len(want_union)
                assert uidx[s, g, :ucnt[s, g]].tolist() == sorted(want_union)
                assert ucnt[s, g] <= min(npg, G * A * k)


def pin_needles_rank_high(lib):
    cfg = W.gqa_16k().replace(prefix_lens=(4096,), cfg_id=90)
    lay = W.make_layer(cfg, n_steps=1)
    orc = new_oracle(lib, lay)
    orc.page_meta()
    hits = 0
    for (s, g), (pages, h, t) in lay.needles.items():
        act = np.zeros((1, cfg.n_qhead, 1), np.int32)
        act[0, :, 0] = t
        psel, _, _, _ = orc.select_pages(lay.q[0], act)
        hits += len(set(psel[0, h, 0].tolist()) & set(pages.tolist()))
    # 8 needle pages per KV head, budget 8 pages: nearly all must be selected.
    assert hits >= 0.9 * 8 * len(lay.needles), hits


# ---------------------------------------------------------------------------
# a6-a10: attention, reuse, merge, first step

def pin_sparse_prefix_equals_sdpa(lib):
    cfg = W.small_case(30, n_seq=2, n_qhead=4, n_kvhead=2, head_dim=32, budget=32, n_active=2,
                       dtype="bf16", prefix_lens=(300, 77), n_steps=2)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    scale = 1 / math.sqrt(cfg.head_dim)
    G = cfg.group
    for s in range(cfg.n_seq):
        for h in range(cfg.n_qhead):
            g = h // G
            pages = res["union_idx"][s, g, :res["union_cnt"][s, g]].tolist()
            keys, vals = union_tokens(lay, s, g, pages)
            for t in res["active"][s, h].tolist():
                o, lse = sdpa64(lay.q[1][s, t, h], keys, vals, scale)
                close(orc.op[s, h, t], o, 1e-9, 1e-12, "o_p")
                assert abs(orc.lp[s, h, t] - lse) < 1e-9, (s, h, t)


def _dense_reference(lay, step, s, h, t, scale, include_prefix=True):
    c = lay.cfg
    g = h // c.group
    L, off = int(lay.prefix_len[s]), int(lay.kv_off[s])
    kp = lay.k_cache[g, off:off + L] if include_prefix else np.zeros((0, c.head_dim), np.float32)
    vp = lay.v_cache[g, off:off + L] if include_prefix else np.zeros((0, c.head_dim), np.float32)
    keys = np.concatenate([kp, lay.k_blk[step][s, :, g]], 0)
    vals = np.concatenate([vp, lay.v_blk[step][s, :, g]], 0)
    return sdpa64(lay.q[step][s, t, h], keys, vals, scale)


def bf16_nearest(got, ref, what):
    """got must be a bf16 value nearest to the float64 reference ref."""
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(W.round_bf16(got), got), f"{what}: not bf16"
    want = W.round_bf16(ref.astype(np.float32)).astype(np.float64)
    ok = np.abs(got - ref) <= np.abs(want - ref) + 1e-9 * np.abs(ref) + 1e-30
    assert np.all(ok), f"{what}: not the nearest bf16 ({np.argwhere(~ok)[:3].tolist()})"


def _check_out(cfg, got, ref, what):
    if cfg.dtype == "bf16":
        bf16_nearest(got, ref, what)
    else:
        close(got, ref, 1e-6, 1e-7, what)


def pin_dense_first_step_equals_attention(lib):
    for cid, (dtype, lens, G) in enumerate([("f32", (200,), 4), ("bf16", (123, 16), 2),
                                            ("bf16", (0, 50), 1)]):
        cfg = W.small_case(40 + cid, n_seq=len(lens), n_qhead=2 * G, n_kvhead=2, head_dim=32,
                           dtype=dtype, prefix_lens=lens, n_steps=1)
        lay = W.make_layer(cfg)
        orc = new_oracle(lib, lay)
        out = orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
        scale = 1 / math.sqrt(cfg.head_dim)
        for s in range(cfg.n_seq):
            for h in range(cfg.n_qhead):
                g = h // cfg.group
                L, off = int(lay.prefix_len[s]), int(lay.kv_off[s])
                for t in range(cfg.block):
                    o, _ = _dense_reference(lay, 0, s, h, t, scale)
                    _check_out(cfg, out[s, t, h], o, f"dense {cid} {s} {h} {t}")
                    op, lp = sdpa64(lay.q[0][s, t, h], lay.k_cache[g, off:off + L],
                                    lay.v_cache[g, off:off + L], scale)
                    close(orc.op[s, h, t], op, 1e-9, 1e-12, "dense o_p")
                    if L == 0:
                        assert orc.lp[s, h, t] == -math.inf
                    else:
                        assert abs(orc.lp[s, h, t] - lp) < 1e-9


def pin_dense_row_equals_attention(lib):
    cfg = W.small_case(45, n_seq=2, n_qhead=4, n_kvhead=2, head_dim=32, dtype="bf16",
                       prefix_lens=(150, 0), n_steps=1)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    scale = 1 / math.sqrt(cfg.head_dim)
    for (s, h, t) in [(0, 0, 0), (0, 3, 15), (1, 2, 7), (0, 1, 9)]:
        op, lp, out = orc.dense_row(lay.q[0], lay.k_blk[0], lay.v_blk[0], s, h, t)
        o, _ = _dense_reference(lay, 0, s, h, t, scale)
        bf16_nearest(out, o, f"dense row {s} {h} {t}")
        g = h // cfg.group
        L, off = int(lay.prefix_len[s]), int(lay.kv_off[s])
        o_p, l_p = sdpa64(lay.q[0][s, t, h], lay.k_cache[g, off:off + L],
                          lay.v_cache[g, off:off + L], scale)
        close(op, o_p, 1e-9, 1e-12, "dense row o_p")
        assert (lp == l_p == -math.inf) or abs(lp - l_p) < 1e-9


def pin_all_active_full_budget_is_dense(lib):
    """|A| = B and a budget covering the prefix: a LoSA step is dense attention."""
    for cid, (dtype, lens) in enumerate([("bf16", (96, 40)), ("f32", (64,))]):
        cfg = W.small_case(50 + cid, n_seq=len(lens), n_qhead=4, n_kvhead=2, head_dim=32,
                           block=8, n_active=8, budget=128, dtype=dtype, prefix_lens=lens,
                           n_steps=3, n_drift=2)
        lay = W.make_layer(cfg)
        orc = new_oracle(lib, lay)
        orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
        scale = 1 / math.sqrt(cfg.head_dim)
        for step in (1, 2):
            res = orc.step(lay.q[step], lay.q[step - 1], lay.k_blk[step], lay.v_blk[step])
            for s in range(cfg.n_seq):
                for h in range(cfg.n_qhead):
                    for t in range(cfg.block):
                        o, _ = _dense_reference(lay, step, s, h, t, scale)
                        _check_out(cfg, res["out"][s, t, h], o, f"all-active {cid} {step}")


def pin_stable_reuse_and_merge(lib):
    """|A| = 0: the cache is untouched and out = softmax-merge(cache, new suffix)."""
    cfg = W.small_case(60, n_qhead=4, n_kvhead=2, head_dim=32, n_active=0, dtype="f32",
                       prefix_lens=(160,), n_steps=2, n_drift=3)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    op0, lp0 = orc.op.copy(), orc.lp.copy()
    res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    assert np.array_equal(orc.op, op0) and np.array_equal(orc.lp, lp0)
    scale = 1 / math.sqrt(cfg.head_dim)
    for h in range(cfg.n_qhead):
        g = h // cfg.group
        for t in range(cfg.block):
            os_, ls = sdpa64(lay.q[1][0, t, h], lay.k_blk[1][0, :, g], lay.v_blk[1][0, :, g], scale)
            # closed form of one softmax over the union of both key sets
            w_p = 1.0 / (1.0 + math.exp(ls - lp0[0, h, t]))
            want = w_p * op0[0, h, t] + (1 - w_p) * os_
            close(res["out"][0, t, h], want, 1e-6, 1e-7, "reuse merge")


def pin_mixed_step_rows(lib):
    """In a partial step, active rows hold fresh union statistics and stable rows
    the previous ones; every output is the merge of its row's cache entry."""
    cfg = W.small_case(61, n_seq=2, n_qhead=4, n_kvhead=2, head_dim=32, n_active=3, budget=32,
                       dtype="f32", prefix_lens=(200, 48), n_steps=2)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    op0, lp0 = orc.op.copy(), orc.lp.copy()
    res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    scale = 1 / math.sqrt(cfg.head_dim)
    for s in range(cfg.n_seq):
        for h in range(cfg.n_qhead):
            g = h // cfg.group
            act = set(res["active"][s, h].tolist())
            for t in range(cfg.block):
                if t not in act:
                    assert np.array_equal(orc.op[s, h, t], op0[s, h, t])
                    assert orc.lp[s, h, t] == lp0[s, h, t]
                os_, ls = sdpa64(lay.q[1][s, t, h], lay.k_blk[1][s, :, g], lay.v_blk[1][s, :, g],
                                 scale)
                w_p = 1.0 / (1.0 + math.exp(ls - orc.lp[s, h, t]))
                close(res["out"][s, t, h], w_p * orc.op[s, h, t] + (1 - w_p) * os_, 1e-6, 1e-7,
                      "mixed merge")


def pin_naive_sparse_per_query(lib):
    cfg = W.small_case(70, n_qhead=4, n_kvhead=2, head_dim=32, budget=32, dtype="bf16",
                       prefix_lens=(180,), n_steps=1)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    orc.page_meta()
    orc.naive_sparse_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    scale = 1 / math.sqrt(cfg.head_dim)
    B, G = cfg.block, cfg.group
    for h in range(cfg.n_qhead):
        act = np.zeros((1, cfg.n_qhead, 1), np.int32)
        for t in range(B):
            act[0, :, 0] = t
            psel, _, _, _ = orc.select_pages(lay.q[0], act)
            keys, vals = union_tokens(lay, 0, h // G, psel[0, h, 0].tolist())
            o, lse = sdpa64(lay.q[0][0, t, h], keys, vals, scale)
            close(orc.op[0, h, t], o, 1e-9, 1e-12, "naive o_p")
            assert abs(orc.lp[0, h, t] - lse) < 1e-9


# ---------------------------------------------------------------------------
# reading variants (flags)

ROW_MASK, SHARED_ACTIVE, NO_WRITEBACK = 1, 2, 4


def pin_row_mask_attends_own_pages(lib):
    """ROW_MASK: each active row's (o_p, L_p) is attention over the tokens of the
    pages it selected itself (torch float64), and some row's pages differ from
    its KV head's union (so the variant is exercised)."""
    cfg = W.small_case(80, n_seq=2, n_qhead=4, n_kvhead=2, head_dim=32, budget=32, n_active=2,
                       dtype="bf16", prefix_lens=(300, 77), n_steps=2, flags=ROW_MASK)
    lay = W.make_layer(cfg)
    orc = new_oracle(lib, lay)
    orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    scale = 1 / math.sqrt(cfg.head_dim)
    narrower = 0
    for s in range(cfg.n_seq):
        for h in range(cfg.n_qhead):
            g = h // cfg.group
            for a, t in enumerate(res["active"][s, h].tolist()):
                own = [p for p in res["page_sel"][s, h, a].tolist() if p >= 0]
                narrower += len(own) < int(res["union_cnt"][s, g])
                keys, vals = union_tokens(lay, s, g, own)
                o, lse = sdpa64(lay.q[1][s, t, h], keys, vals, scale)
                close(orc.op[s, h, t], o, 1e-9, 1e-12, "row-mask o_p")
                assert abs(orc.lp[s, h, t] - lse) < 1e-9, (s, h, t)
    assert narrower > 0


def pin_shared_active_set_constructed(lib):
    """SHARED_ACTIVE: one set per sequence from the head-summed locality.  Queries
    are built so that only dimension 0 changes, by hand-chosen amounts: token 3
    by 1 in all four heads, token 7 by 1.5 in head 0, token 9 by 1.9 in head 1,
    token 12 by 1.2 in heads 0 and 1.  Summed over heads: 4, 2.25, 3.61, 2.88
    (over d), so |A| = 2 keeps tokens 3 and 9 in every head, while head 0 alone
    would keep 7 and 12; |A| = 1 keeps token 3 (a maximum over heads, or a sum
    missing any one head, would keep token 9)."""
    cfg = W.small_case(81, n_qhead=4, n_kvhead=2, head_dim=32, budget=32, n_active=2,
                       dtype="f32", prefix_lens=(96,), n_steps=2)
    lay = W.make_layer(cfg)
    q_prev = lay.q[0].copy()
    q_prev[..., 0] = 0.0
    q_t = q_prev.copy()
    for t, h, m in [(3, 0, 1.0), (3, 1, 1.0), (3, 2, 1.0), (3, 3, 1.0), (7, 0, 1.5),
                    (9, 1, 1.9), (12, 0, 1.2), (12, 1, 1.2)]:
        q_t[0, t, h, 0] = np.float32(m)
    for flags, n_act, want in [(SHARED_ACTIVE, 2, [[3, 9]] * 4), (SHARED_ACTIVE, 1, [[3]] * 4),
                               (0, 2, [[7, 12], [9, 12], [0, 3], [0, 3]])]:
        c2 = cfg.replace(flags=flags, n_active=n_act)
        orc = Oracle(c2, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache,
                     lib=lib)
        orc.dense_first_step(q_prev, lay.k_blk[0], lay.v_blk[0])
        res = orc.step(q_t, q_prev, lay.k_blk[1], lay.v_blk[1])
        assert res["active"][0].tolist() == want, (flags, res["active"][0].tolist())


def pin_no_writeback_keeps_cache(lib):
    """NO_WRITEBACK: the step leaves the (o_p, L_p) cache bit for bit as the dense
    step left it, and its output equals the plain reading's (the fresh
    statistics of the active rows serve that step either way)."""
    cfg = W.small_case(82, n_seq=2, n_qhead=4, n_kvhead=2, head_dim=32, budget=32, n_active=3,
                       dtype="bf16", prefix_lens=(200, 48), n_steps=2)
    lay = W.make_layer(cfg)
    outs = []
    for flags in (NO_WRITEBACK, 0):
        orc = new_oracle(lib, lay) if flags == 0 else Oracle(
            cfg.replace(flags=flags), lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache,
            lay.v_cache, lib=lib)
        orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
        op0, lp0 = orc.op.copy(), orc.lp.copy()
        res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
        if flags:
            assert np.array_equal(orc.op, op0) and np.array_equal(orc.lp, lp0)
        else:
            assert not np.array_equal(orc.lp, lp0)
        outs.append(res["out"])
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# hand-worked values that only the ascending fp32 chains reproduce

GOLDEN_DIR = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def chain_order_golden():
    import json
    with open(__import__("os").path.join(GOLDEN_DIR, "chain_order.json")) as f:
        return json.load(f)


def chain_order_layer(g):
    """The golden's inputs placed into a small bf16 layer (every other value drawn)."""
    sh = g["shape"]
    cfg = W.small_case(390, dtype="bf16", head_dim=sh["head_dim"], block=sh["block"],
                       n_active=sh["n_active"], budget=sh["budget"],
                       prefix_lens=(sh["prefix_len"],), n_kvhead=1, n_qhead=sh["n_qhead"],
                       n_steps=2)
    lay = W.make_layer(cfg)
    P, d = cfg.page_size, cfg.head_dim
    for pg in (g["page_a"], g["page_b"]):
        k = np.zeros(d, np.float32)
        k[:len(pg["key"])] = pg["key"]
        lay.k_cache[0, pg["page"] * P:(pg["page"] + 1) * P] = k
    for row in (g["bound_row"], g["locality_row"]):
        q = np.zeros(d, np.float32)
        q[:len(row["q_t"])] = row["q_t"]
        if row.get("fill_ones"):
            q[len(row["q_t"]):] = 1.0
        lay.q[1][0, row["token"], row["head"]] = q
        lay.q[0][0, row["token"], row["head"]] = 0.0
    return lay, cfg


def pin_chain_order_golden(lib):
    g = chain_order_golden()
    lay, cfg = chain_order_layer(g)
    orc = new_oracle(lib, lay)
    orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
    res = orc.step(lay.q[1], lay.q[0], lay.k_blk[1], lay.v_blk[1])
    e, lr, br = g["expected"], g["locality_row"], g["bound_row"]
    got = float(res["locality"][0, lr["head"], lr["token"]])
    assert got == e["locality"], f"locality chain {got} != {e['locality']}"
    act = list(res["active"][0, br["head"]])
    assert br["token"] in act, "the bound row must be active"
    sel = res["page_sel"][0, br["head"], act.index(br["token"])].tolist()
    assert sel == e["page_sel"], f"page bound chain selects {sel}, not {e['page_sel']}"


ALL_PINS = [
    pin_chain_order_golden,
    pin_page_meta, pin_locality_value, pin_locality_planted_drift, pin_active_set_order_and_ties,
    pin_page_bound_is_box_maximum, pin_topk_and_union, pin_needles_rank_high,
    pin_sparse_prefix_equals_sdpa, pin_dense_first_step_equals_attention,
    pin_dense_row_equals_attention,
    pin_all_active_full_budget_is_dense, pin_stable_reuse_and_merge, pin_mixed_step_rows,
    pin_naive_sparse_per_query, pin_row_mask_attends_own_pages, pin_shared_active_set_constructed,
    pin_no_writeback_keeps_cache,
]
