#!/usr/bin/env python3
"""Benchmark of LoSA per-denoising-step attention on one MI355X.

Workload: the long-context layer shape (prefix L = 65536 tokens, block B = 16,
32 query / 8 KV heads, head_dim 128, bf16, budget 128 tokens, |A| = 4, needle
pages, 8 denoising steps per block).  One bench step = one block: a forced
dense first step and 7 LoSA steps, for each of --layers independent layers
run in model order (step-major, layer-minor), so a layer's metadata and KV are
not re-read from the on-die cache between its steps (16 layers x ~24 MiB of
sparse-step traffic exceed the 256 MB MALL).  The page metadata of the fixed
prefix is built before timing (it changes once per committed block).

Prints one JSON line: value = attention microseconds per (layer, denoising
step), amortised over the block (dense first step included), from K timed
replays of the block captured as two HIP graphs, its dense first steps and its
LoSA steps -- the same launches with no host launch overhead, checked bit for
bit against an eager block (--no-graph times eager launches; the eager rate is
reported beside).  Events before, between and after the two graphs give
dense_step_us and sparse_step_us, so value = (dense + 7 sparse) / 8 up to the
events' own cost.  Per-kernel durations come from the committed rocprofv3
summary of this workload (profiles/kernels_long_64k_b<budget>_a<|A|>.json) wherever the
digest of the kernel's sources matches, else from HIP events the library
records between its launches in a second timed pass of K blocks (both are
reported); then the roofline of the dominant kernel, and the CPU oracle timed
on one layer-block of the same workload, on all host cores and on one.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention us per block-step + HBM GB/s, 64K ctx, B=16, budget 128"
PEAK_HBM_GBPS = 8000.0
STEPS_PER_BLOCK = 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_profile(kernel_tag: str):
    """HBM bytes per launch from the committed rocprofv3 counter passes, if they were
    taken on the current kernel sources (else None)."""
    from sparse_attention_block_amd.profiling import KERNEL_TAGS, source_digest

    path = os.path.join(ROOT, "profiles", f"counters_{kernel_tag}.json")
    if kernel_tag not in KERNEL_TAGS or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(KERNEL_TAGS[kernel_tag][1]):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, lay):
    """The oracle, as it stands, on one layer-block of the same workload: once on
    all host cores (row-parallel dense step, one thread per KV head in the LoSA
    steps: the same per-row and per-head oracle calls, the same bits), once on
    one thread."""
    from oracle import Oracle, host_threads

    def run(threaded):
        orc = Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
        orc.page_meta()
        t0 = time.perf_counter()
        if threaded:
            orc.dense_first_step_threaded(lay.q[0], lay.k_blk[0], lay.v_blk[0])
        else:
            orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])
        for t in range(1, STEPS_PER_BLOCK):
            step = orc.step_threaded if threaded else orc.step
            step(lay.q[t], lay.q[t - 1], lay.k_blk[t], lay.v_blk[t])
        return time.perf_counter() - t0

    n = host_threads()
    sec_all = run(True)
    sec_one = run(False)
    per = lambda sec: sec * 1e6 / STEPS_PER_BLOCK
    return {"value": per(sec_all), "unit": "us per block-step", "cores": n, "kind": "oracle",
            "value_1_thread": per(sec_one),
            "sample": f"one layer, one {STEPS_PER_BLOCK}-step block (1 dense + "
                      f"{STEPS_PER_BLOCK - 1} LoSA steps) of the same 64K workload: {sec_all:.2f} s "
                      f"on {n} threads (dense rows over {n} threads, LoSA steps one thread per "
                      f"KV head, {cfg.n_kvhead}), {sec_one:.2f} s on one thread"}


def rocprof_durations(workload: str):
    """Average kernel durations from the committed rocprofv3 trace summary of this
    workload, per kernel tag, kept only where the digest of the kernel's sources
    still matches (else the summary describes other code)."""
    from sparse_attention_block_amd.profiling import KERNEL_TAGS, source_digest

    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.json")
    if not os.path.exists(path):
        return {}, None
    with open(path) as f:
        rec = json.load(f)
    out = {}
    for tag, k in rec.get("kernels", {}).items():
        if tag in KERNEL_TAGS and k.get("source_digest") == source_digest(KERNEL_TAGS[tag][1]):
            out[tag] = k["avg_us"]
    return out, os.path.relpath(path, ROOT)


def floors_record(floors, rp):
    """The floors of this run (event-bracketed), with the probe kernels' own
    durations from the committed rocprofv3 summary where its digest matches."""
    rec = dict(floors)
    rec["empty_kernel_us_rocprof"] = rp.get("probe_empty")
    for mib, _ in FLOOR_READS:
        r = rec["read"][f"{mib}MiB"]
        us = rp.get(f"probe_read_{mib}MiB")
        r["us_rocprof"] = us
        r["gbps_rocprof"] = (mib << 20) / (us * 1e-6) / 1e9 if us else None
        r["frac_rocprof"] = r["gbps_rocprof"] / PEAK_HBM_GBPS if us else None
    if "gather" in rec:
        us = rp.get("probe_gather")
        rec["gather"] = dict(rec["gather"], us_rocprof=us,
                             gbps_rocprof=rec["gather"]["bytes"] / (us * 1e-6) / 1e9 if us else None)
    return rec


# ---------------------------------------------------------------------------
# --sweep: the |A| x budget sweep, the KV-union density study against a
# QUEST-style step (every block token active, same inputs) and a dense step
# every step, other workload shapes, the 36-layer trace, and latency floors.

SWEEP_LAYERS = 8          # layer replicas per 64K case (8 x 272 MiB defeats the 256 MB MALL)


def _selftest():
    from sparse_attention_block_amd.build import SELFTEST_LIB

    st = ctypes.CDLL(SELFTEST_LIB)
    st.losa_selftest_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_int, ctypes.c_void_p]
    st.losa_selftest_empty.argtypes = [ctypes.c_void_p]
    st.losa_selftest_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_void_p]
    st.losa_selftest_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return st


FLOOR_READS = ((1, 256), (8, 512), (16, 1024), (64, 2048))  # (MiB, workgroups)
FLOOR_REPS = 8
# the sparse prefix pass's memory pattern on the headline layer: 28 chunks of
# 4 union pages for each of 8 KV heads, every page 8 KiB (keys and values),
# drawn without repeats from a cold 32 MiB window per repetition
FLOOR_GATHER_BLOCKS = 224
FLOOR_GATHER_WINDOW = 32 << 20


def latency_floors(hip, stream, reps=50):
    """Floors for reading the kernels' durations: an empty kernel (back to back,
    and between two events), an empty event pair, and pure reads of 1/8/16/64 MiB
    (the selftest library's k_probe_read, FLOOR_REPS of each).  Every read takes a
    region of a pool that no kernel has touched since the pool was filled, at
    least 1 GiB of writes earlier, so none is served from the 256 MB MALL or an
    L2.  Durations here are event-bracketed (about 1 us more than the kernel);
    the committed rocprofv3 summary of the bench command holds the same
    kernels' own durations (k_empty, k_probe_read<MiB>)."""
    import torch

    st = _selftest()
    out = {}
    e0, e1 = hip.event(), hip.event()
    for _ in range(20):
        st.losa_selftest_empty(stream)
    torch.cuda.synchronize()
    hip.record(e0, stream)
    for _ in range(reps):
        assert st.losa_selftest_empty(stream) == 0
    hip.record(e1, stream)
    torch.cuda.synchronize()
    out["empty_kernel_back_to_back_us"] = hip.ms(e0, e1) * 1e3 / reps
    evs = [hip.event() for _ in range(2 * 50)]
    for i in range(50):
        hip.record(evs[2 * i], stream)
        st.losa_selftest_empty(stream)
        hip.record(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    out["empty_kernel_between_events_us"] = float(sorted(
        hip.ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(50))[25])
    evs = [hip.event() for _ in range(2 * 50)]
    for i in range(50):
        hip.record(evs[2 * i], stream)
        hip.record(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    out["empty_event_pair_us"] = float(sorted(
        hip.ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(50))[25])
    # a 2 GiB pool, filled; then 512 MiB between 1 and 1.5 GiB are read (in
    # 32 MiB pieces, k_probe_read<0>), which evicts the fill's dirty tail from
    # the MALL, so that no write-back runs beside the timed reads; those read
    # the first GiB, each byte once
    pool_bytes = 2048 << 20
    pool = torch.ones(pool_bytes // 4, dtype=torch.float32, device="cuda")
    for i in range(16):
        assert st.losa_selftest_read(pool.data_ptr() + (1024 << 20) + (i << 25), 32 << 20, 1024, 0,
                                     None, stream) == 0
    need = sum(m << 20 for m, _ in FLOOR_READS) * FLOOR_REPS
    assert need <= 1024 << 20
    off = 0
    reads = {}
    for mib, blocks in FLOOR_READS:
        nb = mib << 20
        evs = [hip.event() for _ in range(2 * FLOOR_REPS)]
        torch.cuda.synchronize()
        for r in range(FLOOR_REPS):
            hip.record(evs[2 * r], stream)
            assert st.losa_selftest_read(pool.data_ptr() + off, nb, blocks, 0, None, stream) == 0
            hip.record(evs[2 * r + 1], stream)
            off += nb
        torch.cuda.synchronize()
        us = sorted(hip.ms(evs[2 * r], evs[2 * r + 1]) * 1e3 for r in range(FLOOR_REPS))
        med = float(us[len(us) // 2])
        reads[f"{mib}MiB"] = {"workgroups": blocks, "us_events": med,
                              "gbps_events": nb / (med * 1e-6) / 1e9}
    out["read"] = reads
    # gathers (k_probe_gather): a page list copied into place just before (as
    # the selection kernel writes the rows' page lists), then the
    # pages, then partial-sized stores; each repetition in a window no kernel
    # has touched
    import numpy as np
    rng = np.random.default_rng(20260)
    n_pg = 4 * FLOOR_GATHER_BLOCKS
    win_pages = FLOOR_GATHER_WINDOW // 8192
    assert off + FLOOR_REPS * FLOOR_GATHER_WINDOW <= 1024 << 20
    lists = np.stack([np.sort(rng.choice(win_pages, n_pg, replace=False)) +
                      (off + r * FLOOR_GATHER_WINDOW) // 8192 for r in range(FLOOR_REPS)])
    assert lists.max() < pool_bytes // 8192
    list_src = torch.from_numpy(lists.astype(np.int32)).cuda()
    list_dst = torch.empty(n_pg, dtype=torch.int32, device="cuda")
    part = torch.empty(FLOOR_GATHER_BLOCKS * 16 * 130, dtype=torch.float32, device="cuda")
    evs = [hip.event() for _ in range(2 * FLOOR_REPS)]
    torch.cuda.synchronize()
    for r in range(FLOOR_REPS):
        list_dst.copy_(list_src[r])  # a device copy on the same (current) stream
        hip.record(evs[2 * r], stream)
        assert st.losa_selftest_gather(list_dst.data_ptr(), pool.data_ptr(), pool_bytes,
                                       part.data_ptr(), FLOOR_GATHER_BLOCKS, stream) == 0
        hip.record(evs[2 * r + 1], stream)
    torch.cuda.synchronize()
    us = sorted(hip.ms(evs[2 * r], evs[2 * r + 1]) * 1e3 for r in range(FLOOR_REPS))
    out["gather"] = {"workgroups": FLOOR_GATHER_BLOCKS, "pages": n_pg, "bytes": n_pg * 8192,
                     "us_events": float(us[len(us) // 2])}
    del pool
    torch.cuda.empty_cache()
    return out


def page_meta_times(hip, lay, kv, reps):
    """Full metadata build of a layer vs the update after one committed block of
    16 tokens (losa_update_page_meta), over the layer replicas, each captured as
    one HIP graph so that host launch cost does not enter."""
    import numpy as np
    import torch

    from sparse_attention_block_amd import binding as L
    from sparse_attention_block_amd.layer import LayerState

    c = lay.cfg
    new_len = np.asarray(lay.prefix_len, np.int32)
    old_len = np.maximum(new_len - c.block, 0).astype(np.int32)
    states = [LayerState(n_seq=c.n_seq, block=c.block, n_qhead=c.n_qhead, n_kvhead=c.n_kvhead,
                         head_dim=c.head_dim, budget_tokens=c.budget, n_active=c.n_active,
                         dtype=c.dtype, k_cache=k, v_cache=v, kv_off=lay.kv_off,
                         prefix_len=new_len) for k, v in kv]
    first = torch.as_tensor(old_len).cuda()
    gst = torch.cuda.Stream()
    sid = gst.cuda_stream

    def full():
        for st in states:
            L.losa_build_page_meta(st.shape, st.k_cache, st.kv_off, st.prefix_len, st.page_meta,
                                   sid)

    def update():
        for st in states:
            L.losa_update_page_meta(st.shape, st.k_cache, st.kv_off, st.prefix_len, first,
                                    c.block, st.page_meta, sid)

    def timed(fn):
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        g = hip.capture(sid, fn)
        hip.launch(g, sid)
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sid)
        for _ in range(reps):
            hip.launch(g, sid)
        hip.record(e1, sid)
        torch.cuda.synchronize()
        return hip.ms(e0, e1) * 1e3 / (reps * len(states))

    full_us = timed(full)
    upd_us = timed(update)
    k_bytes = c.n_kvhead * int(new_len.sum()) * c.head_dim * (2 if c.dtype == "bf16" else 4)
    del states
    torch.cuda.empty_cache()
    return {"full_build_us": full_us, "full_build_gbps_on_keys": k_bytes / (full_us * 1e-6) / 1e9,
            "commit_16_tokens_us": upd_us}


def measure_case(hip, lay_kv, inputs_of, *, cfg, budget, active_of, dense_every_step, reps,
                 union_layers=(0,), flags=0, page_table=None):
    """Time one case over the device KV replicas ``lay_kv`` = (layer, [(k, v), ...]).

    inputs_of(li) -> (q, k_blk, v_blk) device tensor lists per step for layer li.
    Returns per-(layer, step) microseconds of the dense and of the other steps,
    the mean union size (pages, all KV heads) of each layer in ``union_layers``
    and the median per-stage event durations of the other steps."""
    import numpy as np
    import torch

    from sparse_attention_block_amd import binding as L
    from sparse_attention_block_amd.layer import LayerState

    lay, kv = lay_kv
    S_steps = cfg.n_steps
    layers = []
    for li, (k, v) in enumerate(kv):
        ls = LayerState(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead,
                        n_kvhead=cfg.n_kvhead, head_dim=cfg.head_dim, budget_tokens=budget,
                        n_active=active_of(li), dtype=cfg.dtype, k_cache=k, v_cache=v,
                        kv_off=lay.kv_off, prefix_len=lay.prefix_len, flags=flags,
                        page_table=page_table)
        ls.build_page_meta()
        layers.append(ls)
    # union sizes over the block (from the library's debug outputs)
    union = {}
    for li in ([] if dense_every_step else union_layers):
        ls0, (q, kb, vb) = layers[li], inputs_of(li)
        dbg = L.Debug.alloc(ls0.shape)
        ls0.dense_first_step(q[0], kb[0], vb[0])
        counts = []
        for t in range(1, S_steps):
            ls0.step(q[t], q[t - 1], kb[t], vb[t], debug=dbg)
            torch.cuda.synchronize()
            counts.append(float(dbg.union_cnt.sum().item()))
        union[li] = float(np.mean(counts))
        del dbg
    gst = torch.cuda.Stream()
    sid = gst.cuda_stream
    dense_calls, step_calls = [], []
    for li, ls in enumerate(layers):
        q, kb, vb = inputs_of(li)
        dense_calls.append(ls.prepare_dense_first_step(q[0], kb[0], vb[0], stream=sid))
    for t in range(1, S_steps):
        for li, ls in enumerate(layers):
            q, kb, vb = inputs_of(li)
            step_calls.append(ls.prepare_dense_first_step(q[t], kb[t], vb[t], stream=sid)
                              if dense_every_step else
                              ls.prepare_step(q[t], q[t - 1], kb[t], vb[t], stream=sid))
    run = lambda cs: [c() for c in cs]
    for _ in range(2):
        run(dense_calls)
        run(step_calls)
    torch.cuda.synchronize()
    g_dense = hip.capture(sid, lambda: run(dense_calls))
    g_steps = hip.capture(sid, lambda: run(step_calls))

    def timed(g):
        e0, e1 = hip.event(), hip.event()
        hip.launch(g, sid)
        torch.cuda.synchronize()
        hip.record(e0, sid)
        for _ in range(reps):
            hip.launch(g, sid)
        hip.record(e1, sid)
        torch.cuda.synchronize()
        return hip.ms(e0, e1) * 1e3 / reps

    dense_us = timed(g_dense) / len(layers)
    step_us = timed(g_steps) / (len(layers) * (S_steps - 1))
    # per-stage durations of the non-first steps, from the library's stage events
    names = ["prepare", "score", "select", "prefix", "finish"]
    evs = [[hip.event() for _ in range(L.LOSA_STAGE_EVENTS)] for _ in step_calls]
    for c, e in zip(step_calls, evs):
        c.set_events(e)
    run(dense_calls)
    run(step_calls)
    torch.cuda.synchronize()
    for c in step_calls:
        c.set_events(None)
    stage = {n: float(np.median([hip.ms(e[i], e[i + 1]) * 1e3 for e in evs]))
             for i, n in enumerate(names)}
    del layers, dense_calls, step_calls
    torch.cuda.empty_cache()
    return {"dense_us": dense_us, "step_us": step_us, "stage_us": stage,
            "union_pages": union.get(union_layers[0]), "union_by_layer": union}


def sweep(args):
    import numpy as np
    import torch

    from sparse_attention_block_amd import binding as L
    from sparse_attention_block_amd import workloads as W
    from sparse_attention_block_amd.hiprt import HipRuntime
    from sparse_attention_block_amd.layer import to_device

    L.load()
    torch.cuda.set_device(0)
    hip = HipRuntime()
    stream = torch.cuda.current_stream().cuda_stream
    t_start = time.perf_counter()
    floors = latency_floors(hip, stream)
    log(f"[sweep] floors {json.dumps(floors)}")
    rows = []

    def dev_inputs(lay, dtype):
        return ([to_device(x, dtype) for x in lay.q], [to_device(x, dtype) for x in lay.k_blk],
                [to_device(x, dtype) for x in lay.v_blk])

    def replicas(lay, n):
        k0, v0 = to_device(lay.k_cache, lay.cfg.dtype), to_device(lay.v_cache, lay.cfg.dtype)
        return [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(n - 1)]

    def bytes_model(cfg, union_pages, n_active):
        sT = 2 if cfg.dtype == "bf16" else 4
        Hk, d, P, S, B, Hq = cfg.n_kvhead, cfg.head_dim, cfg.page_size, cfg.n_seq, cfg.block, cfg.n_qhead
        n_pages = sum((L_ + P - 1) // P for L_ in cfg.prefix_lens)
        meta = Hk * n_pages * 2 * d * sT
        union = (union_pages if union_pages is not None else Hk * n_pages) * P * 2 * d * sT
        small = (2 * S * B * Hq * d * sT + 2 * S * B * Hk * d * sT + S * Hq * B * (d + 1) * 4
                 + S * Hq * n_active * (d + 1) * 4 + S * B * Hq * d * sT)
        return meta, union, small, Hk * n_pages

    def add_row(group, label, cfg, budget, n_active, n_layers, res, dense_mode):
        meta, union, small, pages_all = bytes_model(cfg, res["union_pages"], n_active)
        st = res["stage_us"]
        row = {"group": group, "case": label, "workload": cfg.name, "budget": budget,
               "n_active": n_active, "layers": n_layers, "mode": "dense" if dense_mode else "losa",
               "dense_step_us": res["dense_us"], "step_us": res["step_us"],
               "block_us": (res["dense_us"] + (cfg.n_steps - 1) * res["step_us"]) / cfg.n_steps,
               "stage_us": st}
        if not dense_mode:
            up = res["union_pages"]
            row.update({
                "union_pages_per_kv_head": up / (cfg.n_seq * cfg.n_kvhead),
                "density": up / pages_all,
                "union_bytes": union, "step_bytes": meta + union + small,
                "step_gbps": (meta + union + small) / (res["step_us"] * 1e-6) / 1e9,
                "prefix_gbps_on_union": union / (st["prefix"] * 1e-6) / 1e9,
                "prefix_frac": union / (st["prefix"] * 1e-6) / 1e9 / PEAK_HBM_GBPS})
        rows.append(row)
        log(f"[sweep] {group} {label}: step {row['step_us']:.2f} us, dense {row['dense_step_us']:.2f} us"
            + (f", union/head {row['union_pages_per_kv_head']:.1f}, prefix {st['prefix']:.2f} us"
               if not dense_mode else ""))

    # 64K: |A| x budget, QUEST-style (all 16 tokens active on the |A|=4 inputs), dense
    base = W.long_64k(128, 4)
    lay = W.make_layer(base, n_steps=base.n_steps)
    kv = (lay, replicas(lay, SWEEP_LAYERS))
    for budget in (128, 256):
        for a in (2, 4, 8):
            c = W.long_64k(budget, a)
            li = W.make_layer(c, n_steps=c.n_steps, cache=False)
            inp = dev_inputs(li, c.dtype)
            res = measure_case(hip, kv, lambda i: inp, cfg=c, budget=budget, active_of=lambda i: a,
                               dense_every_step=False, reps=args.steps)
            add_row("64K", f"LoSA |A|={a}", c, budget, a, SWEEP_LAYERS, res, False)
        inp4 = dev_inputs(lay, base.dtype)
        res = measure_case(hip, kv, lambda i: inp4, cfg=base, budget=budget,
                           active_of=lambda i: base.block, dense_every_step=False, reps=args.steps)
        add_row("64K", "QUEST-style (all 16 tokens active, |A|=4 inputs)", base, budget,
                base.block, SWEEP_LAYERS, res, False)
        # naive per-query sparse attention: every token its own pages (row masks),
        # no reuse; the union of all 16 tokens' pages is what it loads
        res = measure_case(hip, kv, lambda i: inp4, cfg=base, budget=budget,
                           active_of=lambda i: base.block, dense_every_step=False, reps=args.steps,
                           flags=1)
        add_row("64K", "naive per-query (all 16 tokens active, own pages)", base, budget,
                base.block, SWEEP_LAYERS, res, False)
    inp4 = dev_inputs(lay, base.dtype)
    res = measure_case(hip, kv, lambda i: inp4, cfg=base, budget=128, active_of=lambda i: 4,
                       dense_every_step=True, reps=args.steps)
    add_row("64K", "dense every step", base, 128, 4, SWEEP_LAYERS, res, True)
    # the reading variants (losa_shape.flags) on the same inputs
    for flags, label in ((1, "row mask"), (2, "shared active set"), (4, "no write-back")):
        res = measure_case(hip, kv, lambda i: inp4, cfg=base, budget=128, active_of=lambda i: 4,
                           dense_every_step=False, reps=args.steps, flags=flags)
        add_row("64K", f"LoSA |A|=4, {label}", base, 128, 4, SWEEP_LAYERS, res, False)
    floors["page_meta"] = page_meta_times(hip, lay, kv[1], reps=args.steps)
    log(f"[sweep] page metadata {json.dumps(floors['page_meta'])}")
    del kv, lay
    torch.cuda.empty_cache()

    # 16K GQA layer and the ragged batch: LoSA, QUEST-style, dense
    for c, n_layers in ((W.gqa_16k(), 16), (W.ragged_batch(), 4)):
        lay = W.make_layer(c, n_steps=c.n_steps)
        kv = (lay, replicas(lay, n_layers))
        inp = dev_inputs(lay, c.dtype)
        cases = [(f"LoSA |A|={c.n_active}", c.n_active, False, 0),
                 (f"QUEST-style (all {c.block} tokens active)", c.block, False, 0),
                 ("dense every step", c.n_active, True, 0)]
        if c.group * c.block <= 64:  # row masks take at most 64 stacked rows per KV head
            cases.append((f"naive per-query (all {c.block} tokens active, own pages)", c.block,
                          False, 1))
        for label, a, dense_mode, fl in cases:
            res = measure_case(hip, kv, lambda i: inp, cfg=c, budget=c.budget,
                               active_of=lambda i: a, dense_every_step=dense_mode, reps=args.steps,
                               flags=fl)
            add_row(c.name, label, c, c.budget, a, n_layers, res, dense_mode)
        if c.n_seq > 1:
            # the same batch read through a page table from a shuffled pool
            kp, vp, pt = W.paged_pool(lay, seed=5)
            kvp = (lay, [(to_device(kp, c.dtype), to_device(vp, c.dtype))] +
                   [(to_device(kp, c.dtype), to_device(vp, c.dtype)) for _ in range(n_layers - 1)])
            for label, a, dense_mode in ((f"LoSA |A|={c.n_active}, paged pool", c.n_active, False),
                                         ("dense every step, paged pool", c.n_active, True)):
                res = measure_case(hip, kvp, lambda i: inp, cfg=c, budget=c.budget,
                                   active_of=lambda i: a, dense_every_step=dense_mode,
                                   reps=args.steps, page_table=pt)
                add_row(c.name, label, c, c.budget, a, n_layers, res, dense_mode)
            del kvp
        del kv, lay, inp
        torch.cuda.empty_cache()

    # the 36-layer 128K trace: |A| = 2 in the first and last four layers, 6 between;
    # one block of every layer per replay (the whole model's attention per block)
    c0, c4 = W.trace_128k(0), W.trace_128k(4)
    lay = W.make_layer(c0, n_steps=c0.n_steps)
    lay6 = W.make_layer(c4, n_steps=c4.n_steps, cache=False)
    inp2, inp6 = dev_inputs(lay, c0.dtype), dev_inputs(lay6, c4.dtype)
    n_tr = 36
    kv = (lay, replicas(lay, n_tr))
    act = W.trace_layer_active
    res = measure_case(hip, kv, lambda i: inp2 if act(i) == 2 else inp6, cfg=c0, budget=c0.budget,
                       active_of=act, dense_every_step=False, reps=max(2, args.steps // 4),
                       union_layers=(0, 4))
    u = res["union_by_layer"]
    n2 = sum(1 for i in range(n_tr) if act(i) == 2)
    res["union_pages"] = (n2 * u[0] + (n_tr - n2) * u[4]) / n_tr
    add_row("trace 128K x 36", "LoSA, per-layer |A| (2/6)", c0, c0.budget,
            (n2 * 2 + (n_tr - n2) * 6) / n_tr, n_tr, res, False)
    rows[-1]["note"] = ("union statistics: layer-weighted mean of layer 0 (|A| = 2) and layer 4 "
                        "(|A| = 6); n_active = the layer mean")
    rows[-1]["union_pages_per_kv_head_by_active"] = {
        "2": u[0] / (c0.n_seq * c0.n_kvhead), "6": u[4] / (c0.n_seq * c0.n_kvhead)}
    rows[-1]["model_step_us"] = res["step_us"] * n_tr
    rows[-1]["model_dense_step_us"] = res["dense_us"] * n_tr
    del kv, lay, lay6
    torch.cuda.empty_cache()
    hip.close()

    rec = {"sweep": "LoSA step sweep on one MI355X", "floors": floors, "rows": rows,
           "wall_s": time.perf_counter() - t_start}
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            json.dump(rec, f, indent=1)
    print(json.dumps({"sweep_rows": len(rows), "out": args.sweep_out,
                      "wall_s": rec["wall_s"]}), flush=True)



def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed blocks")
    ap.add_argument("--warmup", type=int, default=2, help="untimed blocks")
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--budget", type=int, default=128)
    ap.add_argument("--active", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true",
                    help="time without the per-kernel stage events")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of the captured block")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="launch one plain copy kernel of MIB MiB before timing (reference "
                         "dispatch for profiler byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: the |A| x budget sweep, the density study, "
                         "other workload shapes, the 36-layer trace and latency floors")
    ap.add_argument("--sweep-out", default=None, help="JSON file for --sweep results")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the LoSA step is measured on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return sweep(args)

    import numpy as np
    import torch

    from sparse_attention_block_amd import binding as L
    from sparse_attention_block_amd import workloads as W
    from sparse_attention_block_amd.hiprt import HipRuntime
    from sparse_attention_block_amd.layer import LayerState, to_device

    L.load()
    torch.cuda.set_device(0)
    cfg = W.long_64k(args.budget, args.active)
    log(f"[bench] generating {cfg.name}")
    lay = W.make_layer(cfg, n_steps=STEPS_PER_BLOCK)
    dev = lambda x: to_device(x, cfg.dtype)
    base = LayerState.from_layer(lay)
    layers = [base]
    for _ in range(args.layers - 1):
        layers.append(LayerState(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead,
                                 n_kvhead=cfg.n_kvhead, head_dim=cfg.head_dim,
                                 budget_tokens=cfg.budget, n_active=cfg.n_active, dtype=cfg.dtype,
                                 k_cache=base.k_cache.clone(), v_cache=base.v_cache.clone(),
                                 kv_off=lay.kv_off, prefix_len=lay.prefix_len))
    for ls in layers:
        ls.build_page_meta()
    q = [dev(x) for x in lay.q]
    kb = [dev(x) for x in lay.k_blk]
    vb = [dev(x) for x in lay.v_blk]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipRuntime()

    # union sizes of every LoSA step (identical across the replicated layers)
    union_cnt = []
    dbg = L.Debug.alloc(base.shape)
    base.dense_first_step(q[0], kb[0], vb[0])
    for t in range(1, STEPS_PER_BLOCK):
        base.step(q[t], q[t - 1], kb[t], vb[t], debug=dbg)
        torch.cuda.synchronize()
        union_cnt.append(dbg.union_cnt.cpu().numpy().copy())
    union_pages = np.array([u.sum() for u in union_cnt], dtype=np.float64)  # per step, all KV heads

    # one prepared call per (step, layer): checks and marshalling happen here,
    # once; the same calls bound to a side stream are captured into graphs
    gstream = torch.cuda.Stream()
    calls, gcalls = {}, {}
    for t in range(STEPS_PER_BLOCK):
        for li, ls in enumerate(layers):
            for table, st in ((calls, None), (gcalls, gstream.cuda_stream)):
                table[(t, li)] = (ls.prepare_dense_first_step(q[0], kb[0], vb[0], stream=st) if t == 0
                                  else ls.prepare_step(q[t], q[t - 1], kb[t], vb[t], stream=st))

    def run_steps(steps, events=None, table=calls):
        """Steps `steps` of the block for every layer, in model order (step-major,
        layer-minor); events[(t, l)] = stage events or None."""
        for t in steps:
            for li in range(len(layers)):
                c = table[(t, li)]
                c.set_events(events[(t, li)] if events is not None else None)
                c()

    dense_steps, sparse_steps = [0], list(range(1, STEPS_PER_BLOCK))

    def run_block(events=None):
        run_steps(dense_steps + sparse_steps, events)

    def new_events():
        return {(t, li): [hip.event() for _ in range(L.LOSA_STAGE_EVENTS)]
                for t in range(STEPS_PER_BLOCK) for li in range(len(layers))}

    def block_outputs():
        return [torch.cat([ls.out.flatten().view(torch.int16), ls.op_cache.flatten().view(torch.int16),
                           ls.lp_cache.flatten().view(torch.int16)]).clone() for ls in layers]

    if args.copy_calibration:
        from sparse_attention_block_amd.build import SELFTEST_LIB
        st = ctypes.CDLL(SELFTEST_LIB)
        st.losa_selftest_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_int, ctypes.c_void_p]
        nb = args.copy_calibration << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        assert st.losa_selftest_copy(src.data_ptr(), dst.data_ptr(), nb, 4096, stream) == 0
        torch.cuda.synchronize()
        assert bool(torch.equal(src, dst))
        del src, dst
        log(f"[bench] copy calibration: {args.copy_calibration} MiB read + written once")
    log(f"[bench] warmup {args.warmup} blocks x {len(layers)} layers")
    for _ in range(args.warmup):
        run_block()
    torch.cuda.synchronize()
    eager_ref = block_outputs()

    # the block captured into two HIP graphs, its dense first steps and its LoSA
    # steps (the same launches, replayed without host launch overhead); every
    # check replay must reproduce the eager block bit for bit, with eager work
    # and synchronisations between
    graphs = None
    if not args.no_graph:
        torch.cuda.synchronize()
        g_dense = hip.capture(gstream.cuda_stream, lambda: run_steps(dense_steps, table=gcalls))
        g_sparse = hip.capture(gstream.cuda_stream, lambda: run_steps(sparse_steps, table=gcalls))
        graphs = (g_dense, g_sparse)
        for rep_i in range(3):
            hip.launch(g_dense, gstream.cuda_stream)
            hip.launch(g_sparse, gstream.cuda_stream)
            torch.cuda.synchronize()
            got = block_outputs()
            for a, b in zip(got, eager_ref):
                if not torch.equal(a, b):
                    raise SystemExit("graph replay differs from the eager block")
            run_block()  # eager work between replays
            torch.cuda.synchronize()
        log("[bench] graph replays match the eager block")

    # value: exactly K blocks with nothing but the library's launches in the
    # timed region, plus one event before, between and after the block's two
    # graphs (the dense first steps, then the LoSA steps), which splits the
    # block time into the two kinds of step
    def timed(use_graph):
        st = gstream.cuda_stream if use_graph else stream
        evs = [[hip.event() for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for k in range(args.steps):
            hip.record(evs[k][0], st)
            if use_graph:
                hip.launch(graphs[0], st)
            else:
                run_steps(dense_steps)
            hip.record(evs[k][1], st)
            if use_graph:
                hip.launch(graphs[1], st)
            else:
                run_steps(sparse_steps)
            hip.record(evs[k][2], st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        total = hip.ms(evs[0][0], evs[-1][2])
        dense = sum(hip.ms(e[0], e[1]) for e in evs)
        sparse = sum(hip.ms(e[1], e[2]) for e in evs)
        return total, dense, sparse, wall

    log(f"[bench] timing {args.steps} blocks ({'graph replay' if graphs else 'eager launches'})")
    total_ms, dense_ms, sparse_ms, wall = timed(graphs is not None)
    eager_ms = timed(False)[0] if graphs is not None else total_ms

    # per-kernel durations: a second timed pass of K blocks with the library's
    # stage events recorded between its launches
    use_events = not args.no_events
    ev_blocks = [new_events() for _ in range(args.steps)] if use_events else None
    if use_events:
        log(f"[bench] timing {args.steps} blocks with per-kernel events")
        torch.cuda.synchronize()
        for k in range(args.steps):
            run_block(ev_blocks[k])
        torch.cuda.synchronize()

    # launch and streaming floors, outside the timed region (their kernels also
    # appear in the rocprofv3 summary of this command)
    log("[bench] latency floors")
    floors = latency_floors(hip, stream)

    n_calls = args.steps * STEPS_PER_BLOCK * len(layers)
    value_us = total_ms * 1e3 / n_calls
    ms_per_step = total_ms / args.steps
    eager_us = eager_ms * 1e3 / n_calls
    dense_step_us = dense_ms * 1e3 / (args.steps * len(layers))
    sparse_step_us = sparse_ms * 1e3 / (args.steps * (STEPS_PER_BLOCK - 1) * len(layers))

    # per-kernel durations from the library's stage events (one kernel per stage)
    names = ["prepare", "score", "select", "prefix", "finish"]
    stages = {"dense": {n: [] for n in names}, "sparse": {n: [] for n in names}}
    if use_events:
        for evs in ev_blocks:
            for (t, li), e in evs.items():
                kind = "dense" if t == 0 else "sparse"
                for i, n in enumerate(names):
                    stages[kind][n].append(hip.ms(e[i], e[i + 1]) * 1e3)
    mean = lambda xs: float(np.mean(xs)) if xs else None

    # algorithmic bytes (bf16 storage)
    sT = 2
    Hk, d, P, L_ = cfg.n_kvhead, cfg.head_dim, cfg.page_size, cfg.prefix_lens[0]
    n_pages = (L_ + P - 1) // P
    kv_page_bytes = P * d * 2 * sT
    union_bytes = float(union_pages.mean()) * kv_page_bytes
    meta_bytes = Hk * n_pages * 2 * d * sT
    dense_kv_bytes = Hk * L_ * 2 * d * sT
    S, B, Hq = cfg.n_seq, cfg.block, cfg.n_qhead
    small_bytes = (2 * S * B * Hq * d * sT + 2 * S * B * Hk * d * sT + S * Hq * B * (d + 1) * 4
                   + S * Hq * cfg.n_active * (d + 1) * 4 + S * B * Hq * d * sT)
    sparse_step_bytes = meta_bytes + union_bytes + small_bytes
    dense_step_bytes = dense_kv_bytes + 2 * S * B * Hq * d * sT + 2 * S * B * Hk * d * sT \
        + S * Hq * B * (d + 1) * 4
    block_bytes = dense_step_bytes + (STEPS_PER_BLOCK - 1) * sparse_step_bytes
    hbm_gbps = block_bytes / (value_us * STEPS_PER_BLOCK * 1e-6) / 1e9

    # kernels of this shape (bf16: the preparation is folded into scoring, and
    # the dense pass reads the block queries itself, so neither has a stage of
    # its own), with their algorithmic HBM bytes per launch and launches per
    # layer-block; durations from the committed rocprofv3 summary of this
    # workload where it describes the current sources, else from the events
    # (which add the latency of an event record, about 1 us, to every kernel)
    # (the summaries are named for the workload: long_64k_b<budget>_a<|A|>)
    rp, rp_path = rocprof_durations(f"long_64k_b{cfg.budget}_a{cfg.n_active}")
    spec = {
        "page_score": (stages["sparse"]["score"], meta_bytes, STEPS_PER_BLOCK - 1),
        "page_select": (stages["sparse"]["select"], 0, STEPS_PER_BLOCK - 1),
        "sparse_prefix": (stages["sparse"]["prefix"], union_bytes, STEPS_PER_BLOCK - 1),
        "sparse_finish": (stages["sparse"]["finish"], 0, STEPS_PER_BLOCK - 1),
        "dense_prefix": (stages["dense"]["prefix"], dense_kv_bytes, 1),
        "dense_finish": (stages["dense"]["finish"], 0, 1),
    }
    kernels = {}
    for name, (xs, nbytes, per_block) in spec.items():
        ev_us = mean(xs) if use_events else None
        us = rp.get(name, ev_us)
        if us is None:
            continue
        kernels[name] = {"avg_us": us, "avg_us_events": ev_us,
                         "duration_source": "rocprofv3" if name in rp else "hip events",
                         "launches_per_layer_block": per_block, "us_per_layer_block": us * per_block}
        if nbytes:
            gbps = nbytes / (us * 1e-6) / 1e9
            kernels[name].update({"bytes_per_launch": nbytes, "achieved_gbps": gbps,
                                  "frac_of_peak": gbps / PEAK_HBM_GBPS})
    dominant = max((k for k in kernels if "bytes_per_launch" in kernels[k]),
                   key=lambda k: kernels[k]["us_per_layer_block"], default=None)

    def read_floor(nbytes):
        """The pure-read probe of the nearest size at or above nbytes (rocprofv3
        duration where the committed summary matches, else its events)."""
        for mib, _ in FLOOR_READS:
            if (mib << 20) >= nbytes:
                us = rp.get(f"probe_read_{mib}MiB")
                src = "rocprofv3" if us is not None else "hip events"
                if us is None:
                    us = floors["read"][f"{mib}MiB"]["us_events"]
                return {"probe": f"pure read of {mib} MiB (cold)", "us": us, "duration_source": src,
                        "kernel_over_probe": None}
        return None

    def gather_floor():
        """The gather probe with the sparse prefix pass's memory pattern and no
        arithmetic (rocprofv3 duration where the committed summary matches)."""
        g = floors.get("gather")
        if not g:
            return None
        us = rp.get("probe_gather")
        src = "rocprofv3" if us is not None else "hip events"
        if us is None:
            us = g["us_events"]
        return {"probe": f"page lists then {g['pages']} cold pages of 8 KiB, 4 per workgroup "
                         f"({g['workgroups']} workgroups), then partial-sized stores",
                "us": us, "duration_source": src, "kernel_over_probe": None}

    def roofline(name):
        if name is None or "bytes_per_launch" not in kernels.get(name, {}):
            return None
        k = kernels[name]
        fl = read_floor(k["bytes_per_launch"])
        if fl is not None:
            fl["kernel_over_probe"] = k["avg_us"] / fl["us"]
        pf = gather_floor() if name == "sparse_prefix" else None
        if pf is not None:
            pf["kernel_over_probe"] = k["avg_us"] / pf["us"]
        return {"kernel": name, "bound": "hbm", "achieved": k["achieved_gbps"],
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": k["frac_of_peak"],
                "traffic": traffic_from_profile(name),
                "bytes_per_launch": k["bytes_per_launch"], "avg_launch_us": k["avg_us"],
                "avg_launch_us_events": k["avg_us_events"],
                "duration_source": (f"rocprofv3 kernel trace, {rp_path}" if name in rp
                                    else "hip events around the kernel"),
                "read_floor": fl, **({"pattern_floor": pf} if pf is not None else {})}

    rec = {
        "metric": METRIC,
        "value": value_us,
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "prefix_len": L_, "block": B, "n_qhead": Hq,
                   "n_kvhead": Hk, "head_dim": d, "page_size": P, "budget_tokens": cfg.budget,
                   "n_active": cfg.n_active, "steps_per_block": STEPS_PER_BLOCK,
                   "layers": len(layers), "step": "one block of 8 denoising steps "
                   "(1 dense + 7 LoSA) for every layer"},
        "hbm_gbps": hbm_gbps,
        "sparse_step_us": sparse_step_us,
        "dense_step_us": dense_step_us,
        "speedup_vs_dense": dense_step_us / sparse_step_us,
        "union_pages_per_kv_head": float(union_pages.mean()) / (cfg.n_seq * Hk),
        "density": float(union_pages.mean()) / (cfg.n_seq * Hk * n_pages),
        "roofline": roofline(dominant),
        "roofline_sparse_prefix": roofline("sparse_prefix"),
        "kernels": kernels,
        "launch": ("hip graph replays of the captured block (dense first steps, then LoSA "
                   "steps)" if graphs else "eager launches"),
        "value_eager_launch": eager_us,
        "wall_s": wall,
        "floors": floors_record(floors, rp),
    }
    hip.close()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on one layer-block")
        rec["cpu_baseline"] = cpu_baseline(cfg, lay)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
