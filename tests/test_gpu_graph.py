"""Stream capture of LoSA steps into a HIP graph: every replay of a captured
dense first step followed by LoSA steps reproduces the eager launches bit for
bit, with eager work and synchronisations between the replays.  The library
records no memset and allocates nothing, so its launches capture as plain
kernel nodes."""
import numpy as np
import pytest
import torch

from gpu_support import assert_close, assert_lp, host, say
from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.hiprt import HipRuntime
from sparse_attention_block_amd.layer import LayerState, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("dtype,prefix", [("bf16", (4096, 2000)), ("f32", (1024,))])
def test_graph_replays_match_eager(dtype, prefix):
    say(f"[graph] {dtype} prefix {prefix}")
    cfg = W.small_case(60 + len(prefix), n_seq=len(prefix), dtype=dtype, prefix_lens=prefix,
                       n_qhead=8, n_kvhead=2, head_dim=128 if dtype == "bf16" else 64,
                       budget=128, n_active=4, n_steps=3, needles=True)
    lay = W.make_layer(cfg)
    ls = LayerState.from_layer(lay)
    ls.build_page_meta()
    dev = lambda x: to_device(x, cfg.dtype)
    q = [dev(x) for x in lay.q]
    kb = [dev(x) for x in lay.k_blk]
    vb = [dev(x) for x in lay.v_blk]
    side = torch.cuda.Stream()

    def calls(stream):
        out = [ls.prepare_dense_first_step(q[0], kb[0], vb[0], stream=stream)]
        for t in range(1, cfg.n_steps):
            out.append(ls.prepare_step(q[t], q[t - 1], kb[t], vb[t], stream=stream))
        return out

    eager, captured = calls(None), calls(side.cuda_stream)

    def run(cs):
        for c in cs:
            c()

    def snapshot():
        return [t.clone() for t in (ls.out, ls.op_cache, ls.lp_cache)]

    run(eager)
    torch.cuda.synchronize()
    ref = snapshot()
    hip = HipRuntime()
    try:
        torch.cuda.synchronize()
        g = hip.capture(side.cuda_stream, lambda: run(captured))
        for rep in range(3):
            ls.out.fill_(0)
            ls.op_cache.fill_(0)
            ls.lp_cache.fill_(0)
            torch.cuda.synchronize()
            hip.launch(g, side.cuda_stream)
            torch.cuda.synchronize()
            for got, want in zip(snapshot(), ref):
                assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), f"replay {rep}"
            run(eager)  # eager work between replays
            torch.cuda.synchronize()
    finally:
        hip.close()


def test_layer_stack_graph_matches_oracle():
    """A block of four layers with the trace's per-layer |A| (2 in the outer
    layers, 6 in the inner ones), captured step-major as one graph: every
    replay's output of every (layer, step), and each layer's final (o_p, L_p)
    cache, against the oracle run layer by layer."""
    n_layers, n_steps = 4, 3
    act = [2, 6, 6, 2]
    base = W.small_case(80, dtype="bf16", head_dim=128, block=16, n_qhead=32, n_kvhead=8,
                        budget=128, n_active=2, prefix_lens=(6000,), n_steps=n_steps,
                        needles=True)
    cfgs = [base.replace(n_active=a, n_drift=a, cfg_id=80 + li) for li, a in enumerate(act)]
    lays = [W.make_layer(c, layer=li) for li, c in enumerate(cfgs)]
    # the oracle, layer by layer
    refs = []
    for c, lay in zip(cfgs, lays):
        orc = Oracle(c, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
        outs = [orc.dense_first_step(lay.q[0], lay.k_blk[0], lay.v_blk[0])]
        for t in range(1, n_steps):
            outs.append(orc.step(lay.q[t], lay.q[t - 1], lay.k_blk[t], lay.v_blk[t])["out"])
        refs.append((outs, orc.op.copy(), orc.lp.copy()))
    say(f"[layer stack] {n_layers} layers, |A| {act}, oracle done")
    states, calls = [], []
    side = torch.cuda.Stream()
    dev = lambda x: to_device(x, base.dtype)
    inputs = []
    for c, lay in zip(cfgs, lays):
        ls = LayerState.from_layer(lay)
        ls.build_page_meta()
        states.append(ls)
        inputs.append(([dev(x) for x in lay.q], [dev(x) for x in lay.k_blk],
                       [dev(x) for x in lay.v_blk]))
    outs = [[torch.empty_like(states[li].out) for _ in range(n_steps)] for li in range(n_layers)]
    for t in range(n_steps):  # step-major, layer-minor: the model's order
        for li, ls in enumerate(states):
            q, kb, vb = inputs[li]
            if t == 0:
                calls.append(ls.prepare_dense_first_step(q[0], kb[0], vb[0], out=outs[li][0],
                                                         stream=side.cuda_stream))
            else:
                calls.append(ls.prepare_step(q[t], q[t - 1], kb[t], vb[t], out=outs[li][t],
                                             stream=side.cuda_stream))
    torch.cuda.synchronize()
    hip = HipRuntime()
    try:
        g = hip.capture(side.cuda_stream, lambda: [c() for c in calls])
        for rep in range(3):
            for li in range(n_layers):
                for o in outs[li]:
                    o.fill_(0)
                states[li].op_cache.fill_(0)
                states[li].lp_cache.fill_(0)
            torch.cuda.synchronize()
            hip.launch(g, side.cuda_stream)
            torch.cuda.synchronize()
            for li in range(n_layers):
                ref_outs, ref_op, ref_lp = refs[li]
                for t in range(n_steps):
                    assert_close(host(outs[li][t]), ref_outs[t], base.dtype,
                                 f"replay {rep} layer {li} step {t} out")
                assert_close(host(states[li].op_cache), ref_op, base.dtype,
                             f"replay {rep} layer {li} o_p")
                assert_lp(host(states[li].lp_cache), ref_lp, base.dtype,
                          f"replay {rep} layer {li} L_p")
            # eager work between replays: one eager block of layer 0 on the default stream
            q, kb, vb = inputs[0]
            states[0].dense_first_step(q[0], kb[0], vb[0])
            torch.cuda.synchronize()
    finally:
        hip.close()
