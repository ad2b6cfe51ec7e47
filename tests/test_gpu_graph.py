"""Stream capture of LoSA steps into a HIP graph: every replay of a captured
dense first step followed by LoSA steps reproduces the eager launches bit for
bit, with eager work and synchronisations between the replays.  The library
records no memset and allocates nothing, so its launches capture as plain
kernel nodes."""
import pytest
import torch

from gpu_support import say
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
