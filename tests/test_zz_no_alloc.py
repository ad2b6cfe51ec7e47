"""losa_step_noalloc (the library's static per-GPU scratch, no workspace
argument) against losa_step (caller's workspace) on the same inputs: the same
kernels, so every output, cache entry and debug index must be identical bit
for bit.  Two calls in a row, the second with a smaller shape, so the second
runs on scratch the first left behind."""
import pytest
import torch

from gpu_support import say
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.layer import LayerState, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _run_pair(cfg, tag):
    say(f"[noalloc] {tag}: S={cfg.n_seq} L={list(cfg.prefix_lens)} Hq={cfg.n_qhead} "
        f"Hkv={cfg.n_kvhead} A={cfg.n_active} budget={cfg.budget}")
    lay = W.make_layer(cfg, n_steps=2)
    ls = LayerState.from_layer(lay)
    ls.build_page_meta()
    dev = lambda x: to_device(x, cfg.dtype)
    q0, q1 = dev(lay.q[0]), dev(lay.q[1])
    kb0, kb1, vb0, vb1 = dev(lay.k_blk[0]), dev(lay.k_blk[1]), dev(lay.v_blk[0]), dev(lay.v_blk[1])
    ls.dense_first_step(q0, kb0, vb0)
    op0, lp0 = ls.op_cache.clone(), ls.lp_cache.clone()
    # losa_step with the caller's workspace
    dbg_a = L.Debug.alloc(ls.shape)
    out_a = torch.empty_like(ls.out)
    ls.step(q1, q0, kb1, vb1, debug=dbg_a, out=out_a)
    op_a, lp_a = ls.op_cache.clone(), ls.lp_cache.clone()
    # losa_step_noalloc on the same starting cache
    ls.op_cache.copy_(op0)
    ls.lp_cache.copy_(lp0)
    dbg_b = L.Debug.alloc(ls.shape)
    out_b = torch.full_like(ls.out, float("nan"))
    L.losa_step_noalloc(ls.shape, q1, q0, kb1, vb1, ls.k_cache, ls.v_cache, ls.page_meta,
                        ls.kv_off, ls.prefix_len, ls.op_cache, ls.lp_cache, out_b, dbg_b)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert same(out_a, out_b), f"{tag}: out differs"
    assert same(op_a, ls.op_cache) and same(lp_a, ls.lp_cache), f"{tag}: cache differs"
    for f in ("locality", "active", "page_sel", "union_idx", "union_cnt"):
        assert same(getattr(dbg_a, f), getattr(dbg_b, f)), f"{tag}: debug {f} differs"
    say(f"[noalloc] {tag}: identical (union pages {dbg_b.union_cnt.sum().item()})")


def test_noalloc_matches_workspace_call_twice_shrinking():
    big = W.long_64k(128, 4)
    small = W.small_case(610, dtype="bf16", head_dim=128, block=16, n_qhead=8, n_kvhead=2,
                         n_active=3, budget=64, prefix_lens=(1500, 300), n_steps=2, needles=True)
    _run_pair(big, "first call, 64K layer")
    _run_pair(small, "second call, smaller shape")
