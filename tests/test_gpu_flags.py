"""The reading variants (losa_shape.flags) on the GPU against the oracle: per-row
page masks inside the loaded union, one active set shared by all heads from the
head-summed locality, and sparse steps that leave the (o_p, L_p) cache as the
dense step wrote it.  Indices bit for bit, values within gpu_support.TOL."""
import numpy as np
import pytest
import torch

from gpu_support import Pair, host, say
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W

pytestmark = pytest.mark.gpu

ROW_MASK, SHARED_ACTIVE, NO_WRITEBACK = 1, 2, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


CASES = [
    ("row_mask_bf16_ragged", ROW_MASK, dict(dtype="bf16", head_dim=128, block=16, n_active=4,
                                             budget=64, prefix_lens=(1000, 48, 16, 0), n_kvhead=2,
                                             n_qhead=8, needles=True)),
    ("row_mask_bf16_G8", ROW_MASK, dict(dtype="bf16", head_dim=128, block=16, n_active=8,
                                         budget=128, prefix_lens=(5000,), n_kvhead=1, n_qhead=8)),
    ("row_mask_f32_d64", ROW_MASK, dict(dtype="f32", head_dim=64, block=16, n_active=4, budget=64,
                                         prefix_lens=(1024,), n_kvhead=1, n_qhead=4)),
    ("row_mask_full_budget", ROW_MASK, dict(dtype="bf16", head_dim=64, block=16, n_active=4,
                                             budget=1024, prefix_lens=(700,), n_kvhead=2,
                                             n_qhead=4)),
    ("shared_bf16", SHARED_ACTIVE, dict(dtype="bf16", head_dim=128, block=16, n_active=4,
                                        budget=64, prefix_lens=(2000, 333), n_kvhead=2,
                                        n_qhead=8)),
    ("shared_f32_B32", SHARED_ACTIVE, dict(dtype="f32", head_dim=64, block=32, n_active=8,
                                           budget=64, prefix_lens=(1500,), n_kvhead=2, n_qhead=8)),
    # bf16 shapes whose preparation does not fold into scoring: G * B rows too
    # many for its LDS, and query heads x block tokens past what it stages
    ("shared_bf16_G8_B32", SHARED_ACTIVE, dict(dtype="bf16", head_dim=128, block=32, n_active=8,
                                               budget=64, prefix_lens=(900, 1600), n_kvhead=1,
                                               n_qhead=8)),
    ("shared_bf16_96_heads", SHARED_ACTIVE, dict(dtype="bf16", head_dim=64, block=16, n_active=2,
                                                 budget=32, prefix_lens=(260,), n_kvhead=48,
                                                 n_qhead=96)),
    ("no_writeback_bf16", NO_WRITEBACK, dict(dtype="bf16", head_dim=128, block=16, n_active=4,
                                             budget=64, prefix_lens=(1000, 300), n_kvhead=2,
                                             n_qhead=8)),
    ("all_flags_bf16", ROW_MASK | SHARED_ACTIVE | NO_WRITEBACK,
     dict(dtype="bf16", head_dim=128, block=16, n_active=3, budget=48,
          prefix_lens=(1040, 17, 2064), n_kvhead=2, n_qhead=4, needles=True)),
]


@pytest.mark.parametrize("name,flags,kw", CASES, ids=[c[0] for c in CASES])
def test_flag_variant(name, flags, kw):
    cid = 400 + [c[0] for c in CASES].index(name)
    cfg = W.small_case(cid, n_steps=3, flags=flags, **kw)
    p = Pair(W.make_layer(cfg), name)
    p.dense(0)
    op0, lp0 = host(p.gpu.op_cache).copy(), host(p.gpu.lp_cache).copy()
    for step in (1, 2):
        r = p.sparse(step)
        if flags & NO_WRITEBACK:
            assert np.array_equal(host(p.gpu.op_cache), op0), f"{name}: o_p cache changed"
            assert np.array_equal(host(p.gpu.lp_cache), lp0), f"{name}: L_p cache changed"
        if flags & SHARED_ACTIVE:  # one set per sequence (compared bit for bit above)
            act = r["res"]["active"]
            assert (act == act[:, :1]).all(), f"{name}: heads disagree"


def test_row_mask_long_64k():
    """Row masks at the full long-context shape (64K prefix, 32/8 heads, |A| = 4)."""
    cfg = W.long_64k(128, 4).replace(flags=ROW_MASK, cfg_id=77, name="row_mask_64k")
    lay = W.make_layer(cfg, n_steps=3)
    p = Pair(lay, cfg.name)
    op, lp = W.make_cache_state(cfg)
    p.set_cache(op, lp)
    for step in (1, 2):
        p.sparse(step)


def test_shared_long_64k():
    """The shared active set at the full long-context shape (64K prefix, 32/8 heads)."""
    cfg = W.long_64k(128, 4).replace(flags=SHARED_ACTIVE, cfg_id=78, name="shared_64k")
    lay = W.make_layer(cfg, n_steps=3)
    p = Pair(lay, cfg.name)
    op, lp = W.make_cache_state(cfg)
    p.set_cache(op, lp)
    for step in (1, 2):
        act = p.sparse(step)["res"]["active"]
        assert (act == act[:, :1]).all(), "heads disagree"
