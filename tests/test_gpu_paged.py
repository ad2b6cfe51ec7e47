"""A paged KV pool on the GPU: every sequence's prefix pages scattered over a
pool of physical pages in a seeded random order (workloads.paged_pool), read
through a page table, against the oracle on the same prefix laid out
contiguously.  The pages' content is what the method reads, so indices
(locality, active sets, page lists, unions: all in the sequence's own page
numbers) must match bit for bit and values within the checks' bounds.  Also:
the metadata of the pool's pages against the oracle's per-page minima and
maxima, the block-commit update through a page table, and sequences that share
physical pages."""
import numpy as np
import pytest
import torch

from gpu_support import Pair, say, stratified_rows
from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.layer import LayerState, to_device
from test_gpu_page_meta import decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


CASES = [
    ("paged_bf16_ragged", dict(dtype="bf16", head_dim=128, block=16, n_active=4, budget=64,
                               prefix_lens=(1000, 48, 16, 0), n_kvhead=2, n_qhead=8,
                               needles=True), 0),
    ("paged_f32_d64", dict(dtype="f32", head_dim=64, block=16, n_active=4, budget=64,
                           prefix_lens=(1024, 300), n_kvhead=1, n_qhead=4), 0),
    ("paged_bf16_shared", dict(dtype="bf16", head_dim=128, block=16, n_active=3, budget=48,
                               prefix_lens=(2000, 1500, 700), n_kvhead=2, n_qhead=4,
                               needles=True), 40),
    ("paged_bf16_d64_B32_full_budget", dict(dtype="bf16", head_dim=64, block=32, n_active=8,
                                            budget=1024, prefix_lens=(900, 333), n_kvhead=2,
                                            n_qhead=8), 0),
]


@pytest.mark.parametrize("name,kw,share", CASES, ids=[c[0] for c in CASES])
def test_paged_steps(name, kw, share):
    cid = 520 + [c[0] for c in CASES].index(name)
    cfg = W.small_case(cid, n_steps=3, **kw)
    lay = W.make_layer(cfg)
    pool = W.paged_pool(lay, seed=1, share_pages=share)
    p = Pair(lay, name, paged=pool)
    p.dense(0)
    for step in (1, 2):
        p.sparse(step)


def test_paged_ragged_batch():
    """The ragged batch (8 sequences, 8K-64K prefixes, B = 32, budget 256) from a
    shuffled pool: dense rows stratified over every (sequence, KV head), then
    LoSA steps."""
    cfg = W.ragged_batch()
    lay = W.make_layer(cfg, n_steps=3)
    pool = W.paged_pool(lay, seed=2)
    p = Pair(lay, "paged_ragged_batch", paged=pool)
    p.dense(0, rows=stratified_rows(cfg, 4, seed=99))
    op, lp = W.make_cache_state(cfg)
    p.set_cache(op, lp)
    for step in (1, 2):
        p.sparse(step)


def test_paged_page_meta_matches_oracle():
    cfg = W.small_case(530, dtype="bf16", head_dim=128, prefix_lens=(1000, 48, 16, 0, 4097),
                       n_kvhead=2, n_qhead=8, budget=64, n_active=4, n_steps=1, needles=True)
    lay = W.make_layer(cfg)
    k_pool, v_pool, pt = W.paged_pool(lay, seed=3)
    say(f"[paged page_meta] pool of {k_pool.shape[1] // 16} pages")
    ls = LayerState(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead, n_kvhead=cfg.n_kvhead,
                    head_dim=cfg.head_dim, budget_tokens=cfg.budget, n_active=cfg.n_active,
                    dtype=cfg.dtype, k_cache=to_device(k_pool, cfg.dtype),
                    v_cache=to_device(v_pool, cfg.dtype), kv_off=lay.kv_off,
                    prefix_len=lay.prefix_len, page_table=pt)
    ls.build_page_meta()
    torch.cuda.synchronize()
    maxp_len = int(ls.shape.max_prefix_len)
    kmin, kmax, amax = decode(ls.page_meta.cpu().numpy(), cfg, k_pool.shape[1], maxp_len)
    orc = Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
    omin, omax = orc.page_meta()
    P = cfg.page_size
    max_pages = (maxp_len + P - 1) // P
    for s in range(cfg.n_seq):
        n = (int(lay.prefix_len[s]) + P - 1) // P
        gp0 = int(lay.kv_off[s]) // P
        mp = slice(s * max_pages, s * max_pages + n)  # the sequence's metadata pages
        assert np.array_equal(kmin[:, mp].view(np.uint32), omin[:, gp0:gp0 + n].view(np.uint32)), s
        assert np.array_equal(kmax[:, mp].view(np.uint32), omax[:, gp0:gp0 + n].view(np.uint32)), s
        want = np.maximum(np.abs(omin[:, gp0:gp0 + n]), np.abs(omax[:, gp0:gp0 + n])).max(axis=2)
        assert np.array_equal(amax[:, mp], want), s


def test_paged_update_after_commit():
    """Block commit through a page table: metadata built at the old lengths,
    then updated for the committed tokens, equals a full build at the new
    lengths, byte for byte."""
    old, added = (1000, 48, 16, 0, 777), (16, 16, 16, 16, 0)
    new = tuple(o + a for o, a in zip(old, added))
    cfg = W.small_case(531, n_seq=len(old), dtype="bf16", head_dim=128, prefix_lens=new,
                       n_kvhead=2, n_qhead=4, budget=64, n_active=4, n_steps=1)
    lay = W.make_layer(cfg)
    k_pool, v_pool, pt = W.paged_pool(lay, seed=4)
    kd, vd = to_device(k_pool, cfg.dtype), to_device(v_pool, cfg.dtype)
    mk = lambda lens: LayerState(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead,
                                 n_kvhead=cfg.n_kvhead, head_dim=128, budget_tokens=cfg.budget,
                                 n_active=cfg.n_active, dtype=cfg.dtype, k_cache=kd, v_cache=vd,
                                 kv_off=lay.kv_off, prefix_len=np.asarray(lens, np.int32),
                                 max_prefix_len=max(new), page_table=pt)
    full, step = mk(new), mk(old)
    full.build_page_meta()
    step.build_page_meta()
    step.prefix_len.copy_(torch.as_tensor(np.asarray(new, np.int32)))
    step.update_page_meta(np.asarray(old, np.int32), max(added))
    torch.cuda.synchronize()
    assert torch.equal(step.page_meta, full.page_meta)
