"""Page metadata on the GPU: bit for bit against the oracle's per-page minima and
maxima, and the block-commit update (losa_update_page_meta) against a full
rebuild at the new prefix lengths.  The library's documented metadata layout
(page_meta.hip: per KV head, tiles of 64 pages; chunk c of every page of a tile
back to back, 16 bytes per page; then the largest |key| of every page; then
the page-major copy, each page's chunks back to back) is decoded on the host."""
import numpy as np
import pytest
import torch

from gpu_support import say
from oracle import Oracle
from sparse_attention_block_amd import binding as L
from sparse_attention_block_amd import workloads as W
from sparse_attention_block_amd.layer import LayerState

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def decode(meta: np.ndarray, cfg, kv_tokens: int, max_prefix_len: int):
    """(kmin, kmax) [Hk][M][d] and the largest |key| [Hk][M] of every metadata
    page, M = max(T/16, n_seq * max_pages): a sequence's page p is metadata page
    kv_off/16 + p (contiguous layout) or s * max_pages + p (page table)."""
    Hk, d = cfg.n_kvhead, cfg.head_dim
    max_pages = (max_prefix_len + cfg.page_size - 1) // cfg.page_size
    TP = max(kv_tokens // cfg.page_size, cfg.n_seq * max_pages)
    n_tiles = (TP + 63) // 64
    bf = cfg.dtype == "bf16"
    nch = d // (4 if bf else 2)
    main = Hk * n_tiles * 64 * d * 2 * (2 if bf else 4)
    u = meta[:main].view(np.uint32).reshape(Hk, n_tiles, nch, 64, 4)
    u = u.transpose(0, 1, 3, 2, 4).reshape(Hk, n_tiles * 64, nch, 4)[:, :TP]
    pm_off = main + Hk * n_tiles * 64 * 4
    pm = meta[pm_off:pm_off + main].view(np.uint32).reshape(Hk, n_tiles * 64, nch, 4)[:, :TP]
    assert np.array_equal(pm, u), "page-major copy differs from the chunk-major metadata"
    if bf:  # one word per dimension: max in the low half, min in the high half
        kmax = (u << 16).view(np.float32).reshape(Hk, TP, d)
        kmin = (u & 0xFFFF0000).view(np.float32).reshape(Hk, TP, d)
    else:  # (max_0, min_0, max_1, min_1) per chunk of two dimensions
        kmax = np.ascontiguousarray(u[..., [0, 2]]).view(np.float32).reshape(Hk, TP, d)
        kmin = np.ascontiguousarray(u[..., [1, 3]]).view(np.float32).reshape(Hk, TP, d)
    amax = meta[main:main + Hk * n_tiles * 64 * 4].view(np.float32).reshape(Hk, n_tiles * 64)[:, :TP]
    return kmin, kmax, amax


def seq_pages(lay):
    P = lay.cfg.page_size
    return [(int(o) // P, (int(n) + P - 1) // P) for o, n in zip(lay.kv_off, lay.prefix_len)]


CASES = [
    ("f32_d64", dict(dtype="f32", head_dim=64, prefix_lens=(1024,), n_kvhead=1, n_qhead=4)),
    ("bf16_d128_ragged", dict(dtype="bf16", head_dim=128, prefix_lens=(1000, 48, 16, 0, 4097),
                              n_kvhead=2, n_qhead=8)),
    ("bf16_d64", dict(dtype="bf16", head_dim=64, prefix_lens=(2000, 333), n_kvhead=2, n_qhead=8)),
    ("f32_d128", dict(dtype="f32", head_dim=128, prefix_lens=(1500, 48), n_kvhead=2, n_qhead=8)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_page_meta_matches_oracle(name, kw):
    say(f"[page_meta] {name}")
    cfg = W.small_case(320 + [c[0] for c in CASES].index(name), budget=64, n_active=4,
                       n_steps=1, needles=True, **kw)
    lay = W.make_layer(cfg)
    ls = LayerState.from_layer(lay)
    ls.build_page_meta()
    torch.cuda.synchronize()
    kmin, kmax, amax = decode(ls.page_meta.cpu().numpy(), cfg, lay.kv_tokens,
                              int(ls.shape.max_prefix_len))
    orc = Oracle(cfg, lay.kv_off, lay.prefix_len, lay.kv_tokens, lay.k_cache, lay.v_cache)
    omin, omax = orc.page_meta()
    for s, (gp0, n) in enumerate(seq_pages(lay)):
        sl = slice(gp0, gp0 + n)
        assert np.array_equal(kmin[:, sl].view(np.uint32), omin[:, sl].view(np.uint32)), f"min, seq {s}"
        assert np.array_equal(kmax[:, sl].view(np.uint32), omax[:, sl].view(np.uint32)), f"max, seq {s}"
        want = np.maximum(np.abs(omin[:, sl]), np.abs(omax[:, sl])).max(axis=2)
        assert np.array_equal(amax[:, sl], want), f"largest |key|, seq {s}"


@pytest.mark.parametrize("dtype,d,old,added", [
    ("bf16", 128, (1000, 48, 16, 0, 777), (16, 16, 16, 16, 0)),
    ("bf16", 64, (2000, 333), (32, 32)),
    ("f32", 128, (1500, 48), (16, 5)),
    ("bf16", 128, (65536 - 16,), (16,)),
])
def test_update_after_commit(dtype, d, old, added):
    """Metadata built at the old lengths, then updated for the committed tokens,
    equals a full build at the new lengths, byte for byte."""
    new = tuple(o + a for o, a in zip(old, added))
    say(f"[page_meta commit] {dtype} d={d} old={old} new={new}")
    cfg = W.small_case(340 + len(old) + d, n_seq=len(old), dtype=dtype, head_dim=d,
                       prefix_lens=new, n_kvhead=2, n_qhead=4, budget=64, n_active=4, n_steps=1)
    lay = W.make_layer(cfg)
    full = LayerState.from_layer(lay)
    full.build_page_meta()
    step = LayerState(n_seq=cfg.n_seq, block=cfg.block, n_qhead=cfg.n_qhead, n_kvhead=cfg.n_kvhead,
                      head_dim=d, budget_tokens=cfg.budget, n_active=cfg.n_active, dtype=dtype,
                      k_cache=full.k_cache, v_cache=full.v_cache, kv_off=lay.kv_off,
                      prefix_len=np.asarray(old, np.int32), max_prefix_len=max(new))
    step.build_page_meta()
    step.prefix_len.copy_(torch.as_tensor(np.asarray(new, np.int32)))
    step.update_page_meta(np.asarray(old, np.int32), max(added))
    torch.cuda.synchronize()
    assert torch.equal(step.page_meta, full.page_meta)
