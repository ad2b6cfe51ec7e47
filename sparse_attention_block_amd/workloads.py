"""Seeded synthetic inputs for LoSA's per-denoising-step attention.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It holds none of the method's arithmetic: only random draws, the
rounding of those draws to the storage type, and the planted structure the
workloads call for (a few drifting tokens per step, needle pages whose keys
point at one query).

Workload recipes (shapes from the long-context setting the LoSA pages time:
64K-token prefix, block of 16 tokens, budgets of 128/256 tokens; the pages
measure on LongBench, which these synthetic draws stand in for):

* keys/values of the prefix cache and of the block ~ N(0, 1);
* first-step queries Q_1 ~ N(0, 1);
* step t >= 2: a fresh uniform set of ``n_active`` block tokens receives
  N(0, 0.5) drift, every other token N(0, 1e-3) (second argument = std); the
  same tokens drift in every head; the in-block K/V drift the same way;
* needles (8B-class shapes): per sequence and KV head, 8 distinct pages whose
  keys are turned towards the direction of one random first-step query of that
  KV head's group, at cosine 0.8 and with their norms kept;
* tie cases (edge cases of the method's orderings, not a workload of the
  pages): runs of pages that repeat one page's keys, and stable tokens with no
  drift at all (stable_sigma = 0), so that bounds and localities tie exactly.

Every array is float32 holding values exactly representable in the storage
type (bf16 draws are rounded once, round-to-nearest-even), so both sides read
the same bits.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# Stream identifiers for the counter-style seeding below.
_S_K, _S_V, _S_Q, _S_KB, _S_VB, _S_NEEDLE, _S_LENS = 0, 1, 2, 3, 4, 5, 6
_S_DRIFT_TOK, _S_DRIFT_Q, _S_DRIFT_KB, _S_DRIFT_VB = 10, 11, 12, 13


@dataclass(frozen=True)
class Config:
    """One workload: the shapes of a LoSA layer-step and the draw recipe."""

    name: str
    cfg_id: int
    n_seq: int
    block: int
    n_qhead: int
    n_kvhead: int
    head_dim: int
    page_size: int
    budget: int            # per-query budget, in tokens
    n_active: int          # |A|, active tokens per head per step
    dtype: str             # "f32" or "bf16"
    prefix_lens: tuple     # prefix length L of every sequence
    n_steps: int           # denoising steps per block (the first one is dense)
    needles: bool = False
    n_needles: int = 8
    needle_cos: float = 0.8
    active_sigma: float = 0.5
    stable_sigma: float = 1e-3
    n_drift: Optional[int] = None   # drifting tokens per step (default: n_active)
    flags: int = 0                  # reading variants (row mask, shared active set, no write-back)
    dup_pages: int = 1              # runs of this many pages share the keys of their first page

    @property
    def group(self) -> int:
        return self.n_qhead // self.n_kvhead

    @property
    def drift_count(self) -> int:
        return self.n_active if self.n_drift is None else self.n_drift

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); finite inputs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _rng(cfg_id: int, layer: int, stream: int, step: int = 0, extra: int = 0):
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, stream, step, extra]))


def _normal(rng, shape, sigma=1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


@dataclass
class Layer:
    """One layer's inputs for one block: the prefix cache and every step's block."""

    cfg: Config
    layer: int
    kv_off: np.ndarray          # int32 [n_seq], first cache token of each sequence
    prefix_len: np.ndarray      # int32 [n_seq]
    kv_tokens: int              # cache capacity T (tokens per KV head)
    k_cache: np.ndarray         # float32 [H_kv][T][d]
    v_cache: np.ndarray         # float32 [H_kv][T][d]
    q: List[np.ndarray] = field(default_factory=list)       # per step [n_seq][B][H_q][d]
    k_blk: List[np.ndarray] = field(default_factory=list)   # per step [n_seq][B][H_kv][d]
    v_blk: List[np.ndarray] = field(default_factory=list)
    drift_tokens: List[Optional[np.ndarray]] = field(default_factory=list)  # per step [n_seq][n_drift]
    needles: dict = field(default_factory=dict)  # (s, kv) -> (pages, q_head, token)


def prefix_layout(prefix_lens: Sequence[int], page: int):
    """Pack sequences back to back in the cache; each starts on a page boundary."""
    lens = np.asarray(prefix_lens, dtype=np.int64)
    padded = (lens + page - 1) // page * page
    off = np.zeros(len(lens), dtype=np.int64)
    if len(lens) > 1:
        off[1:] = np.cumsum(padded)[:-1]
    total = int(padded.sum())
    total = max(total, page)
    return off.astype(np.int32), lens.astype(np.int32), total


def make_layer(cfg: Config, layer: int = 0, n_steps: Optional[int] = None,
               cache: bool = True) -> Layer:
    """Draw one layer's prefix cache and ``n_steps`` denoising steps of its block."""
    n_steps = cfg.n_steps if n_steps is None else n_steps
    S, B, Hq, Hkv, d, P = cfg.n_seq, cfg.block, cfg.n_qhead, cfg.n_kvhead, cfg.head_dim, cfg.page_size
    G = cfg.group
    kv_off, lens, T = prefix_layout(cfg.prefix_lens, P)
    cid = cfg.cfg_id

    if cache:
        k_cache = to_storage(_normal(_rng(cid, layer, _S_K), (Hkv, T, d)), cfg.dtype)
        v_cache = to_storage(_normal(_rng(cid, layer, _S_V), (Hkv, T, d)), cfg.dtype)
    else:
        k_cache = np.zeros((Hkv, T, d), np.float32)
        v_cache = np.zeros((Hkv, T, d), np.float32)
    # Positions past a sequence's prefix (page padding) hold zeros.
    for s in range(S):
        a, b = int(kv_off[s]) + int(lens[s]), int(kv_off[s]) + (int(lens[s]) + P - 1) // P * P
        k_cache[:, a:b] = 0.0
        v_cache[:, a:b] = 0.0

    q1 = to_storage(_normal(_rng(cid, layer, _S_Q), (S, B, Hq, d)), cfg.dtype)
    kb1 = to_storage(_normal(_rng(cid, layer, _S_KB), (S, B, Hkv, d)), cfg.dtype)
    vb1 = to_storage(_normal(_rng(cid, layer, _S_VB), (S, B, Hkv, d)), cfg.dtype)

    lay = Layer(cfg=cfg, layer=layer, kv_off=kv_off, prefix_len=lens, kv_tokens=T,
                k_cache=k_cache, v_cache=v_cache)

    if cfg.needles and cache:
        rng = _rng(cid, layer, _S_NEEDLE)
        for s in range(S):
            n_pages = (int(lens[s]) + P - 1) // P
            for g in range(Hkv):
                if n_pages == 0:
                    continue
                pages = np.sort(rng.choice(n_pages, size=min(cfg.n_needles, n_pages), replace=False))
                j = int(rng.integers(G))
                t = int(rng.integers(B))
                u = q1[s, t, g * G + j].astype(np.float64)
                u /= np.linalg.norm(u)
                c = cfg.needle_cos
                for p in pages:
                    lo = int(kv_off[s]) + int(p) * P
                    hi = int(kv_off[s]) + min((int(p) + 1) * P, int(lens[s]))
                    kk = k_cache[g, lo:hi].astype(np.float64)
                    nrm = np.linalg.norm(kk, axis=1, keepdims=True)
                    w = kk - (kk @ u)[:, None] * u[None, :]
                    w /= np.maximum(np.linalg.norm(w, axis=1, keepdims=True), 1e-30)
                    k_new = nrm * (c * u[None, :] + np.sqrt(1.0 - c * c) * w)
                    k_cache[g, lo:hi] = to_storage(k_new.astype(np.float32), cfg.dtype)
                lay.needles[(s, g)] = (pages.astype(np.int32), g * G + j, t)

    if cfg.dup_pages > 1 and cache:
        # ties: within each run of dup_pages whole pages, every page repeats the
        # keys of the run's first page (so their per-page min/max, and every
        # query's bound for them, are equal); partial last pages are left alone
        r = cfg.dup_pages
        for s in range(S):
            full = int(lens[s]) // P
            for p in range(full):
                if p % r:
                    src = int(kv_off[s]) + (p - p % r) * P
                    dst = int(kv_off[s]) + p * P
                    k_cache[:, dst:dst + P] = k_cache[:, src:src + P]

    q, kb, vb = q1, kb1, vb1
    for step in range(n_steps):
        if step == 0:
            lay.drift_tokens.append(None)
        else:
            tok_rng = _rng(cid, layer, _S_DRIFT_TOK, step)
            nd = min(cfg.drift_count, B)
            toks = np.stack([np.sort(tok_rng.choice(B, size=nd, replace=False)) for _ in range(S)]) \
                if nd > 0 else np.zeros((S, 0), np.int64)
            lay.drift_tokens.append(toks.astype(np.int32))

            def drift(x, stream, heads):
                r = _rng(cid, layer, stream, step)
                noise = _normal(r, (S, B, heads, d), cfg.stable_sigma)
                big = _normal(r, (S, B, heads, d), cfg.active_sigma)
                for s in range(S):
                    noise[s, toks[s]] = big[s, toks[s]]
                return to_storage(x + noise, cfg.dtype)

            q = drift(q, _S_DRIFT_Q, Hq)
            kb = drift(kb, _S_DRIFT_KB, Hkv)
            vb = drift(vb, _S_DRIFT_VB, Hkv)
        lay.q.append(q)
        lay.k_blk.append(kb)
        lay.v_blk.append(vb)
    return lay


def paged_pool(lay: Layer, seed: int = 0, spare: float = 0.25, share_pages: int = 0):
    """The layer's prefix scattered over a pool of physical pages (a paged KV
    cache): returns (k_pool, v_pool, page_table) with k_pool, v_pool
    [H_kv][16 * n_pool][d] and page_table [n_seq][max(1, pages of the longest
    prefix)] int32, where page p of sequence s is pool page page_table[s][p].
    The pool has ``spare`` more pages than the prefixes use, filled with N(0, 1)
    noise, and the pages are placed in a seeded random order.  With share_pages
    = n, every sequence after the first reuses the first sequence's first n
    whole pages: their keys and values are first copied into ``lay``'s own
    cache (so a contiguous reading sees the same prefix), then mapped to the
    same pool pages.  Data movement only."""
    c = lay.cfg
    P, S = c.page_size, c.n_seq
    lens = [int(x) for x in lay.prefix_len]
    pages = [(L + P - 1) // P for L in lens]
    if share_pages:
        full0 = lens[0] // P
        for s in range(1, S):
            n = min(share_pages, full0, lens[s] // P)
            a, b = int(lay.kv_off[0]), int(lay.kv_off[s])
            lay.k_cache[:, b:b + n * P] = lay.k_cache[:, a:a + n * P]
            lay.v_cache[:, b:b + n * P] = lay.v_cache[:, a:a + n * P]
    own = [pages[0]] + [pages[s] - (min(share_pages, lens[0] // P, lens[s] // P) if share_pages else 0)
                        for s in range(1, S)]
    used = sum(own)
    n_pool = max(1, used + int(np.ceil(used * spare)))
    rng = _rng(c.cfg_id, lay.layer, 30, 0, seed)
    order = rng.permutation(n_pool)
    k_pool = to_storage(_normal(rng, (c.n_kvhead, n_pool * P, c.head_dim)), c.dtype)
    v_pool = to_storage(_normal(rng, (c.n_kvhead, n_pool * P, c.head_dim)), c.dtype)
    max_pages = max(1, max(pages) if pages else 1)
    pt = np.zeros((S, max_pages), np.int32)
    nxt = 0
    for s in range(S):
        for p in range(pages[s]):
            if s > 0 and share_pages and p < min(share_pages, lens[0] // P, lens[s] // P):
                pt[s, p] = pt[0, p]
                continue
            e = int(order[nxt])
            nxt += 1
            pt[s, p] = e
            src = int(lay.kv_off[s]) + p * P
            k_pool[:, e * P:(e + 1) * P] = lay.k_cache[:, src:src + P]
            v_pool[:, e * P:(e + 1) * P] = lay.v_cache[:, src:src + P]
    return k_pool, v_pool, pt


def make_cache_state(cfg: Config, layer: int = 0, stream: int = 20):
    """A seeded (o_p, L_p) cache state: the prefix statistics a previous step left
    behind, for starting a step without running the dense pass first.
    o_p ~ N(0, 0.3); L_p = log(L) + N(0, 0.5) (-inf where the prefix is empty)."""
    rng = _rng(cfg.cfg_id, layer, stream)
    S, Hq, B, d = cfg.n_seq, cfg.n_qhead, cfg.block, cfg.head_dim
    op = _normal(rng, (S, Hq, B, d), 0.3)
    lp = _normal(rng, (S, Hq, B), 0.5)
    for s, L in enumerate(cfg.prefix_lens):
        if L > 0:
            lp[s] += np.float32(np.log(L))
        else:
            lp[s] = -np.inf
            op[s] = 0.0
    return op, lp


# ---------------------------------------------------------------------------
# The five workloads.

def tiny_f32() -> Config:
    """Single layer, fp32, two steps: L=1024, B=16, 4 query heads on 1 KV head, d=64,
    budget 64 tokens (4 pages), |A|=4; no needles."""
    return Config("tiny_f32_L1024", 1, 1, 16, 4, 1, 64, 16, 64, 4, "f32", (1024,), 2)


def gqa_16k() -> Config:
    """8B-class layer, bf16, four steps: L=16384, B=16, 32/8 heads, d=128, budget 128, |A|=4."""
    return Config("bf16_L16384_B16", 2, 1, 16, 32, 8, 128, 16, 128, 4, "bf16", (16384,), 4,
                  needles=True)


def long_64k(budget: int = 128, n_active: int = 4) -> Config:
    """Long-context layer, bf16, eight steps: L=65536, B=16, 32/8 heads, d=128."""
    return Config(f"bf16_L65536_B16_b{budget}_A{n_active}", 3, 1, 16, 32, 8, 128, 16, budget,
                  n_active, "bf16", (65536,), 8, needles=True)


def ragged_batch(seed_lens: int = 0) -> Config:
    """Eight sequences, prefixes uniform in [8192, 65536] (multiples of 16), B=32,
    budget 256, |A|=8 (25% of the block), six steps."""
    rng = _rng(4, 0, _S_LENS, 0, seed_lens)
    lens = tuple(int(x) * 16 for x in rng.integers(8192 // 16, 65536 // 16 + 1, size=8))
    return Config("bf16_ragged8_B32_b256_A8", 4, 8, 32, 32, 8, 128, 16, 256, 8, "bf16", lens, 6,
                  needles=True)


def trace_layer_active(layer: int) -> int:
    """|A| of the 36-layer trace: 2 in the first and last four layers, 6 in between."""
    return 2 if (layer < 4 or layer >= 32) else 6


def trace_128k(layer: int = 0) -> Config:
    """One layer of the 36-layer denoising trace: L=131072, B=16, 32/8 heads, d=128,
    budget 128, eight steps; |A| depends on the layer."""
    return Config(f"bf16_L131072_trace_layer{layer}", 5, 1, 16, 32, 8, 128, 16, 128,
                  trace_layer_active(layer), "bf16", (131072,), 8, needles=True)


def small_case(cfg_id: int, *, n_seq=None, block=16, n_qhead=4, n_kvhead=1, head_dim=64,
               page_size=16, budget=64, n_active=4, dtype="f32", prefix_lens=(1024,),
               n_steps=2, needles=False, n_drift=None, flags=0, stable_sigma=1e-3,
               dup_pages=1) -> Config:
    """A free-form small workload for sweeps over shapes and edge cases; one
    sequence per prefix length."""
    if n_seq is None:
        n_seq = len(prefix_lens)
    assert n_seq == len(prefix_lens), (n_seq, prefix_lens)
    return Config(f"small_{cfg_id}", 100 + cfg_id, n_seq, block, n_qhead, n_kvhead, head_dim,
                  page_size, budget, n_active, dtype, tuple(prefix_lens), n_steps,
                  needles=needles, n_drift=n_drift, flags=flags, stable_sigma=stable_sigma,
                  dup_pages=dup_pages)
