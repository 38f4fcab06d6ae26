"""Seeded synthetic workloads: shapes, per-head budgets and Q/K/V tensors.

This module only draws random inputs.  It holds none of the method's arithmetic
(no pooling, scoring, selection, attention or scheduling), so both the HIP path
and the CPU oracle may consume what it produces.

Shapes follow the attention layers the S-HPLB summaries evaluate (Llama-3.1-8B:
32 query / 8 KV heads, head_dim 128; Qwen2.5-72B: 64 / 8, head_dim 128; contexts
up to 128K -- Italian summary §4, Chinese summary §4).  Gaussian Q/K/V with
planted "hot" key blocks stand in for long-context retrieval content; no
benchmark item, dataset or weight is used.

Random streams: ``torch.Generator`` on the target device for the bulk Q/K/V
draws (the same seed gives the same tensor on the same device type), numpy
``PCG64`` for the small per-head draws (budgets, roles, hot blocks, directions).
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# purposes of the independent random streams
_P_Q, _P_K, _P_V, _P_DIR, _P_HOT, _P_BUDGET, _P_PAGES = range(7)


@dataclass(frozen=True)
class PrefillSpec:
    """One causal prefill attention layer."""

    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    block: int
    budget_kind: str  # "count", "loguniform" or "bimodal"
    counts: tuple = ()  # count mode: blocks per head (cycled over heads)
    lo: float = 0.0  # loguniform draw range, or bimodal (low, high) levels
    hi: float = 0.0
    mean: float = 0.0  # target mean ratio after the fixed-total rescale
    budget_fit: str = "rescale"  # "rescale" | "clamp" | "span" (see prefill_budgets)
    frac_high: float = 0.0  # bimodal: share of heads at the high level
    n_hot: int = 8
    hot_k: float = 2.0  # K gets +hot_k * u_h on hot blocks
    hot_q: float = 1.0  # Q gets +hot_q * u_h on every row

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "PrefillSpec":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class DecodeSpec:
    """One batched decode step: one query token per sequence over a contiguous
    KV cache of ``kv_len`` tokens."""

    name: str
    dtype: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_len: int
    n_streaming: int = 12
    stream_gran: int = 16
    stream_sink: int = 4
    stream_local: int = 64
    granularities: tuple = (16, 32, 64)
    tok_lo: int = 1024
    tok_hi: int = 8192
    n_hot: int = 8
    hot_k: float = 2.0
    hot_q: float = 1.0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "DecodeSpec":
        return dataclasses.replace(self, **kw)


TINY_F32 = PrefillSpec("tiny-causal-prefill-f32", "f32", 1, 4, 1, 64, 1024, 64, "count",
                       counts=(2, 4, 6, 8), n_hot=3)
LLAMA_32K = PrefillSpec("llama3.1-8b-prefill-32k", "bf16", 1, 32, 8, 128, 32768, 128, "loguniform",
                        lo=0.02, hi=0.50, mean=0.125)
LLAMA_128K = PrefillSpec("llama3.1-8b-prefill-128k", "bf16", 1, 32, 8, 128, 131072, 128, "loguniform",
                         lo=0.01, hi=0.40, mean=0.0625)
QWEN_64K = PrefillSpec("qwen2.5-72b-prefill-64k", "bf16", 1, 64, 8, 128, 65536, 128, "bimodal",
                       lo=0.03, hi=0.30, mean=0.12, frac_high=0.30)
DECODE_128K = DecodeSpec("llama3.1-8b-decode-128k-b16", "bf16", 16, 32, 8, 128, 131072)

# all named workloads; a workload's default seed is 1000 + its position here
WORKLOADS = [TINY_F32, LLAMA_32K, LLAMA_128K, QWEN_64K, DECODE_128K]
BY_NAME = {w.name: w for w in WORKLOADS}


def seed_of(spec) -> int:
    """Default seed of a named workload (by name, so variants made with
    ``with_`` keep the seed of the workload they derive from only if renamed
    back; pass an explicit seed for those)."""
    return 1000 + [w.name for w in WORKLOADS].index(spec.name)


def _rng(seed: int, purpose: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, purpose, *extra])))


def _torch_gen(device, seed: int, purpose: int, *extra: int) -> torch.Generator:
    ss = np.random.SeedSequence([seed, purpose, *extra]).generate_state(2, dtype=np.uint32)
    g = torch.Generator(device=device)
    g.manual_seed(int(ss[0]) << 32 | int(ss[1]))
    return g


def _unit_vectors(seed: int, n: int, d: int) -> np.ndarray:
    u = _rng(seed, _P_DIR).standard_normal((n, d))
    return (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


# ----------------------------------------------------------------------------
# per-head budgets (input convention; the budget *rule* lives in the method)
# ----------------------------------------------------------------------------


def prefill_budgets(spec: PrefillSpec, seed: int) -> dict:
    """Per-head budget parameters for a prefill spec.

    * ``count``: head ``h`` keeps ``counts[h % len(counts)]`` blocks per row.
    * ``loguniform``: ratios drawn log-uniform in ``[lo, hi]``, then scaled by a
      common factor so their mean is ``mean`` (the total is fixed; scaling every
      head by the same factor gives every head the same share of its demand).
    * ``bimodal``: ``round(frac_high * H)`` heads (a seeded choice) at ``hi``,
      the rest at ``lo``, then the same mean-preserving scale.

    ``budget_fit="clamp"`` (the alternative reading of the fixed-total shift):
    the common factor c is instead found by bisection so that the ratios
    clamped to ``[lo, hi]`` have mean ``mean``; every ratio stays inside the
    stated range (the plain rescale can move them below ``lo``).
    ``budget_fit="span"`` (log-uniform draws only): the drawn log-ratios are
    stretched onto the whole range, x = (log f - log f_min) / (log f_max -
    log f_min), and r = lo * (hi / lo) ** (x ** g) with g found by bisection so
    that the mean is ``mean``: the lowest head at ``lo``, the highest at ``hi``.

    Ratios are quantised once to units of 2**-16 (round half to even).
    """
    H = spec.n_q_heads
    r = _rng(seed, _P_BUDGET)
    min_blocks = np.full(H, 2, dtype=np.int32)
    ratio = np.zeros(H, dtype=np.int64)
    if spec.budget_kind == "count":
        min_blocks = np.array([spec.counts[h % len(spec.counts)] for h in range(H)], dtype=np.int32)
    elif spec.budget_kind in ("loguniform", "bimodal"):
        if spec.budget_kind == "loguniform":
            f = np.exp(r.uniform(math.log(spec.lo), math.log(spec.hi), H))
        else:
            n_high = int(round(spec.frac_high * H))
            f = np.full(H, spec.lo)
            f[r.permutation(H)[:n_high]] = spec.hi
        if spec.budget_fit == "rescale":
            f = f * (spec.mean / f.mean())
        elif spec.budget_fit == "clamp":
            if not spec.lo <= spec.mean <= spec.hi:
                raise ValueError("clamp fit needs lo <= mean <= hi")
            c_lo, c_hi = 0.0, spec.hi / f.min()  # mean of the clamped ratios grows with c, from lo to hi
            for _ in range(200):
                c = 0.5 * (c_lo + c_hi)
                if np.clip(c * f, spec.lo, spec.hi).mean() < spec.mean:
                    c_lo = c
                else:
                    c_hi = c
            f = np.clip(0.5 * (c_lo + c_hi) * f, spec.lo, spec.hi)
        elif spec.budget_fit == "span" and spec.budget_kind == "loguniform":
            x = (np.log(f) - np.log(f.min())) / (np.log(f.max()) - np.log(f.min()))
            g_lo, g_hi = 1e-3, 1e3  # the mean falls as g grows (x in [0, 1])
            for _ in range(200):
                g = math.sqrt(g_lo * g_hi)
                if (spec.lo * (spec.hi / spec.lo) ** (x ** g)).mean() > spec.mean:
                    g_lo = g
                else:
                    g_hi = g
            f = spec.lo * (spec.hi / spec.lo) ** (x ** math.sqrt(g_lo * g_hi))
        else:
            raise ValueError(spec.budget_fit)
        ratio = np.rint(f * 65536.0).astype(np.int64)
    else:
        raise ValueError(spec.budget_kind)
    return {
        "min_blocks": min_blocks,
        "ratio_q16": ratio.astype(np.int64),
        "n_sink": np.ones(H, dtype=np.int32),
        "n_local": np.ones(H, dtype=np.int32),
        "granularity": np.full(H, spec.block, dtype=np.int32),
    }


def decode_budgets(spec: DecodeSpec, seed: int) -> dict:
    """Per-head roles and budgets for a decode spec (same for every sequence).

    ``n_streaming`` heads (seeded choice) keep only their sink and local blocks
    at ``stream_gran`` tokens per block.  The others (retrieval heads) get a
    granularity drawn uniformly from ``granularities`` and a token budget drawn
    log-uniform in ``[tok_lo, tok_hi]``, floored to a multiple of the
    granularity; they keep the first and the last block and score the rest.
    """
    H = spec.n_q_heads
    r = _rng(seed, _P_BUDGET)
    streaming = np.zeros(H, dtype=bool)
    streaming[r.permutation(H)[: spec.n_streaming]] = True
    gran = np.empty(H, dtype=np.int32)
    min_blocks = np.empty(H, dtype=np.int32)
    n_sink = np.empty(H, dtype=np.int32)
    n_local = np.empty(H, dtype=np.int32)
    for h in range(H):
        if streaming[h]:
            gran[h] = spec.stream_gran
            n_sink[h], n_local[h] = spec.stream_sink, spec.stream_local
            min_blocks[h] = spec.stream_sink + spec.stream_local
        else:
            g = int(r.choice(spec.granularities))
            tok = math.exp(r.uniform(math.log(spec.tok_lo), math.log(spec.tok_hi)))
            gran[h] = g
            n_sink[h], n_local[h] = 1, 1
            min_blocks[h] = max(2, int(tok) // g)
    return {
        "min_blocks": min_blocks,
        "ratio_q16": np.zeros(H, dtype=np.int64),
        "n_sink": n_sink,
        "n_local": n_local,
        "granularity": gran,
        "streaming": streaming,
    }


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------


@dataclass
class PrefillInputs:
    spec: PrefillSpec
    seed: int
    q: torch.Tensor  # [b, Hq, S, D]
    k: torch.Tensor  # [b, Hkv, S, D]
    v: torch.Tensor
    budget: dict
    hot: np.ndarray  # [b, Hq, n_hot] planted key blocks
    u: np.ndarray  # [Hq, D] planted directions


@dataclass
class DecodeInputs:
    spec: DecodeSpec
    seed: int
    q: torch.Tensor  # [b, Hq, D]
    k: torch.Tensor  # [b, Hkv, L, D]
    v: torch.Tensor
    budget: dict
    hot: dict = field(default_factory=dict)  # (b, h) -> planted blocks
    u: Optional[np.ndarray] = None


def make_prefill(spec: PrefillSpec, seed: int, device="cpu") -> PrefillInputs:
    """Gaussian Q/K/V with planted hot key blocks, rounded once to ``spec.dtype``.

    Per query head ``h``: ``n_hot`` distinct key blocks drawn uniformly from
    ``1 .. NB-1``; every key row of those blocks in KV head ``h // G`` gets
    ``+hot_k * u_h`` (plants of different heads add), and every query row of
    head ``h`` gets ``+hot_q * u_h``, with ``u_h`` a seeded unit vector.
    """
    b, H, Hk, D, S, B = spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.seq_len, spec.block
    nb = spec.n_blocks
    G = H // Hk
    dev = torch.device(device)
    u = _unit_vectors(seed, H, D)
    rh = _rng(seed, _P_HOT)
    n_hot = min(spec.n_hot, max(0, nb - 1))
    hot = np.zeros((b, H, n_hot), dtype=np.int64)
    for bi in range(b):
        for h in range(H):
            hot[bi, h] = np.sort(rh.choice(np.arange(1, nb), size=n_hot, replace=False)) if n_hot else []
    dt = _torch_dtype(spec.dtype)

    def draw(shape, purpose):
        g = _torch_gen(dev, seed, purpose)
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32)

    ut = torch.from_numpy(u).to(dev)
    q = draw((b, H, S, D), _P_Q)
    q += spec.hot_q * ut[None, :, None, :]
    q = q.to(dt)
    k = draw((b, Hk, S, D), _P_K)
    for bi in range(b):
        for h in range(H):
            for n in hot[bi, h]:
                k[bi, h // G, n * B:min(S, (n + 1) * B)] += spec.hot_k * ut[h]
    k = k.to(dt)
    v = draw((b, Hk, S, D), _P_V).to(dt)
    return PrefillInputs(spec, seed, q, k, v, prefill_budgets(spec, seed), hot, u)


def make_decode(spec: DecodeSpec, seed: int, device="cpu") -> DecodeInputs:
    """Gaussian decode query and KV cache with planted hot blocks.

    Per sequence and retrieval head ``h`` (granularity ``g_h``): ``n_hot``
    distinct blocks drawn from ``1 .. L/g_h - 2`` get ``+hot_k * u_h`` on every
    key row in KV head ``h // G``, and the query gets ``+hot_q * u_h``.  The KV
    cache is drawn one sequence at a time.
    """
    b, H, Hk, D, L = spec.batch, spec.n_q_heads, spec.n_kv_heads, spec.head_dim, spec.kv_len
    G = H // Hk
    dev = torch.device(device)
    budget = decode_budgets(spec, seed)
    u = _unit_vectors(seed, H, D)
    ut = torch.from_numpy(u).to(dev)
    dt = _torch_dtype(spec.dtype)
    q = torch.randn((b, H, D), generator=_torch_gen(dev, seed, _P_Q), device=dev, dtype=torch.float32)
    k = torch.empty((b, Hk, L, D), device=dev, dtype=dt)
    v = torch.empty((b, Hk, L, D), device=dev, dtype=dt)
    hot = {}
    for bi in range(b):
        rh = _rng(seed, _P_HOT, bi)
        kb = torch.randn((Hk, L, D), generator=_torch_gen(dev, seed, _P_K, bi), device=dev, dtype=torch.float32)
        for h in range(H):
            if budget["streaming"][h]:
                continue
            g = int(budget["granularity"][h])
            nc = -(-L // g)
            cand = np.arange(1, max(1, nc - 1))
            nh = min(spec.n_hot, cand.size)
            blocks = np.sort(rh.choice(cand, size=nh, replace=False)) if nh else np.zeros(0, np.int64)
            hot[bi, h] = blocks
            for n in blocks:
                kb[h // G, n * g:min(L, (n + 1) * g)] += spec.hot_k * ut[h]
            q[bi, h] += spec.hot_q * ut[h]
        k[bi] = kb.to(dt)
        del kb
        v[bi] = torch.randn((Hk, L, D), generator=_torch_gen(dev, seed, _P_V, bi), device=dev,
                            dtype=torch.float32).to(dt)
    return DecodeInputs(spec, seed, q.to(dt), k, v, budget, hot, u)


@dataclass
class PagedKV:
    k_pages: torch.Tensor  # [Hkv, pages_per_head, page_size, D]
    v_pages: torch.Tensor
    table: torch.Tensor  # int32 [b, Hkv, max_pages]: physical page of each logical page
    page_size: int
    kv_len: int


def make_paged(k: torch.Tensor, v: torch.Tensor, page_size: int, seed: int, spare_pages: int = 3) -> PagedKV:
    """The same cache scattered into per-KV-head page pools: logical page p of
    sequence b goes to a physical page drawn by a seeded permutation of the head's
    pool (``spare_pages`` pages of the pool stay unused, holding zeros).  Rows of
    a last page past the cache end are zero.  Pure data movement."""
    b, hk, L, D = k.shape
    mp = -(-L // page_size)
    pph = b * mp + spare_pages
    dev = k.device
    table = torch.empty((b, hk, mp), dtype=torch.int32)
    pools = []
    for x in (k, v):
        pool = torch.zeros((hk, pph, page_size, D), dtype=x.dtype, device=dev)
        pools.append(pool)
    for j in range(hk):
        perm = torch.from_numpy(_rng(seed, _P_PAGES, j).permutation(pph)[:b * mp].astype(np.int64))
        table[:, j, :] = perm.view(b, mp).to(torch.int32)
        idx = perm.to(dev)
        for x, pool in zip((k, v), pools):
            rows = torch.zeros((b, mp * page_size, D), dtype=x.dtype, device=dev)
            rows[:, :L] = x[:, j]
            pool[j].index_copy_(0, idx, rows.view(b * mp, page_size, D))
            del rows
    return PagedKV(pools[0], pools[1], table.to(dev), page_size, L)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor; bf16 tensors come back as uint16 bit patterns."""
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()
