"""Seeded synthetic inputs for heterogeneous batched LoRA.

This module only draws random numbers and lays out input arrays. It holds none of
the LoRA arithmetic: no products, no page tables, no routing resolution. Both the
CPU oracle and the GPU path consume what it produces, and nothing else is shared
between them.

Five workloads are defined, sized after the serving scenario the S-LoRA pages
describe (review "S-LoRA: Serving Thousands of Concurrent LoRA Adapters",
abstract: thousands of adapters kept in host memory, the active ones fetched to
the GPU; "Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik": every token in
one batch may use its own adapter, ranks such as 8, 16 and 64 coexist).

Readings where the workload description is silent (all seeded, all stated):
  * N(0, 0.02) means standard deviation 0.02.
  * scale = alpha / rank with alpha = 16 for every workload.
  * x and y0 are drawn independently per projection, N(0, 1).
  * bounded Zipf: p(k) proportional to (k + 1) ** -a over k in [0, N), id 0 the
    most popular, drawn with Generator.choice.
  * integer lengths are uniform over inclusive ranges.
  * every draw has its own stream: SeedSequence(seed, spawn_key=(purpose, ...)).

Arrays of fp16 / bf16 values are returned as uint16 bit patterns. fp16 rounding
is numpy's float32 -> float16 cast; bf16 rounding is round-to-nearest-even on
the float32 bit pattern (inputs are finite Gaussians, so no NaN handling).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

ALPHA = 16.0

# purposes for independent random streams
_RANKS, _ROUTING, _LENGTHS, _X, _Y0, _ADAPTER, _KVLEN, _POOLSEED, _EXTRA = range(9)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + rounding) >> 16).astype(np.uint16)


def to_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f32_to_f16_bits(a)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def normal_bits(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bits(a, dtype)


def zipf_choice(rng: np.random.Generator, n: int, size: int, a: float) -> np.ndarray:
    p = np.arange(1, n + 1, dtype=np.float64) ** (-a)
    p /= p.sum()
    return rng.choice(n, size=size, p=p).astype(np.int32)


@dataclass(frozen=True)
class Projection:
    name: str
    d_in: int
    d_out: int


@dataclass
class Workload:
    """One seeded workload: routing, ranks, scales, pool geometry and lazily drawn arrays."""

    name: str
    dtype: str  # "f16" | "bf16"
    page_elems: int
    n_pages: int
    projections: List[Projection]
    n_adapters: int
    ranks: np.ndarray  # int32 [n_adapters]
    scales: np.ndarray  # float64 [n_adapters] (alpha / rank, 0 for rank 0)
    seg_offsets: np.ndarray  # int32 [S + 1]
    seg_adapter: np.ndarray  # int32 [S]
    token_adapter: np.ndarray  # int32 [T - seg_offsets[S]], -1 = none
    kv_seq_lens: np.ndarray  # int32: KV sequences that fill the pool after the adapters
    seed: int
    pool_seed: int
    description: str = ""
    _cache: Dict = field(default_factory=dict, repr=False)

    @property
    def n_tokens(self) -> int:
        return int(self.seg_offsets[-1]) + int(self.token_adapter.shape[0])

    @property
    def n_segments(self) -> int:
        return int(self.seg_adapter.shape[0])

    def active_adapters(self) -> np.ndarray:
        seg_len = np.diff(self.seg_offsets)
        used = np.concatenate([self.seg_adapter[seg_len > 0], self.token_adapter])
        used = used[used >= 0]
        return np.unique(used).astype(np.int32)

    def proj(self, name: str) -> Tuple[int, Projection]:
        for i, p in enumerate(self.projections):
            if p.name == name:
                return i, p
        raise KeyError(name)

    def adapter(self, adapter_id: int, proj: int) -> Tuple[np.ndarray, np.ndarray]:
        """(AT [r x d_in], B [r x d_out]) as uint16 bits; row k of AT is column k of A."""
        key = ("w", adapter_id, proj)
        if key in self._cache:
            return self._cache[key]
        p = self.projections[proj]
        r = int(self.ranks[adapter_id])
        rng = _rng(self.seed, _ADAPTER, adapter_id, proj)
        at = normal_bits(rng, (r, p.d_in), 0.02, self.dtype)
        b = normal_bits(rng, (r, p.d_out), 0.02, self.dtype)
        return at, b

    def x(self, proj: int) -> np.ndarray:
        p = self.projections[proj]
        return normal_bits(_rng(self.seed, _X, proj), (self.n_tokens, p.d_in), 1.0, self.dtype)

    def y0(self, proj: int) -> np.ndarray:
        p = self.projections[proj]
        return normal_bits(_rng(self.seed, _Y0, proj), (self.n_tokens, p.d_out), 1.0, self.dtype)

    def adapter_pages(self, adapter_id: int) -> int:
        """Pages one adapter occupies over all projections (one page per P elements of a row)."""
        r = int(self.ranks[adapter_id])
        P = self.page_elems
        return sum(r * (-(-p.d_in // P) + -(-p.d_out // P)) for p in self.projections)

    def weight_bytes(self, adapters) -> int:
        e = 2
        return int(sum(int(self.ranks[a]) * (p.d_in + p.d_out) * e
                       for a in adapters for p in self.projections))


def _scales(ranks: np.ndarray) -> np.ndarray:
    s = np.zeros(ranks.shape, dtype=np.float64)
    nz = ranks > 0
    s[nz] = ALPHA / ranks[nz]
    return s


def tiny(seed: int = 0) -> Workload:
    """8 decode tokens, h=256, one h->h projection, 4 adapters ranks {4,8,8,16}, fp16, 256-element pages."""
    ranks = np.array([4, 8, 8, 16], dtype=np.int32)
    tok = _rng(seed, _ROUTING).integers(0, 4, size=8).astype(np.int32)
    return Workload(
        name="tiny_decode", dtype="f16", page_elems=256, n_pages=256,
        projections=[Projection("proj", 256, 256)], n_adapters=4, ranks=ranks,
        scales=_scales(ranks), seg_offsets=np.zeros(1, np.int32),
        seg_adapter=np.zeros(0, np.int32), token_adapter=tok,
        kv_seq_lens=np.zeros(0, np.int32), seed=seed, pool_seed=seed,
        description="T=8, h=256, 4 adapters r={4,8,8,16}, fp16, P=256, 256-page pool")


def decode7b(seed: int = 0) -> Workload:
    """256 decode tokens, q-projection 4096->4096, 1000 host adapters r in {8,16,32,64}, Zipf(1.0) ids, fp16."""
    n = 1000
    ranks = _rng(seed, _RANKS).choice(np.array([8, 16, 32, 64], np.int32), size=n).astype(np.int32)
    tok = zipf_choice(_rng(seed, _ROUTING), n, 256, 1.0)
    return Workload(
        name="decode_7b", dtype="f16", page_elems=4096, n_pages=65536,
        projections=[Projection("q", 4096, 4096)], n_adapters=n, ranks=ranks,
        scales=_scales(ranks), seg_offsets=np.zeros(1, np.int32),
        seg_adapter=np.zeros(0, np.int32), token_adapter=tok,
        kv_seq_lens=np.zeros(0, np.int32), seed=seed, pool_seed=seed,
        description="T=256 decode, 4096->4096 q-proj, 1000 adapters r~U{8,16,32,64}, "
                    "Zipf(1.0) routing, fp16, P=4096, 65536-page pool")


def prefill(seed: int = 0) -> Workload:
    """64 requests, lengths U{8..512}, q/k/v/o 4096->4096, 200 adapters r in {8,16,32,64}, bf16."""
    n = 200
    ranks = _rng(seed, _RANKS).choice(np.array([8, 16, 32, 64], np.int32), size=n).astype(np.int32)
    lens = _rng(seed, _LENGTHS).integers(8, 512, size=64, endpoint=True).astype(np.int32)
    seg_adapter = _rng(seed, _ROUTING).integers(0, n, size=64).astype(np.int32)
    offs = np.zeros(65, np.int32)
    offs[1:] = np.cumsum(lens)
    projs = [Projection(nm, 4096, 4096) for nm in ("q", "k", "v", "o")]
    return Workload(
        name="prefill_sgmv", dtype="bf16", page_elems=4096, n_pages=65536,
        projections=projs, n_adapters=n, ranks=ranks, scales=_scales(ranks),
        seg_offsets=offs, seg_adapter=seg_adapter, token_adapter=np.zeros(0, np.int32),
        kv_seq_lens=np.zeros(0, np.int32), seed=seed, pool_seed=seed,
        description="64 segments U{8..512}, q/k/v/o 4096->4096, 200 adapters "
                    "r~U{8,16,32,64}, bf16, P=4096, 65536-page pool")


def mixed13b(seed: int = 0) -> Workload:
    """48 prefill segments U{16..256} + 512 decode tokens, q/k/v/o 5120->5120, 2000 adapters, Zipf(0.8), fp16."""
    n = 2000
    ranks = _rng(seed, _RANKS).choice(np.array([8, 16, 32, 64, 128], np.int32), size=n).astype(np.int32)
    lens = _rng(seed, _LENGTHS).integers(16, 256, size=48, endpoint=True).astype(np.int32)
    req = zipf_choice(_rng(seed, _ROUTING), n, 48 + 512, 0.8)
    offs = np.zeros(49, np.int32)
    offs[1:] = np.cumsum(lens)
    kv = _rng(seed, _KVLEN).integers(64, 2048, size=560, endpoint=True).astype(np.int32)
    projs = [Projection(nm, 5120, 5120) for nm in ("q", "k", "v", "o")]
    return Workload(
        name="mixed_13b", dtype="f16", page_elems=5120, n_pages=196608,
        projections=projs, n_adapters=n, ranks=ranks, scales=_scales(ranks),
        seg_offsets=offs, seg_adapter=req[:48].copy(), token_adapter=req[48:].copy(),
        kv_seq_lens=kv, seed=seed, pool_seed=seed,
        description="48 segments U{16..256} + 512 decode tokens, q/k/v/o 5120->5120, "
                    "2000 adapters r~U{8..128}, Zipf(0.8), fp16, P=5120, 196608-page pool "
                    "(KV for 560 sequences U{64..2048} fills the rest)")


def mlp(seed: int = 0, n_active: int = 500) -> Workload:
    """4096 decode tokens over n_active adapters (uniform), gate/up 4096->11008, down 11008->4096, bf16."""
    ranks = _rng(seed, _RANKS).choice(np.array([16, 32, 64, 128], np.int32), size=n_active).astype(np.int32)
    tok = _rng(seed, _ROUTING, n_active).integers(0, n_active, size=4096).astype(np.int32)
    projs = [Projection("gate", 4096, 11008), Projection("up", 4096, 11008),
             Projection("down", 11008, 4096)]
    # 524,288 pages hold 500 adapters' pages with room for KV; more adapters get a
    # proportionally larger pool (a multiple of 65,536 pages)
    n_pages = 524288 if n_active <= 500 else -(-int(n_active / 500 * 1.15 * 524288) // 65536) * 65536
    return Workload(
        name="mlp_asym" if n_active == 500 else f"mlp_asym_a{n_active}", dtype="bf16",
        page_elems=4096, n_pages=n_pages, projections=projs, n_adapters=n_active,
        ranks=ranks, scales=_scales(ranks), seg_offsets=np.zeros(1, np.int32),
        seg_adapter=np.zeros(0, np.int32), token_adapter=tok,
        kv_seq_lens=np.zeros(0, np.int32), seed=seed, pool_seed=seed,
        description=f"T=4096 decode over {n_active} adapters r~U{{16,32,64,128}}, "
                    "gate/up 4096->11008, down 11008->4096, bf16, P=4096, 524288-page pool")


CONFIGS = {
    "tiny_decode": tiny,
    "decode_7b": decode7b,
    "prefill_sgmv": prefill,
    "mixed_13b": mixed13b,
    "mlp_asym": mlp,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    return CONFIGS[name](seed, **kw)


def random_small(seed: int, *, dtype: str = "f16", n_adapters: int = 5, d_in: int = 96,
                 d_out: int = 80, page_elems: int = 32, n_tokens: int = 23,
                 n_segments: int = 3, rank_choices=(0, 1, 3, 8, 16), p_none: float = 0.15,
                 n_pages: int = 0) -> Workload:
    """Small random case for pins and parity: ragged segments, absent adapters, rank 0, d % P != 0."""
    rng = _rng(seed, _EXTRA)
    ranks = rng.choice(np.array(rank_choices, np.int32), size=n_adapters).astype(np.int32)
    n_seg_tok = int(rng.integers(0, n_tokens + 1)) if n_segments > 0 else 0
    cuts = np.sort(rng.integers(0, n_seg_tok + 1, size=max(n_segments - 1, 0)))
    offs = np.concatenate([[0], cuts, [n_seg_tok]]).astype(np.int32) if n_segments > 0 \
        else np.zeros(1, np.int32)
    seg_adapter = rng.integers(-1, n_adapters, size=n_segments).astype(np.int32)
    tok = rng.integers(0, n_adapters, size=n_tokens - n_seg_tok).astype(np.int32)
    tok[rng.random(tok.shape[0]) < p_none] = -1
    if n_pages == 0:
        c = -(-d_in // page_elems) + -(-d_out // page_elems)
        n_pages = int(ranks.sum()) * c + 17
    return Workload(
        name=f"random_small_{seed}", dtype=dtype, page_elems=page_elems, n_pages=n_pages,
        projections=[Projection("p", d_in, d_out)], n_adapters=n_adapters, ranks=ranks,
        scales=_scales(ranks), seg_offsets=offs, seg_adapter=seg_adapter,
        token_adapter=tok, kv_seq_lens=np.zeros(0, np.int32), seed=seed, pool_seed=seed,
        description="random small case")
