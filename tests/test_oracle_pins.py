"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin_* function takes a loaded oracle library and raises AssertionError on a
mismatch. The pytest tests run them on the real oracle; test_oracle_mutations.py
runs them on copies of the oracle with planted mistakes and requires that every
planted mistake fails at least one pin.

What pins what:
  * decoders      - exhaustive over all 65536 fp16 / bf16 bit patterns vs numpy.
  * arithmetic    - closed form: numpy fp64 y0 + s * (x @ A) @ B from the host
                    store (not the pool) on random small cases with d % P != 0,
                    ragged segments, absent adapters and rank 0; the tiny decode
                    workload; a hand-worked golden example (tests/golden).
  * single adapter- reduces to a plain GEMM (numpy matmul, other association).
  * routing       - id -1 / rank 0 give y0 exactly; segment and per-token
                    encodings agree bit for bit; permuting tokens permutes rows.
  * paging        - permuting physical pages gives bit-identical results;
                    one-hot probes read back exact pool values (shrink and expand).
  * scale         - doubling s doubles the delta exactly (y0 = 0).
"""

import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers (numpy only)

def np_decode(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def token_adapters(wl):
    """Per-token adapter id by expanding segments (numpy repeat)."""
    seg = np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets))
    return np.concatenate([seg, wl.token_adapter]).astype(np.int64)


def dense_reference(wl, proj, x=None, y0=None):
    """numpy fp64: y0 + s * ((x @ A) @ B) per token, from the host store."""
    p = wl.projections[proj]
    x = np_decode(wl.x(proj) if x is None else x, wl.dtype)
    y = np_decode(wl.y0(proj) if y0 is None else y0, wl.dtype).copy()
    ids = token_adapters(wl)
    for a in np.unique(ids):
        if a < 0 or wl.ranks[a] == 0:
            continue
        at, b = wl.adapter(int(a), proj)
        A = np_decode(at, wl.dtype).T  # d_in x r
        B = np_decode(b, wl.dtype)  # r x d_out
        rows = np.nonzero(ids == a)[0]
        y[rows] += wl.scales[a] * ((x[rows] @ A) @ B)
    return y


def _reference(wl, proj, lib, perm_seed=1, x=None, y0=None, want_v=False, eval_tokens=None,
               scales=None):
    p = wl.projections[proj]
    x = wl.x(proj) if x is None else x
    y0 = wl.y0(proj) if y0 is None else y0
    adapters = {int(a): wl.adapter(int(a), proj) for a in range(wl.n_adapters)
                if wl.ranks[a] > 0}
    pool, pt, base = oracle.build_pool(adapters, wl.n_adapters, p.d_in, p.d_out, wl.page_elems,
                                       wl.dtype, np.random.default_rng(perm_seed))
    return oracle.lora(dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out, x=x, y0=y0, pool=pool,
                       page_elems=wl.page_elems, page_table=pt, base=base, rank=wl.ranks,
                       scale=wl.scales if scales is None else scales,
                       seg_offsets=wl.seg_offsets, seg_adapter=wl.seg_adapter,
                       token_adapter=wl.token_adapter, eval_tokens=eval_tokens,
                       want_v=want_v, lib=lib)


def close(a, b, rel=1e-12):
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), "non-finite oracle output"
    assert err <= rel * scale, f"max err {err} > {rel} * {scale}"


SMALL_CASES = [
    dict(seed=1),
    dict(seed=2, dtype="bf16"),
    dict(seed=3, d_in=100, d_out=40, page_elems=16, n_segments=5),
    dict(seed=4, dtype="bf16", d_in=64, d_out=130, page_elems=64, n_segments=0),
    dict(seed=5, d_in=8, d_out=8, page_elems=8, n_tokens=9, rank_choices=(1, 2, 4)),
    dict(seed=6, d_in=200, d_out=56, page_elems=24, n_tokens=31, n_adapters=7,
         rank_choices=(0, 2, 5, 16, 24)),
]


# ----------------------------------------------------------------------------- pins

def pin_decoders(lib):
    allb = np.arange(65536, dtype=np.uint16)
    for dtype, f in (("f16", lib.oracle_half_to_double), ("bf16", lib.oracle_bfloat16_to_double)):
        got = np.array([f(int(b)) for b in allb], dtype=np.float64)
        ref = np_decode(allb, dtype)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), dtype
        assert np.array_equal(got[~nan], ref[~nan]), dtype


def pin_dense_small(lib):
    for kw in SMALL_CASES:
        wl = workloads.random_small(**kw)
        y, _ = _reference(wl, 0, lib, perm_seed=7)
        close(y, dense_reference(wl, 0))


def pin_dense_tiny_workload(lib):
    wl = workloads.tiny(0)
    y, _ = _reference(wl, 0, lib, perm_seed=3)
    close(y, dense_reference(wl, 0))


def pin_golden_hand_example(lib):
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    d_in, d_out, P, dtype = g["d_in"], g["d_out"], g["page_elems"], g["dtype"]
    ids = sorted(int(k) for k in g["adapters"])
    n_ad = max(ids) + 1
    ranks = np.zeros(n_ad, np.int32)
    scales = np.zeros(n_ad, np.float64)
    adapters = {}
    for k in ids:
        a = g["adapters"][str(k)]
        ranks[k] = a["rank"]
        scales[k] = a["scale"]
        adapters[k] = (workloads.f32_to_f16_bits(np.array(a["AT"], np.float32)),
                       workloads.f32_to_f16_bits(np.array(a["B"], np.float32)))
    toks = g["tokens"]
    x = workloads.f32_to_f16_bits(np.array([t["x"] for t in toks], np.float32))
    y0 = workloads.f32_to_f16_bits(np.array([t["y0"] for t in toks], np.float32))
    want = np.array([t["y"] for t in toks], np.float64)
    ta = np.array([t["adapter"] for t in toks], np.int32)
    for perm_seed in (0, 1):
        pool, pt, base = oracle.build_pool(adapters, n_ad, d_in, d_out, P, dtype,
                                           np.random.default_rng(perm_seed))
        y, _ = oracle.lora(dtype=dtype, d_in=d_in, d_out=d_out, x=x, y0=y0, pool=pool,
                           page_elems=P, page_table=pt, base=base, rank=ranks, scale=scales,
                           seg_offsets=np.zeros(1, np.int32), seg_adapter=np.zeros(0, np.int32),
                           token_adapter=ta, lib=lib)
        assert np.array_equal(y, want), (y, want)
    # the same routing with tokens 0..2 given as three one-token segments
    pool, pt, base = oracle.build_pool(adapters, n_ad, d_in, d_out, P, dtype,
                                       np.random.default_rng(5))
    y, _ = oracle.lora(dtype=dtype, d_in=d_in, d_out=d_out, x=x, y0=y0, pool=pool,
                       page_elems=P, page_table=pt, base=base, rank=ranks, scale=scales,
                       seg_offsets=np.array([0, 1, 2, 3], np.int32),
                       seg_adapter=np.array([0, 1, -1], np.int32),
                       token_adapter=np.array([0], np.int32), lib=lib)
    assert np.array_equal(y, want), (y, want)


def pin_single_adapter_gemm(lib):
    wl = workloads.random_small(11, d_in=72, d_out=48, page_elems=16, n_tokens=20,
                                n_segments=0, rank_choices=(8,), p_none=0.0, n_adapters=1)
    y, _ = _reference(wl, 0, lib)
    x = np_decode(wl.x(0), wl.dtype)
    y0 = np_decode(wl.y0(0), wl.dtype)
    at, b = wl.adapter(0, 0)
    W = np_decode(at, wl.dtype).T @ np_decode(b, wl.dtype)  # d_in x d_out
    close(y, y0 + wl.scales[0] * (x @ W), rel=1e-11)


def pin_absent_and_rank0_exact(lib):
    wl = workloads.random_small(21, n_tokens=40, n_segments=4, p_none=0.4,
                                rank_choices=(0, 0, 4, 8))
    y, _ = _reference(wl, 0, lib)
    ids = token_adapters(wl)
    idle = (ids < 0) | (wl.ranks[np.maximum(ids, 0)] == 0)
    assert idle.any() and (~idle).any()
    y0 = np_decode(wl.y0(0), wl.dtype)
    assert np.array_equal(y[idle], y0[idle])
    assert not np.array_equal(y[~idle], y0[~idle])


def pin_page_permutation(lib):
    for kw in SMALL_CASES[:4]:
        wl = workloads.random_small(**kw)
        y1, v1 = _reference(wl, 0, lib, perm_seed=100, want_v=True)
        y2, v2 = _reference(wl, 0, lib, perm_seed=200, want_v=True)
        assert np.array_equal(y1, y2) and np.array_equal(v1, v2)


def pin_token_permutation(lib):
    wl = workloads.random_small(31, n_tokens=25, n_segments=0)
    x, y0 = wl.x(0), wl.y0(0)
    y, _ = _reference(wl, 0, lib)
    perm = np.random.default_rng(3).permutation(wl.n_tokens)
    wl2 = workloads.random_small(31, n_tokens=25, n_segments=0)
    wl2.token_adapter = wl.token_adapter[perm].copy()
    y2, _ = _reference(wl2, 0, lib, x=x[perm].copy(), y0=y0[perm].copy())
    assert np.array_equal(y2, y[perm])


def pin_segment_vs_token_encoding(lib):
    wl = workloads.random_small(41, n_tokens=30, n_segments=6, p_none=0.0)
    y, _ = _reference(wl, 0, lib)
    ids = token_adapters(wl).astype(np.int32)
    wl2 = workloads.random_small(41, n_tokens=30, n_segments=6, p_none=0.0)
    wl2.seg_offsets = np.zeros(1, np.int32)
    wl2.seg_adapter = np.zeros(0, np.int32)
    wl2.token_adapter = ids
    y2, _ = _reference(wl2, 0, lib)
    assert np.array_equal(y, y2)
    # and the other way: every token its own segment
    wl3 = workloads.random_small(41, n_tokens=30, n_segments=6, p_none=0.0)
    wl3.seg_offsets = np.arange(31, dtype=np.int32)
    wl3.seg_adapter = ids
    wl3.token_adapter = np.zeros(0, np.int32)
    y3, _ = _reference(wl3, 0, lib)
    assert np.array_equal(y, y3)


def pin_scale_doubling(lib):
    wl = workloads.random_small(51, n_tokens=18, p_none=0.2)
    zero = np.zeros((wl.n_tokens, wl.projections[0].d_out), np.uint16)
    y1, _ = _reference(wl, 0, lib, y0=zero)
    y2, _ = _reference(wl, 0, lib, y0=zero, scales=wl.scales * 2.0)
    assert np.array_equal(y2, 2.0 * y1)
    assert np.any(y1 != 0)


def pin_probe_one_hot(lib):
    """One-hot x reads back A^T columns; one-hot A^T rows route v = e_m to B row m exactly."""
    d_in, d_out, P, r = 40, 36, 16, 5
    rng = np.random.default_rng(9)
    for dtype in ("f16", "bf16"):
        at_vals = rng.integers(-200, 200, size=(r, d_in)).astype(np.float32)
        b_vals = rng.integers(-200, 200, size=(r, d_out)).astype(np.float32)
        at, b = workloads.to_bits(at_vals, dtype), workloads.to_bits(b_vals, dtype)
        adapters = {1: (at, b)}
        pool, pt, base = oracle.build_pool(adapters, 2, d_in, d_out, P, dtype,
                                           np.random.default_rng(4))
        # shrink probe: x = e_j -> v[k] = AT[k, j]
        js = np.array([0, 15, 16, 17, 31, 32, 39])
        x = np.zeros((len(js), d_in), np.float32)
        x[np.arange(len(js)), js] = 1.0
        x = workloads.to_bits(x, dtype)
        y0 = np.zeros((len(js), d_out), np.uint16)
        ranks = np.array([0, r], np.int32)
        _, v = oracle.lora(dtype=dtype, d_in=d_in, d_out=d_out, x=x, y0=y0, pool=pool,
                           page_elems=P, page_table=pt, base=base, rank=ranks,
                           scale=np.array([0, 1.0]), seg_offsets=np.zeros(1, np.int32),
                           seg_adapter=np.zeros(0, np.int32),
                           token_adapter=np.ones(len(js), np.int32), want_v=True, lib=lib)
        assert np.array_equal(v, at_vals[:, js].T.astype(np.float64))
        # expand probe: AT rows one-hot at distinct positions pos[k]; x = e_{pos[m]} -> y = B[m]
        pos = np.array([3, 16, 21, 33, 38])
        oh = np.zeros((r, d_in), np.float32)
        oh[np.arange(r), pos] = 1.0
        adapters = {1: (workloads.to_bits(oh, dtype), b)}
        pool, pt, base = oracle.build_pool(adapters, 2, d_in, d_out, P, dtype,
                                           np.random.default_rng(8))
        x = np.zeros((r, d_in), np.float32)
        x[np.arange(r), pos] = 1.0
        x = workloads.to_bits(x, dtype)
        y, _ = oracle.lora(dtype=dtype, d_in=d_in, d_out=d_out, x=x,
                           y0=np.zeros((r, d_out), np.uint16), pool=pool, page_elems=P,
                           page_table=pt, base=base, rank=ranks, scale=np.array([0, 1.0]),
                           seg_offsets=np.zeros(1, np.int32), seg_adapter=np.zeros(0, np.int32),
                           token_adapter=np.ones(r, np.int32), lib=lib)
        assert np.array_equal(y, b_vals.astype(np.float64))


PINS = [pin_decoders, pin_dense_small, pin_dense_tiny_workload, pin_golden_hand_example,
        pin_single_adapter_gemm, pin_absent_and_rank0_exact, pin_page_permutation,
        pin_token_permutation, pin_segment_vs_token_encoding, pin_scale_doubling,
        pin_probe_one_hot]


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, lib):
    pin(lib)


def test_invalid_inputs_rejected(lib):
    wl = workloads.random_small(61, n_tokens=10, n_segments=2, p_none=0.0, rank_choices=(4,))
    p = wl.projections[0]
    adapters = {a: wl.adapter(a, 0) for a in range(wl.n_adapters)}
    pool, pt, base = oracle.build_pool(adapters, wl.n_adapters, p.d_in, p.d_out, wl.page_elems,
                                       wl.dtype, np.random.default_rng(0))
    common = dict(dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out, x=wl.x(0), y0=wl.y0(0), pool=pool,
                  page_elems=wl.page_elems, page_table=pt, rank=wl.ranks, scale=wl.scales,
                  lib=lib)
    ok = dict(base=base, seg_offsets=wl.seg_offsets, seg_adapter=wl.seg_adapter,
              token_adapter=wl.token_adapter)
    oracle.lora(**common, **ok)
    bad_id = dict(ok, token_adapter=np.full_like(wl.token_adapter, wl.n_adapters))
    bad_off = dict(ok, seg_offsets=np.array([0, 5, 3], np.int32))
    absent = dict(ok, base=np.full_like(base, -1))
    for bad in (bad_id, bad_off, absent):
        with pytest.raises(oracle.OracleError):
            oracle.lora(**common, **bad)


def test_threads_bit_identical(lib):
    wl = workloads.random_small(71, n_tokens=37)
    y1, _ = _reference(wl, 0, lib)
    p = wl.projections[0]
    adapters = {int(a): wl.adapter(int(a), 0) for a in range(wl.n_adapters) if wl.ranks[a] > 0}
    pool, pt, base = oracle.build_pool(adapters, wl.n_adapters, p.d_in, p.d_out, wl.page_elems,
                                       wl.dtype, np.random.default_rng(1))
    y4, _ = oracle.lora(dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out, x=wl.x(0), y0=wl.y0(0),
                        pool=pool, page_elems=wl.page_elems, page_table=pt, base=base,
                        rank=wl.ranks, scale=wl.scales, seg_offsets=wl.seg_offsets,
                        seg_adapter=wl.seg_adapter, token_adapter=wl.token_adapter,
                        n_threads=4, lib=lib)
    assert np.array_equal(y1, y4)


def test_eval_subset_matches_full(lib):
    wl = workloads.random_small(81, n_tokens=29, n_segments=3)
    y, _ = _reference(wl, 0, lib)
    ev = np.array([28, 0, 5, 5, 13], np.int64)
    ys, _ = _reference(wl, 0, lib, eval_tokens=ev)
    assert np.array_equal(ys, y[ev])


def test_reference_helper_matches(lib):
    """oracle.reference (only needed adapters placed) agrees with the full-pool run."""
    wl = workloads.random_small(91, n_tokens=21, n_segments=2)
    y, _ = _reference(wl, 0, lib)
    ev = np.array([3, 20, 7])
    yr, _ = oracle.reference(wl, 0, ev)
    assert np.array_equal(yr, y[ev])
