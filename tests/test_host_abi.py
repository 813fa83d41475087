"""Host-side tests of libslora (CPU only: no HIP call reaches a device here).

* every function include/slora.h declares is exported;
* the unified pool's allocator: disjoint owners, page accounting, seeded
  determinism, all-or-nothing failure, state errors, page-table export layout;
* argument / routing validation of the compute calls (rejected before any launch);
* the planner's work lists, compared entry by entry with an independent Python
  model of the grouping rules.
"""

import re
import sys
import os

import numpy as np
import pytest

import workloads
from heterogeneous_lora_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_DEV = 0x7F0000000000  # never dereferenced by host code


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    hdr = open(os.path.join(ROOT, "include", "slora.h")).read()
    names = set(re.findall(r"^\s*(?:int|const char\*)\s+(slora_\w+)\s*\(", hdr, re.M))
    assert len(names) >= 17
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert _lib.abi_version() == 1


def _pool(n_pages=512, P=64, seed=3, dtype="f16"):
    return _lib.Pool(FAKE_DEV, n_pages, P, dtype, seed)


def test_pool_accounting_and_ownership():
    pool = _pool()
    pool.alloc_adapter(0, 8, [128, 64], [64, 200])   # cA = 2,1; cB = 1,4
    pool.alloc_adapter(5, 4, [128, 64], [64, 200])
    pool.alloc_adapter(2, 0, [128, 64], [64, 200])   # rank 0: no pages
    kv = pool.alloc_kv(37)
    own = pool.owners()
    need0 = 8 * ((2 + 1) + (1 + 4))
    need5 = 4 * ((2 + 1) + (1 + 4))
    assert (own == 0).sum() == need0 and (own == 5).sum() == need5
    assert (own == -2).sum() == 37 and set(own[kv]) == {-2}
    assert pool.info()["n_free"] == 512 - need0 - need5 - 37 == (own == -1).sum()
    for proj, (cA, cB) in enumerate([(2, 1), (1, 4)]):
        pt, base, rank = pool.page_table(proj, 8)
        assert list(rank) == [8, 0, 0, 0, 0, 4, 0, 0]
        assert base[0] == 0 and base[2] == 8 * (cA + cB) and base[5] == base[2]
        assert base[1] == base[3] == base[4] == base[6] == base[7] == -1
        assert pt.size == 12 * (cA + cB)
        assert set(own[pt[:base[5]]]) == {0} and set(own[pt[base[5]:]]) == {5}
    # the two projections' pages are disjoint and together are all the adapter's pages
    pt0, b0, _ = pool.page_table(0, 8)
    pt1, b1, _ = pool.page_table(1, 8)
    assert set(pt0[:24]).isdisjoint(pt1[:40])
    assert set(pt0[:24]) | set(pt1[:40]) == set(np.nonzero(own == 0)[0])
    pool.free_kv(kv[:10])
    assert pool.info()["n_free"] == 512 - need0 - need5 - 27 == pool.n_free()
    pool.free(kv[10:12])  # the scope's name for returning pages: same rules as free_kv
    assert pool.n_free() == 512 - need0 - need5 - 25
    with pytest.raises(_lib.SloraError) as e:
        pool.free(kv[10:11])  # already free
    assert e.value.code == _lib.E_INVALID and pool.n_free() == 512 - need0 - need5 - 25
    pool.alloc_kv(2)
    pool.free_adapter(0)
    assert (pool.owners() == 0).sum() == 0
    assert pool.info()["n_free"] == 512 - need5 - 27
    pool.destroy()


def test_pool_seeded_and_scattered():
    a, b, c = _pool(seed=11), _pool(seed=11), _pool(seed=12)
    for p in (a, b, c):
        p.alloc_adapter(1, 16, [64], [64])
    pa, pb, pc = (p.page_table(0, 2)[0] for p in (a, b, c))
    assert np.array_equal(pa, pb) and not np.array_equal(pa, pc)
    assert not np.array_equal(np.sort(pa), np.arange(pa.min(), pa.min() + pa.size))  # scattered
    for p in (a, b, c):
        p.destroy()


def test_pool_errors_all_or_nothing():
    pool = _pool(n_pages=40, P=64)
    with pytest.raises(_lib.SloraError) as e:
        pool.alloc_adapter(0, 32, [64], [64])  # 64 pages > 40
    assert e.value.code == _lib.E_POOL_FULL
    assert pool.info()["n_free"] == 40 and (pool.owners() == -1).all()
    pool.alloc_adapter(0, 4, [64], [64])
    with pytest.raises(_lib.SloraError) as e:
        pool.alloc_adapter(0, 4, [64], [64])
    assert e.value.code == _lib.E_STATE
    with pytest.raises(_lib.SloraError) as e:
        pool.alloc_kv(33)
    assert e.value.code == _lib.E_POOL_FULL and pool.info()["n_free"] == 32
    with pytest.raises(_lib.SloraError) as e:
        pool.free_adapter(3)
    assert e.value.code == _lib.E_STATE
    own = pool.owners()
    adapter_page = int(np.nonzero(own == 0)[0][0])
    with pytest.raises(_lib.SloraError) as e:
        pool.free_kv(np.array([adapter_page]))
    assert e.value.code == _lib.E_INVALID
    kv = pool.alloc_kv(2)
    with pytest.raises(_lib.SloraError):
        pool.free_kv(np.array([kv[0], kv[0]]))
    assert (pool.owners()[kv] == -2).all()
    for bad in (dict(d_in=[60], d_out=[64]), dict(d_in=[64], d_out=[64], rank=129),
                dict(d_in=[64], d_out=[64], rank=-1)):
        with pytest.raises(_lib.SloraError) as e:
            pool.alloc_adapter(9, bad.get("rank", 4), bad["d_in"], bad["d_out"])
        assert e.value.code == _lib.E_INVALID
    # a batched fetch checks every id before anything reaches a device
    with pytest.raises(_lib.SloraError) as e:
        pool.fetch_many_async([0, 7], [[0x1000], [0x1000]], [[0x1000], [0x1000]], 0, None)
    assert e.value.code == _lib.E_STATE and "adapter 7" in str(e.value)
    with pytest.raises(_lib.SloraError) as e:
        pool.fetch_many_async([0], [[0]], [[0]], 0, None)
    assert e.value.code == _lib.E_INVALID
    with pytest.raises(_lib.SloraError) as e:
        pool.fetch_many_async([0], [[0x1008]], [[0x1000]], 0, None)  # misaligned rows
    assert e.value.code == _lib.E_INVALID
    pool.fetch_many_async([], [], [], 0, None)  # nothing to move, nothing launched
    pool.destroy()
    with pytest.raises(_lib.SloraError):
        _lib.Pool(FAKE_DEV + 8, 10, 64, "f16", 0)  # misaligned
    with pytest.raises(_lib.SloraError):
        _lib.Pool(FAKE_DEV, 10, 60, "f16", 0)  # P % 8 != 0


# ------------------------------------------------------------------ compute-call validation

def _call(wl, policy=_lib.POLICY_AUTO, pool=None, **over):
    pool = pool or _lib.Pool(FAKE_DEV, wl.n_pages, wl.page_elems, wl.dtype, 1)
    p = wl.projections[0]
    for a in wl.active_adapters():
        if a not in getattr(pool, "_resident", set()):
            pool.alloc_adapter(int(a), int(wl.ranks[a]), [p.d_in], [p.d_out])
    pool._resident = set(int(a) for a in wl.active_adapters())
    pt, base, rank = pool.page_table(0, wl.n_adapters)
    args = dict(pool_ptr=FAKE_DEV, n_pages=wl.n_pages, page_elems=wl.page_elems, dtype=wl.dtype,
                d_in=p.d_in, d_out=p.d_out, page_table_ptr=FAKE_DEV, page_table_len=pt.size,
                base=base, rank=wl.ranks, scale=wl.scales, r_max=max(int(wl.ranks.max()), 1),
                n_tokens=wl.n_tokens, seg_offsets=wl.seg_offsets, seg_adapter=wl.seg_adapter,
                token_adapter=wl.token_adapter, policy=policy)
    args.update(over)
    return _lib.Call(**args), pool, pt, base


def _apply_code(call, ws_bytes=1 << 30):
    try:
        _lib.apply(call, FAKE_DEV, FAKE_DEV, FAKE_DEV, ws_bytes, 0)
    except _lib.SloraError as e:
        return e.code
    return 0


def test_validation_rejects_bad_calls():
    wl = workloads.random_small(3, n_tokens=20, n_segments=3, rank_choices=(4, 8))
    call, pool, pt, base = _call(wl)
    used = [a for a in wl.active_adapters()]
    cases = {
        "id_out_of_range": (dict(token_adapter=np.full_like(wl.token_adapter, wl.n_adapters)), _lib.E_INVALID),
        "id_below_minus_one": (dict(token_adapter=np.full_like(wl.token_adapter, -2)), _lib.E_INVALID),
        "offsets_decrease": (dict(seg_offsets=np.array([0, 5, 2, 4], np.int32)), _lib.E_INVALID),
        "offsets_past_end": (dict(seg_offsets=np.array([0, 5, 9, 21], np.int32),
                                  token_adapter=np.zeros(0, np.int32)), _lib.E_INVALID),
        "not_resident": (dict(base=np.full_like(base, -1)), _lib.E_STATE),
        "rank_above_r_max": (dict(r_max=1), _lib.E_INVALID),
        "r_max_too_big": (dict(r_max=129), _lib.E_INVALID),
        "page_table_short": (dict(page_table_len=int(pt.size) - 1), _lib.E_INVALID),
        "d_in_not_multiple_of_8": (dict(d_in=wl.projections[0].d_in + 4), _lib.E_INVALID),
        "bad_policy": (dict(policy=7), _lib.E_INVALID),
        # a row may span at most 32 pages (a wave holds the page ids of two A^T rows)
        "d_in_spans_33_pages": (dict(d_in=33 * wl.page_elems), _lib.E_INVALID),
        "scale_not_finite": (dict(scale=np.full(wl.n_adapters, np.nan, np.float32)), _lib.E_INVALID),
        "empty_segment_bad_id": (dict(seg_offsets=np.array([0, 0, 5, 9], np.int32),
                                      seg_adapter=np.array([wl.n_adapters, 0, 1], np.int32),
                                      token_adapter=np.zeros(wl.n_tokens - 9, np.int32)),
                                 _lib.E_INVALID),
    }
    assert len(wl.token_adapter) > 0 and used
    for name, (over, code) in cases.items():
        c, _, _, _ = _call(wl, pool=pool, **over)
        assert _apply_code(c) == code, name
    # workspace too small is rejected before anything is launched
    c, _, _, _ = _call(wl, pool=pool)
    assert _apply_code(c, ws_bytes=16) == _lib.E_INVALID
    assert "workspace" in _lib.last_error()
    # an all-idle batch (every id -1) does nothing and succeeds without touching HIP
    c, _, _, _ = _call(wl, pool=pool, seg_adapter=np.full_like(wl.seg_adapter, -1),
                       token_adapter=np.full_like(wl.token_adapter, -1))
    assert _apply_code(c) == 0
    # so does an empty call (no tokens, no segments)
    c, _, _, _ = _call(wl, pool=pool, n_tokens=0, seg_offsets=np.zeros(1, np.int32),
                       seg_adapter=np.zeros(0, np.int32), token_adapter=np.zeros(0, np.int32))
    assert _apply_code(c) == 0
    pool.destroy()


# ------------------------------------------------------------------ planner vs Python model

MB_GROUP, SG_TILE = 4, 64
AUTO_SGMV_TOK, AUTO_SGMV_BATCH, AUTO_MBGMV_MIN, AUTO_SGMV_SHARE = 4, 256, 128, 4


def _multi_code(calls, ws_bytes=1 << 30, xs=None, ys=None):
    n = len(calls)
    try:
        _lib.apply_multi(calls, xs or [FAKE_DEV] * n, ys or [FAKE_DEV] * n, FAKE_DEV, ws_bytes, 0)
    except _lib.SloraError as e:
        return e.code
    return 0


def test_apply_multi_validation():
    """slora_apply_multi refuses, before anything runs, projections that cannot share one
    plan (any field that fixes the plan differs, or the base / rank / scale arrays do),
    a projection count outside 1..8, misaligned x / y and a workspace smaller than one
    region per projection; its workspace is n regions of slora_workspace_size rounded
    to 256 bytes."""
    wl = workloads.random_small(3, n_tokens=20, n_segments=3, rank_choices=(4, 8))
    call, pool, pt, base = _call(wl)
    one = _lib.workspace_size(call)
    for n in (1, 3, 8):
        assert _lib.workspace_size_multi([call] * n) == n * ((one + 255) // 256 * 256)
    with pytest.raises(_lib.SloraError):
        _lib.workspace_size_multi([call] * 9)
    assert _multi_code([call] * 9) == _lib.E_INVALID
    assert _multi_code([call] * 2, ws_bytes=_lib.workspace_size_multi([call]) * 2 - 256) == _lib.E_INVALID
    assert "workspace" in _lib.last_error()
    assert _multi_code([call] * 2, xs=[FAKE_DEV, FAKE_DEV + 8]) == _lib.E_INVALID
    differing = {
        "d_out": dict(d_out=wl.projections[0].d_out + 8),
        "dtype": dict(dtype="bf16" if wl.dtype == "f16" else "f16"),
        "r_max": dict(r_max=int(wl.ranks.max()) + 1),
        "page_table_len": dict(page_table_len=int(pt.size) + 1),
        "pool": dict(pool_ptr=FAKE_DEV + 256),
        "base": dict(base=np.where(base >= 0, base + 1, base)),
        "scale": dict(scale=wl.scales * 2),
    }
    for name, over in differing.items():
        c2, _, _, _ = _call(wl, pool=pool, **over)
        assert _multi_code([call, c2]) == _lib.E_INVALID, name
        assert "projection 1" in _lib.last_error(), name
    # the same plan with another page table is accepted by validation; an all-idle batch
    # then returns before any launch
    idle = dict(seg_adapter=np.full_like(wl.seg_adapter, -1), token_adapter=np.full_like(wl.token_adapter, -1))
    c3, _, _, _ = _call(wl, pool=pool, page_table_ptr=FAKE_DEV + 4096, **idle)
    c4, _, _, _ = _call(wl, pool=pool, **idle)
    assert _multi_code([c4, c3]) == 0


def _even_split(toks, cap):
    n = len(toks)
    g = -(-n // cap)
    b, e = divmod(n, g)
    out, at = [], 0
    for i in range(g):
        m = b + (1 if i < e else 0)
        out.append(toks[at:at + m])
        at += m
    return out


def model_plan(wl, base, policy):
    """Independent model of the grouping: returns [(family, adapter, [tokens])] in dispatch order."""
    so, sa, ta = wl.seg_offsets, wl.seg_adapter, wl.token_adapter
    seg_end = int(so[-1])
    live = lambda a: a >= 0 and wl.ranks[a] > 0
    mb, sg, sg_ids = [], [], []
    for s in range(len(sa)):
        toks = list(range(int(so[s]), int(so[s + 1])))
        a = int(sa[s])
        if not toks or not live(a):
            continue
        if policy == _lib.POLICY_MBGMV:
            mb += [(a, t) for t in toks]
        else:
            sg += [(a, c) for c in _even_split(toks, SG_TILE)]
    dec = [(int(a), seg_end + q) for q, a in enumerate(ta) if live(int(a))]
    if policy == _lib.POLICY_AUTO:
        # an adapter's per-token ids go to SGMV from AUTO_SGMV_TOK of them, when segments run
        # anyway or there are at least AUTO_SGMV_BATCH such tokens (and at least a fifth of
        # the ids); when SGMV runs and
        # fewer than AUTO_MBGMV_MIN ids would be left for MBGMV, all of them go to SGMV
        cnt = {}
        for a, _ in dec:
            cnt[a] = cnt.get(a, 0) + 1
        hot = sum(c for c in cnt.values() if c >= AUTO_SGMV_TOK)
        cold = sum(c for c in cnt.values() if c < AUTO_SGMV_TOK)
        sg_runs = len(sg) > 0 or (hot >= AUTO_SGMV_BATCH and hot * AUTO_SGMV_SHARE >= cold)
        sg_hot = hot > 0 and sg_runs
        left = cold if sg_hot else cold + hot
        sg_all = sg_runs and 0 < left < AUTO_MBGMV_MIN
        for a, t in dec:
            (sg_ids if sg_all or (sg_hot and cnt[a] >= AUTO_SGMV_TOK) else mb).append((a, t))
    else:
        for a, t in dec:
            (sg_ids if policy == _lib.POLICY_SGMV else mb).append((a, t))
    def buckets(pairs, cap):
        pairs = sorted(pairs, key=lambda p: p[0])  # stable
        out = []
        for a in sorted(set(p[0] for p in pairs)):
            toks = [t for b, t in pairs if b == a]
            out += [(a, c) for c in _even_split(toks, cap)]
        return out
    mbg = buckets(mb, MB_GROUP)
    sg = sg + buckets(sg_ids, SG_TILE)
    key = lambda g: -int(wl.ranks[g[0]])
    mbg = sorted(mbg, key=key)
    sg = sorted(sg, key=key)
    return [(0, a, t) for a, t in mbg] + [(1, a, t) for a, t in sg]


@pytest.mark.parametrize("wl_name,policy", [
    ("tiny_decode", _lib.POLICY_AUTO), ("decode_7b", _lib.POLICY_AUTO),
    ("decode_7b", _lib.POLICY_SGMV), ("mixed_13b", _lib.POLICY_AUTO),
    ("mixed_13b", _lib.POLICY_MBGMV), ("mixed_13b", _lib.POLICY_SGMV),
    ("prefill_sgmv", _lib.POLICY_AUTO), ("mlp_asym", _lib.POLICY_AUTO), ("random", _lib.POLICY_AUTO),
    ("random", _lib.POLICY_MBGMV), ("random", _lib.POLICY_SGMV)])
def test_plan_matches_model(wl_name, policy):
    if wl_name == "random":
        wl = workloads.random_small(77, n_tokens=150, n_segments=7, rank_choices=(0, 2, 8, 16),
                                    n_adapters=9, p_none=0.2)
    else:
        wl = workloads.make(wl_name)
    call, pool, pt, base = _call(wl, policy)
    groups, toks = _lib.plan_inspect(call)
    model = model_plan(wl, base, policy)
    assert len(groups) == len(model)
    slot = 0
    for (fam, first, n, pt_base, rank), (mfam, ma, mtoks) in zip(groups, model):
        assert fam == mfam and n == len(mtoks) and first == slot
        assert pt_base == base[ma] and rank == wl.ranks[ma]
        assert list(toks[first:first + n]) == mtoks
        slot += n
    # every routed token exactly once
    ids = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
    routed = np.nonzero((ids >= 0) & (wl.ranks[np.maximum(ids, 0)] > 0))[0]
    assert np.array_equal(np.sort(toks), routed)
    pool.destroy()


def test_bench_accounting_follows_the_plan():
    """bench.py splits algorithmic bytes between the families by the library's own plan:
    every routed token is counted once, and a pure decode batch counts each active
    adapter's weights once plus x, y0 and y per token."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    for name in ("decode_7b", "mlp_asym", "mixed_13b"):
        wl = workloads.make(name)
        call, pool, pt, base = _call(wl)
        a = bench.algorithmic(wl, 0, call)
        ids = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
        routed = ids[(ids >= 0) & (wl.ranks[np.maximum(ids, 0)] > 0)]
        assert a["mbgmv_fused"]["tokens"] + a["sgmv_fused"]["tokens"] == routed.size
        if name == "decode_7b":
            p = wl.projections[0]
            w = sum(int(wl.ranks[x]) for x in np.unique(routed)) * (p.d_in + p.d_out) * 2
            assert a["mbgmv_fused"]["bytes"] == w + routed.size * (p.d_in + 2 * p.d_out) * 2
            assert a["sgmv_fused"]["tokens"] == 0
        elif name == "mlp_asym":  # 50 ids of adapters with < 4 tokens: too few for MBGMV
            assert a["mbgmv_fused"]["tokens"] == 0 and a["sgmv_fused"]["tokens"] == routed.size
        else:  # segments and hot adapters' ids on SGMV, ~360 singleton ids on MBGMV
            assert a["sgmv_fused"]["tokens"] > a["mbgmv_fused"]["tokens"] > 0
        assert a["mixed_fused"]["bytes"] == a["mbgmv_fused"]["bytes"] + a["sgmv_fused"]["bytes"]
        assert a["mixed_fused"]["mfma_flops"] == a["sgmv_fused"]["flops"]
        pool.destroy()
    # a step's calls: same-shape runs of projections in one slora_apply_multi each
    groups = {name: bench.projection_groups(workloads.make(name), True)
              for name in ("decode_7b", "prefill_sgmv", "mixed_13b", "mlp_asym")}
    assert groups == {"decode_7b": [[0]], "prefill_sgmv": [[0, 1, 2, 3]], "mixed_13b": [[0, 1, 2, 3]],
                      "mlp_asym": [[0, 1], [2]]}
    assert bench.projection_groups(workloads.make("prefill_sgmv"), False) == [[0], [1], [2], [3]]
    # a multi call's interval carries its projections' work, both families summed
    wl = workloads.make("mixed_13b")
    call, pool, pt, base = _call(wl)
    a = bench.algorithmic(wl, 0, call)
    alg = [a] * 4
    per = bench.launch_work(alg, [[0, 1, 2, 3]])
    assert list(per) == ["multi_fused"] and len(per["multi_fused"]) == 1
    b, f, m = per["multi_fused"][0]
    assert b == 4 * (a["mbgmv_fused"]["bytes"] + a["sgmv_fused"]["bytes"]) == 4 * a["mixed_fused"]["bytes"]
    assert f == 4 * a["mixed_fused"]["flops"] and m == 4 * a["sgmv_fused"]["flops"]
    single = bench.launch_work(alg, [[0], [1], [2], [3]])
    assert len(single["mixed_fused"]) == 4 and single["mixed_fused"][0][0] == a["mixed_fused"]["bytes"]
    pool.destroy()
