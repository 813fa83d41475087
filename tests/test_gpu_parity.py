"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Each case names itself on stderr before it touches the GPU. The oracle builds
its own pool and page table; nothing it consumes comes from the GPU path.
"""

import numpy as np
import pytest

import workloads
from gpu_util import (TOL, CodedWorkload, check_close, coded, full_rows_rel, margin_line, oracle_ref,
                      sample_tokens, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_lora_amd import _lib, runtime
    _lib.load()
    return runtime


def _run(rt, wl, proj=0, policy=0, mode="apply", inst=None, x=None, y0=None):
    from heterogeneous_lora_amd import _lib
    inst = inst or rt.PagedLoRA(wl)
    call = inst.call(proj, policy)
    xd, yd = inst.inputs(proj)
    if x is not None:
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    if y0 is not None:
        yd = torch.from_numpy(np.ascontiguousarray(y0).view(np.int16)).cuda()
    ws = inst.workspace(call)
    if mode == "apply":
        inst.apply(call, xd, yd, ws)
        torch.cuda.synchronize()
        assert _lib.workspace_status(ws.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
        return yd.cpu().numpy().view(np.uint16), inst
    v = torch.zeros(wl.n_tokens, inst.r_max, dtype=torch.float32, device="cuda")
    inst.shrink(call, xd, v, ws)
    torch.cuda.synchronize()
    return v.cpu().numpy(), inst


SMALL = [
    dict(seed=101),
    dict(seed=102, dtype="bf16"),
    dict(seed=103, d_in=1000, d_out=520, page_elems=64, n_tokens=70, n_segments=5,
         rank_choices=(0, 1, 3, 8, 16, 40)),
    dict(seed=104, dtype="bf16", d_in=520, d_out=1032, page_elems=512, n_tokens=41,
         n_segments=0, rank_choices=(8, 64, 128), n_adapters=4),
    dict(seed=105, d_in=4096, d_out=1024, page_elems=1024, n_tokens=37, n_segments=2,
         rank_choices=(5, 16, 33), n_adapters=6),
    dict(seed=106, dtype="bf16", d_in=2048, d_out=4104, page_elems=2048, n_tokens=33,
         n_segments=0, rank_choices=(16, 24), n_adapters=3),
    # rows of 4097..5120 elements: a second, partial shrink batch, with page chunks
    # uniform over a 512-element slice (P = 512) and not (P = 768)
    dict(seed=107, d_in=4608, d_out=520, page_elems=512, n_tokens=40, n_segments=1,
         rank_choices=(8, 16, 40), n_adapters=4),
    dict(seed=108, dtype="bf16", d_in=5120, d_out=256, page_elems=768, n_tokens=29,
         n_segments=0, rank_choices=(3, 64), n_adapters=3),
]


POLICIES = [0, 1, 2]
POLICY_IDS = ["auto", "mbgmv", "sgmv"]


@pytest.mark.parametrize("kw", SMALL, ids=[f"s{k['seed']}" for k in SMALL])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_small_parity(rt, kw, policy):
    wl = workloads.random_small(**kw)
    say(f"[gpu] small parity {kw} policy={policy}")
    y, inst = _run(rt, wl, policy=policy)
    ref, _ = oracle_ref(wl, 0)
    margin_line(f"small s{kw['seed']} policy={POLICY_IDS[policy]}", check_close(y, ref, wl.dtype, f"small {kw}"))
    inst.close()


EDGE = [
    # one decode token, one adapter
    dict(seed=301, n_tokens=1, n_segments=0, p_none=0.0, rank_choices=(16,), n_adapters=1,
         d_in=256, d_out=256, page_elems=256),
    # one prefill token in a segment of its own, then one decode token
    dict(seed=326, n_tokens=2, n_segments=1, p_none=0.0, rank_choices=(8,), n_adapters=2,
         d_in=512, d_out=264, page_elems=128),
    # A^T rows at the 32-page limit, B rows over 33 pages with a ragged last page, rank 128
    dict(seed=303, d_in=2048, d_out=2056, page_elems=64, n_tokens=40, n_segments=2,
         rank_choices=(1, 128), n_adapters=3, p_none=0.0),
]


@pytest.mark.parametrize("kw", EDGE, ids=[f"e{k['seed']}" for k in EDGE])
@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_edge_parity(rt, kw, policy):
    wl = workloads.random_small(**kw)
    routed = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
    assert (routed >= 0).any()
    say(f"[gpu] edge parity {kw} policy={policy}")
    y, inst = _run(rt, wl, policy=policy)
    ref, _ = oracle_ref(wl, 0)
    check_close(y, ref, wl.dtype, f"edge {kw}")
    inst.close()


def test_empty_and_idle_calls(rt):
    """A call with no tokens and a call whose tokens all have no adapter (id -1 or rank
    0) succeed and leave y exactly as it was."""
    from heterogeneous_lora_amd import _lib
    wl = workloads.random_small(306, n_tokens=24, n_segments=2, rank_choices=(0, 8), n_adapters=3)
    say("[gpu] empty and idle calls")
    inst = rt.PagedLoRA(wl)
    x, y = inst.inputs(0)
    y_before = y.clone()
    stream = torch.cuda.current_stream().cuda_stream
    zero_rank = [a for a in range(wl.n_adapters) if wl.ranks[a] == 0]
    idle = lambda ids: np.where(np.arange(ids.size) % 2 == 0, -1,
                                zero_rank[0] if zero_rank else -1).astype(np.int32)
    for name, over in (("empty", dict(n_tokens=0, seg_offsets=np.zeros(1, np.int32),
                                      seg_adapter=np.zeros(0, np.int32),
                                      token_adapter=np.zeros(0, np.int32))),
                       ("idle", dict(seg_adapter=idle(wl.seg_adapter),
                                     token_adapter=idle(wl.token_adapter)))):
        c = _lib.Call(pool_ptr=inst.pool_t.data_ptr(), n_pages=wl.n_pages, page_elems=wl.page_elems,
                      dtype=wl.dtype, d_in=wl.projections[0].d_in, d_out=wl.projections[0].d_out,
                      page_table_ptr=inst.pt_dev[0].data_ptr(), page_table_len=inst.pt_len[0],
                      base=inst.base[0], rank=wl.ranks, scale=wl.scales.astype(np.float32),
                      r_max=inst.r_max, policy=0,
                      **{**dict(n_tokens=wl.n_tokens, seg_offsets=wl.seg_offsets,
                                seg_adapter=wl.seg_adapter, token_adapter=wl.token_adapter), **over})
        ws = inst.workspace(c)
        _lib.apply(c, x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        torch.cuda.synchronize()
        assert torch.equal(y, y_before), name
    inst.close()


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_tiny_decode_parity(rt, policy):
    wl = workloads.tiny(0)
    say(f"[gpu] tiny_decode parity policy={policy}")
    y, inst = _run(rt, wl, policy=policy)
    ref, _ = oracle_ref(wl, 0)
    margin_line(f"tiny_decode policy={POLICY_IDS[policy]} all rows", check_close(y, ref, wl.dtype, "tiny_decode"))
    inst.close()


@pytest.fixture(scope="module")
def decode7b(rt):
    wl = workloads.decode7b(0)
    say("[gpu] building decode_7b instance")
    inst = rt.PagedLoRA(wl)
    yield wl, inst
    inst.close()


def test_decode7b_parity(rt, decode7b):
    wl, inst = decode7b
    say("[gpu] decode_7b parity (all 256 tokens)")
    y, _ = _run(rt, wl, inst=inst)
    ref, _ = oracle_ref(wl, 0)
    rel = check_close(y, ref, wl.dtype, "decode_7b")
    margin_line("decode_7b policy=auto all rows", rel)


def test_decode7b_sgmv_parity(rt, decode7b):
    """The same decode batch with every token forced onto SGMV tiles (adapter buckets)."""
    wl, inst = decode7b
    say("[gpu] decode_7b parity through SGMV")
    y, _ = _run(rt, wl, inst=inst, policy=2)
    ref, _ = oracle_ref(wl, 0)
    margin_line("decode_7b policy=sgmv all rows", check_close(y, ref, wl.dtype, "decode_7b sgmv"))


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_decode7b_shrink_v(rt, decode7b, policy):
    wl, inst = decode7b
    say(f"[gpu] decode_7b shrink v parity policy={policy}")
    v, _ = _run(rt, wl, inst=inst, mode="shrink", policy=policy)
    _, v_ref = oracle_ref(wl, 0, want_v=True)
    ids = wl.token_adapter
    for t in range(wl.n_tokens):
        r = int(wl.ranks[ids[t]])
        scale = max(1.0, float(np.max(np.abs(v_ref[t, :r]))))
        err = float(np.max(np.abs(v[t, :r] - v_ref[t, :r])))
        assert err <= TOL * scale, (t, err, scale)


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_decode7b_expand_only(rt, decode7b, policy):
    """slora_expand fed the oracle's v (as fp32) reproduces the oracle's y."""
    wl, inst = decode7b
    say(f"[gpu] decode_7b expand-only parity policy={policy}")
    ref, v_ref = oracle_ref(wl, 0, want_v=True)
    call = inst.call(0, policy)
    _, yd = inst.inputs(0)
    vt = torch.zeros(wl.n_tokens, inst.r_max, dtype=torch.float32)
    vt[:, :v_ref.shape[1]] = torch.from_numpy(v_ref.astype(np.float32))
    vt = vt.cuda()
    ws = inst.workspace(call)
    inst.expand(call, vt, yd, ws)
    torch.cuda.synchronize()
    check_close(yd.cpu().numpy().view(np.uint16), ref, wl.dtype, "decode_7b expand")


def test_decode7b_batch_invariance(rt, decode7b):
    """A token's output does not depend on which other tokens share its batch (bit-exact)."""
    wl, inst = decode7b
    say("[gpu] decode_7b batch invariance")
    y_all, _ = _run(rt, wl, inst=inst)
    sub = workloads.decode7b(0)
    keep = np.arange(0, wl.n_tokens, 3)
    sub.token_adapter = wl.token_adapter[keep].copy()
    x = wl.x(0)[keep]
    y0 = wl.y0(0)[keep]
    call = inst.call(0, wl=sub)
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    yd = torch.from_numpy(np.ascontiguousarray(y0).view(np.int16)).cuda()
    ws = inst.workspace(call)
    inst.apply(call, xd, yd, ws)
    torch.cuda.synchronize()
    assert np.array_equal(yd.cpu().numpy().view(np.uint16), y_all[keep])


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_page_permutation_bit_identical(rt, policy):
    """Two pools with different shuffles (so every page sits elsewhere) give identical bits,
    and a second call on the same inputs repeats the first bit for bit."""
    wl = workloads.random_small(201, d_in=1024, d_out=1536, page_elems=512, n_tokens=150,
                                n_segments=3, rank_choices=(8, 16, 32, 100), n_pages=8192)
    say(f"[gpu] page permutation policy={policy}")
    a = rt.PagedLoRA(wl, pool_seed=1)
    b = rt.PagedLoRA(wl, pool_seed=2)
    assert not np.array_equal(a.pt_dev[0].cpu().numpy(), b.pt_dev[0].cpu().numpy())
    ya, _ = _run(rt, wl, inst=a, policy=policy)
    yb, _ = _run(rt, wl, inst=b, policy=policy)
    ya2, _ = _run(rt, wl, inst=a, policy=policy)
    assert np.array_equal(ya, yb)
    assert np.array_equal(ya, ya2)
    a.close()
    b.close()


@pytest.mark.parametrize("policy", POLICIES, ids=POLICY_IDS)
def test_idle_tokens_untouched(rt, policy):
    wl = workloads.random_small(202, n_tokens=60, n_segments=0, p_none=0.4,
                                rank_choices=(0, 0, 8, 16), d_in=512, d_out=768, page_elems=256)
    say(f"[gpu] idle tokens pass through policy={policy}")
    y, inst = _run(rt, wl, policy=policy)
    ids = wl.token_adapter
    idle = (ids < 0) | (wl.ranks[np.maximum(ids, 0)] == 0)
    assert idle.any() and (~idle).any()
    assert np.array_equal(y[idle], wl.y0(0)[idle])
    inst.close()


def test_fetch_byte_exact_and_sentinels(rt):
    """Pages hold exactly the host rows; page tails, KV and free pages keep the NaN sentinel."""
    wl = workloads.random_small(203, d_in=1000, d_out=264, page_elems=256, n_tokens=30,
                                n_segments=0, rank_choices=(3, 8), n_adapters=4, n_pages=300)
    say("[gpu] fetch byte-exact")
    inst = rt.PagedLoRA(wl)
    torch.cuda.synchronize()
    pool = inst.pool_t.cpu().numpy().view(np.uint16).reshape(wl.n_pages, wl.page_elems)
    P = wl.page_elems
    p = wl.projections[0]
    cA, cB = -(-p.d_in // P), -(-p.d_out // P)
    pt = inst.pt_dev[0].cpu().numpy()
    sentinel = rt.SENTINEL_I16[wl.dtype]
    touched = np.zeros(wl.n_pages, bool)
    for a in inst.adapters:
        at, b = wl.adapter(a, 0)
        r = at.shape[0]
        base = int(inst.base[0][a])
        for k in range(r):
            for half, rows, c, L in ((0, at, cA, p.d_in), (1, b, cB, p.d_out)):
                for ch in range(c):
                    e = base + (0 if half == 0 else r * cA) + k * c + ch
                    page = pt[e]
                    n = min(P, L - ch * P)
                    assert np.array_equal(pool[page, :n], rows[k, ch * P:ch * P + n]), (a, k, half, ch)
                    assert np.all(pool[page, n:] == sentinel)
                    touched[page] = True
    assert np.all(pool[~touched] == sentinel)
    owners = inst.pool.owners()
    assert set(np.nonzero(touched)[0]) == set(np.nonzero(owners >= 0)[0])
    inst.close()


def _check_pages(rt, wl, inst, adapters):
    """Every page of `adapters` holds exactly its host rows with the sentinel past the row
    end; returns the set of pages checked."""
    pool = inst.pool_t.cpu().numpy().view(np.uint16).reshape(inst.n_pages, wl.page_elems)
    P = wl.page_elems
    sentinel = rt.SENTINEL_I16[wl.dtype]
    seen = set()
    for pi, p in enumerate(wl.projections):
        cA, cB = -(-p.d_in // P), -(-p.d_out // P)
        pt = inst.pt_dev[pi].cpu().numpy()
        for a in adapters:
            at, b = wl.adapter(a, pi)
            r = at.shape[0]
            base = int(inst.base[pi][a])
            for k in range(r):
                for half, rows, c, L in ((0, at, cA, p.d_in), (1, b, cB, p.d_out)):
                    for ch in range(c):
                        page = pt[base + (0 if half == 0 else r * cA) + k * c + ch]
                        n = min(P, L - ch * P)
                        assert np.array_equal(pool[page, :n], rows[k, ch * P:ch * P + n]), (a, pi, k, half, ch)
                        assert np.all(pool[page, n:] == sentinel)
                        seen.add(int(page))
    return seen


def test_fetch_many_rounds_and_duplicates(rt):
    """Batched fetches in more rounds than the library keeps pinned page lists (each list is
    refilled only after its launch finished): every round leaves exactly its adapters' pages
    written, an id given twice included, the other pages untouched."""
    wl = workloads.random_small(213, d_in=1000, d_out=264, page_elems=256, n_tokens=30,
                                n_segments=0, rank_choices=(3, 8, 16), n_adapters=7, n_pages=600)
    say("[gpu] fetch_many rounds")
    inst = rt.PagedLoRA(wl, adapters=list(range(wl.n_adapters)))
    side = torch.cuda.Stream()
    rng = np.random.default_rng(3)
    sentinel = rt.SENTINEL_I16[wl.dtype]
    for rnd in range(6):
        torch.cuda.synchronize()
        inst.pool_t.fill_(sentinel)
        torch.cuda.synchronize()
        pick = [int(a) for a in rng.choice(wl.n_adapters, size=3, replace=False)]
        ids = pick + [pick[0]]
        rows = [inst.store.ptrs(a, 1) for a in ids]
        done = torch.cuda.Event()
        side.wait_stream(torch.cuda.current_stream())
        inst.pool.fetch_many_async(ids, [r[0] for r in rows], [r[1] for r in rows],
                                   side.cuda_stream, done.cuda_event)
        done.synchronize()
        seen = _check_pages(rt, wl, inst, pick)
        pool = inst.pool_t.cpu().numpy().view(np.uint16).reshape(inst.n_pages, wl.page_elems)
        rest = np.ones(inst.n_pages, bool)
        rest[list(seen)] = False
        assert np.all(pool[rest] == sentinel), rnd
    inst.close()


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_probe_codes_bit_exact(rt, policy):
    """Integer-coded adapters: one-hot x reads back every A^T code exactly through shrink
    (page gathers and token routing are bit-exact)."""
    for dt in ("f16", "bf16"):
        base_wl = workloads.random_small(204, dtype=dt, d_in=1536, d_out=1040, page_elems=512,
                                         n_tokens=24, n_segments=0, rank_choices=(4, 8, 16),
                                         p_none=0.0, n_adapters=5)
        wl = coded(base_wl)
        say(f"[gpu] probe codes {dt} policy={policy}")
        inst = rt.PagedLoRA(wl)
        p = wl.projections[0]
        js = np.random.default_rng(5).choice(p.d_in, size=wl.n_tokens)
        x = np.zeros((wl.n_tokens, p.d_in), np.float32)
        x[np.arange(wl.n_tokens), js] = 1.0
        xb = workloads.to_bits(x, dt)
        call = inst.call(0, policy)
        v = torch.zeros(wl.n_tokens, inst.r_max, dtype=torch.float32, device="cuda")
        ws = inst.workspace(call)
        inst.shrink(call, torch.from_numpy(xb.view(np.int16)).cuda(), v, ws)
        torch.cuda.synchronize()
        v = v.cpu().numpy()
        for t in range(wl.n_tokens):
            a = int(wl.token_adapter[t])
            r = int(wl.ranks[a])
            want = _codes(a, r, js[t])
            assert np.array_equal(v[t, :r], want), (dt, t)
        inst.close()


def _codes(a, r, j):
    return np.array([CodedWorkload.code(a, 0, k, j, 0) for k in range(r)], np.float32)


def test_fetch_waits_and_free_state(rt):
    """A fetch queued behind a slow side stream is still complete when apply runs after the
    event; freeing the adapter while that fetch is in flight is refused (E_STATE)."""
    from heterogeneous_lora_amd import _lib
    wl = workloads.random_small(205, d_in=512, d_out=512, page_elems=512, n_tokens=16,
                                n_segments=0, rank_choices=(8,), p_none=0.0, n_adapters=2)
    say("[gpu] fetch ordering / E_STATE")
    inst = rt.PagedLoRA(wl)
    torch.cuda.synchronize()
    inst.pool_t.fill_(rt.SENTINEL_I16[wl.dtype])  # wipe fetched pages
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    done.record(side)
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)  # bounded spin delays the side stream
    side.wait_stream(torch.cuda.current_stream())
    for a in inst.adapters:
        at, b = inst.store.ptrs(a, 1)
        inst.pool.fetch_async(a, at, b, side.cuda_stream, done.cuda_event)
    with pytest.raises(_lib.SloraError) as e:
        inst.pool.free_adapter(inst.adapters[0])
    assert e.value.code == _lib.E_STATE
    torch.cuda.current_stream().wait_event(done)
    y, _ = _run(rt, wl, inst=inst, policy=1)
    ref, _ = oracle_ref(wl, 0)
    check_close(y, ref, wl.dtype, "fetch ordering")
    torch.cuda.synchronize()
    inst.pool.free_adapter(inst.adapters[0])
    inst.close()


@pytest.mark.parametrize("n_streams", [1, 2], ids=["one-stream", "two-streams"])
def test_staging_ring_reuse(rt, n_streams):
    """Work lists sit in a ring of pinned slots that the host refills once the kernels
    that read them are done. With the streams held back by a bounded spin, the host runs
    more than two laps of the ring ahead of the GPU; every call must still run its own
    plan (three workloads alternate, so a slot refilled too early holds another plan)."""
    say(f"[gpu] staging ring reuse, {n_streams} stream(s)")
    wls = [workloads.random_small(seed=110 + i, n_tokens=30 + 9 * i, n_segments=i) for i in range(3)]
    insts = [rt.PagedLoRA(wl) for wl in wls]
    refs = [oracle_ref(wl, 0)[0] for wl in wls]
    ins = [inst.inputs(0) for inst in insts]
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)  # bounded spin: the GPU falls behind the host
    outs = []
    for i in range(40):
        k, s = i % 3, streams[i % n_streams]
        call = insts[k].call(0)
        x, y0 = ins[k]
        with torch.cuda.stream(s):
            y = y0.clone()
            ws = insts[k].workspace(call)
            insts[k].apply(call, x, y, ws, stream=s)
        outs.append((k, y, ws))
    torch.cuda.synchronize()
    first = {}
    for i, (k, y, ws) in enumerate(outs):
        bits = y.cpu().numpy().view(np.uint16)
        check_close(bits, refs[k], wls[k].dtype, f"call {i} (workload {k})")
        assert np.array_equal(bits, first.setdefault(k, bits)), f"call {i} differs from workload {k}'s first call"
    for inst in insts:
        inst.close()


def _rank_split_case():
    """160 short segments over two adapters of rank above 64 and two below, plus
    per-token ids: enough tiles of each kind that SGMV runs them as two launches."""
    import dataclasses
    wl = workloads.random_small(130, dtype="bf16", n_adapters=4, d_in=264, d_out=520,
                                page_elems=256, rank_choices=(8,))
    ranks = np.array([128, 16, 72, 40], np.int32)
    lens = 1 + (np.arange(160) * 7) % 5
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seg_ad = (np.arange(160) % 4).astype(np.int32)
    tok = ((np.arange(40) * 3) % 5 - 1).astype(np.int32)
    pages = int(ranks.sum()) * (-(-264 // 256) + -(-520 // 256)) + 17
    return dataclasses.replace(wl, ranks=ranks, scales=workloads._scales(ranks), seg_offsets=offs,
                               seg_adapter=seg_ad, token_adapter=tok, n_pages=pages)


@pytest.mark.parametrize("policy", [0, 2], ids=["auto", "sgmv"])
def test_rank_split_launches(rt, policy):
    """SGMV tiles of ranks above 64 and the rest in separate launches (82 tiles each):
    every output row against the oracle."""
    from heterogeneous_lora_amd import _lib
    wl = _rank_split_case()
    say(f"[gpu] rank-split SGMV launches, policy={policy}")
    inst = rt.PagedLoRA(wl)
    groups, _ = _lib.plan_inspect(inst.call(0, policy))
    sg = groups[groups[:, 0] == 1]
    assert (sg[:, 4] > 64).sum() >= 64 and (sg[:, 4] <= 64).sum() >= 64
    y, inst = _run(rt, wl, policy=policy, inst=inst)
    ref, _ = oracle_ref(wl, 0)
    check_close(y, ref, wl.dtype, "rank split")
    inst.close()


LARGE = [("mixed_13b", 1), ("mlp_asym", 1), ("prefill_sgmv", 0), ("mixed_13b", 0),
         ("mlp_asym", 2), ("mlp_asym", 0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,policy", LARGE, ids=[f"{n}-{POLICY_IDS[p]}" for n, p in LARGE])
def test_large_sampled(rt, name, policy):
    """Full-size workloads, every projection, checked on sampled rows (segment ends, batch
    ends, random); the projections checked on every row are in test_large_full_rows."""
    wl = workloads.make(name)
    say(f"[gpu] {name} policy={policy}, building instance")
    inst = rt.PagedLoRA(wl)
    ev = sample_tokens(wl, 48)
    for proj in range(len(wl.projections)):
        pname = wl.projections[proj].name
        say(f"[gpu] {name} proj {pname} policy={policy}")
        y, _ = _run(rt, wl, proj=proj, policy=policy, inst=inst)
        ref, _ = oracle_ref(wl, proj, ev)
        rel = check_close(y[ev], ref, wl.dtype, f"{name}/{proj}")
        margin_line(f"{name} proj={pname} policy={POLICY_IDS[policy]} {ev.size} sampled rows", rel)
        ids = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
        idle = ids < 0
        if idle.any():
            assert np.array_equal(y[idle], wl.y0(proj)[idle])
    inst.close()


# (workload, projections checked on every output row, routing policy)
FULL = [("prefill_sgmv", ("q",), 0), ("mixed_13b", ("q",), 0), ("mlp_asym", ("up", "down"), 0)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,projs,policy", FULL, ids=[f"{n}-{'+'.join(p)}" for n, p, _ in FULL])
def test_large_full_rows(rt, name, projs, policy):
    """Full-size workloads against the oracle on every output row of the named
    projections (the launch configuration the benchmark times): the prefill batch
    through SGMV (v rounded once to bf16 before the MFMA expand), the mixed batch
    through both families, the MLP shapes at 4096 -> 11008 and 11008 -> 4096."""
    wl = workloads.make(name)
    say(f"[gpu] {name} full rows, building instance")
    inst = rt.PagedLoRA(wl)
    for pname in projs:
        proj, _ = wl.proj(pname)
        say(f"[gpu] {name} proj {pname} policy={POLICY_IDS[policy]}: GPU apply, then oracle on all "
            f"{wl.n_tokens} rows")
        y, _ = _run(rt, wl, proj=proj, policy=policy, inst=inst)
        rel = full_rows_rel(y, wl, proj, wl.dtype, f"{name}/{pname}")
        margin_line(f"{name} proj={pname} policy={POLICY_IDS[policy]} all {wl.n_tokens} rows", rel)
    inst.close()


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_expand_probe_codes_bit_exact(rt, policy):
    """Expand probe: v = e_k (token t reads rank row k_t alone), B rows hold integer codes,
    y0 = 0 and the scale a power of two, so y[t, :] = s * B[k_t, :] exactly: every B page
    gather (three chunks per row, the last one ragged) and every token's routing read back
    bit for bit, through slora_expand, for both element types."""
    for dt in ("f16", "bf16"):
        base_wl = workloads.random_small(207, dtype=dt, d_in=520, d_out=1040, page_elems=512,
                                         n_tokens=26, n_segments=0, rank_choices=(4, 8, 16),
                                         p_none=0.0, n_adapters=5)
        wl = coded(base_wl)
        say(f"[gpu] expand probe {dt} policy={POLICY_IDS[policy]}")
        inst = rt.PagedLoRA(wl)
        p = wl.projections[0]
        call = inst.call(0, policy)
        ids = wl.token_adapter
        ks = np.array([np.random.default_rng(9 + t).integers(int(wl.ranks[a])) for t, a in enumerate(ids)])
        v = np.zeros((wl.n_tokens, inst.r_max), np.float32)
        v[np.arange(wl.n_tokens), ks] = 1.0
        y = torch.zeros(wl.n_tokens, p.d_out, dtype=torch.int16, device="cuda")  # y0 = +0
        ws = inst.workspace(call)
        inst.expand(call, torch.from_numpy(v).cuda(), y, ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy().view(np.uint16)
        for t in range(wl.n_tokens):
            a = int(ids[t])
            s = float(wl.scales[a])
            assert s in (1.0, 2.0, 4.0)
            codes = np.array([CodedWorkload.code(a, 0, int(ks[t]), n, 1) for n in range(p.d_out)],
                             np.float32)
            want = workloads.to_bits(codes * np.float32(s), dt)
            assert np.array_equal(got[t], want), (dt, t, a, int(ks[t]))
        inst.close()


# decode ids spread over many adapters (MBGMV groups) beside a few segments (SGMV tiles,
# ranks to 128, too few for a launch per rank class)
MIXED_ONE = dict(seed=122, dtype="f16", n_adapters=300, d_in=4096, d_out=4096, page_elems=4096,
                 n_tokens=1024, n_segments=6, rank_choices=(8, 16, 64, 128), p_none=0.05)


def test_mixed_call_one_launch(rt):
    """A call with decode ids and segments under AUTO routing runs both families in one
    launch (the timed kernels are one mixed_fused launch), matches the oracle on every row
    with a clean status, and gives the same bits on a second call. (The give-up path of
    each hand-off is forced in test_wait_giveup_is_sticky_and_cleared; in this launch the
    segment expand items come last and find their flags already set.)"""
    from heterogeneous_lora_amd import _lib
    wl = workloads.random_small(**MIXED_ONE)
    say(f"[gpu] mixed call in one launch: {wl.n_tokens} tokens, "
        f"{int(wl.seg_offsets[-1])} in {len(wl.seg_adapter)} segments")
    inst = rt.PagedLoRA(wl)
    call = inst.call(0)
    groups, _ = _lib.plan_inspect(call)
    assert (groups[:, 0] == 0).any() and (groups[:, 0] == 1).any(), "both families expected"
    assert (groups[groups[:, 0] == 1][:, 4] > 64).any() and (groups[groups[:, 0] == 1][:, 4] <= 64).any()
    x, y0 = inst.inputs(0)
    ws = inst.workspace(call)
    stream = torch.cuda.current_stream().cuda_stream
    _lib.timing_enable(True)
    y = y0.clone()
    inst.apply(call, x, y, ws)
    _lib.timing_enable(False)
    names, _ = _lib.timing_read_all()
    assert names == ["mixed_fused"], names
    assert _lib.workspace_status(ws.data_ptr(), stream) == 0
    ref, _ = oracle_ref(wl, 0)
    margin_line("mixed call in one launch, all rows",
                check_close(y.cpu().numpy().view(np.uint16), ref, wl.dtype, "mixed one launch"))
    first = y.cpu().numpy().view(np.uint16).copy()
    y = y0.clone()
    inst.apply(call, x, y, ws)
    assert _lib.workspace_status(ws.data_ptr(), stream) == 0
    assert np.array_equal(y.cpu().numpy().view(np.uint16), first)
    inst.close()


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_wait_giveup_is_sticky_and_cleared(rt, decode7b, policy):
    """The fused launch's bounded wait (decode v for MBGMV, a tile's partial-sum flags for
    SGMV), forced short from the host (every kernel still ends normally): a give-up in
    any of several calls is reported by the next status read, which clears it; with the
    default bound the same calls run clean and match the oracle."""
    from heterogeneous_lora_amd import _lib
    wl, inst = decode7b
    say(f"[gpu] decode_7b policy={POLICY_IDS[policy]} with a 1-poll wait bound: give-ups reported, then cleared")
    call = inst.call(0, policy)
    x, y0 = inst.inputs(0)
    ws = inst.workspace(call)
    stream = torch.cuda.current_stream().cuda_stream
    try:
        _lib.set_wait_limit(1)
        for _ in range(6):
            y = y0.clone()
            inst.apply(call, x, y, ws)
    finally:
        _lib.set_wait_limit(0)
    assert _lib.workspace_status(ws.data_ptr(), stream) == 1
    assert _lib.workspace_status(ws.data_ptr(), stream) == 0  # read once, then clear
    say(f"[gpu] decode_7b policy={POLICY_IDS[policy]} with the default wait bound after the give-ups")
    y = y0.clone()
    inst.apply(call, x, y, ws)
    assert _lib.workspace_status(ws.data_ptr(), stream) == 0
    ref, _ = oracle_ref(wl, 0)
    check_close(y.cpu().numpy().view(np.uint16), ref, wl.dtype, "decode_7b after give-ups")


@pytest.mark.parametrize("policy", [1, 2], ids=["mbgmv", "sgmv"])
def test_two_stream_decode_applies(rt, decode7b, policy):
    """Applies of the 7B decode batch on two workspaces and two streams, issued
    alternately with the host far ahead of the GPU, through either family's fused
    launch: the library orders the fused launches across the streams, every output
    matches the oracle and both workspaces report a clean status."""
    wl, inst = decode7b
    say(f"[gpu] decode_7b policy={POLICY_IDS[policy]} applies alternating over two streams")
    ref, _ = oracle_ref(wl, 0)
    x, y0 = inst.inputs(0)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    calls = [inst.call(0, policy), inst.call(0, policy)]
    wss = [inst.workspace(c) for c in calls]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)  # bounded spin: the host runs ahead
    outs = []
    for i in range(12):
        k = i % 2
        with torch.cuda.stream(streams[k]):
            y = y0.clone()
            inst.apply(calls[k], x, y, wss[k], stream=streams[k])
        outs.append((k, y))
    torch.cuda.synchronize()
    from heterogeneous_lora_amd import _lib
    for k in range(2):
        assert _lib.workspace_status(wss[k].data_ptr(), streams[k].cuda_stream) == 0
    first = None
    for i, (k, y) in enumerate(outs):
        bits = y.cpu().numpy().view(np.uint16)
        check_close(bits, ref, wl.dtype, f"two-stream call {i}")
        first = bits if first is None else first
        assert np.array_equal(bits, first), f"call {i} differs"
