"""GPU tests of slora_apply_multi (several projections of one batch in one launch),
through the C ABI: every projection's output equals what slora_apply gives for that
projection alone, bit for bit where the two calls split the segment shrink into the same
k-ranges (one projection, decode groups only) and otherwise to rounding (the bound is
stated in gpu_util.assert_same_to_rounding); repeated calls give the same bits, the
workspace status is clean, and one projection of each case is also checked against the
oracle. A multi-projection launch may split the segment shrink into fewer k-ranges than
a one-projection launch, so the same fp32 terms are added in another grouping. Each
case names itself on stderr before it touches the GPU."""

import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import assert_same_to_rounding, check_close, margin_line, oracle_ref, sample_tokens, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_lora_amd import _lib, runtime
    _lib.load()
    return runtime


def _bits(t):
    return t.cpu().numpy().view(np.uint16)


def _assert_same(got, want, dtype, exact, what):
    """got == want bit for bit (exact), else to rounding (assert_same_to_rounding)."""
    if exact:
        assert np.array_equal(got, want), what
    else:
        assert_same_to_rounding(got, want, dtype, what)


def _multi_vs_single(rt, wl, projs=None, policy=0, launches=("multi_fused",), inst=None, exact=None):
    """Runs the projections one by one with slora_apply, then all at once with
    slora_apply_multi (twice: the second call finds the first call's flags and v words
    in the workspace), and requires the same outputs: bit for bit when `exact` (by
    default, for a single projection), else within one unit in the last place. Both
    multi calls must give the same bits. Returns (instance, multi outputs)."""
    from heterogeneous_lora_amd import _lib
    inst = inst or rt.PagedLoRA(wl)
    projs = list(range(len(wl.projections))) if projs is None else projs
    calls = [inst.call(p, policy) for p in projs]
    ins = [inst.inputs(p) for p in projs]
    stream = torch.cuda.current_stream().cuda_stream
    single = []
    for c, (x, y0) in zip(calls, ins):
        y = y0.clone()
        ws = inst.workspace(c)
        inst.apply(c, x, y, ws)
        single.append(_bits(y))
    if exact is None:
        exact = len(projs) == 1
    ws = torch.zeros(_lib.workspace_size_multi(calls), dtype=torch.uint8, device=inst.device)
    first = None
    for rep in range(2):
        ys = [y0.clone() for _, y0 in ins]
        _lib.timing_enable(True)
        _lib.apply_multi(calls, [x.data_ptr() for x, _ in ins], [y.data_ptr() for y in ys],
                         ws.data_ptr(), ws.numel(), stream)
        _lib.timing_enable(False)
        names, _ = _lib.timing_read_all()
        assert names == list(launches), names
        assert _lib.workspace_status(ws.data_ptr(), stream) == 0
        got = [_bits(y) for y in ys]
        for i, p in enumerate(projs):
            _assert_same(got[i], single[i], wl.dtype, exact, (wl.name, p, rep))
        if first is None:
            first = got
        else:
            for i in range(len(projs)):
                assert np.array_equal(got[i], first[i]), (wl.name, projs[i], "repeat")
    return inst, ys


def _small_multi(seed, n_proj, **kw):
    """random_small with n_proj projections of the same shape (a layer's q/k/v...)."""
    one = workloads.random_small(seed, **kw)
    c = -(-one.projections[0].d_in // one.page_elems) + -(-one.projections[0].d_out // one.page_elems)
    wl = workloads.random_small(seed, n_pages=int(one.ranks.sum()) * c * n_proj + 17, **kw)
    p = wl.projections[0]
    return dataclasses.replace(wl, projections=[dataclasses.replace(p, name=f"p{i}") for i in range(n_proj)])


SMALL = [
    # both families, segment ranks on both sides of 64 (the 3-per-CU wide template)
    ("both", dict(seed=301, dtype="f16", n_adapters=40, d_in=1024, d_out=2048, page_elems=512,
                  n_tokens=300, n_segments=4, rank_choices=(8, 16, 64, 128), p_none=0.05), 0),
    # decode groups only (MBGMV items of three projections in one launch)
    ("decode", dict(seed=302, dtype="bf16", n_adapters=60, d_in=2048, d_out=1024, page_elems=1024,
                    n_tokens=200, n_segments=0, rank_choices=(4, 16, 32), p_none=0.1), 1),
    # segments only, ragged geometry (d % P != 0)
    ("segments", dict(seed=303, dtype="bf16", n_adapters=8, d_in=1000, d_out=520, page_elems=64,
                      n_tokens=150, n_segments=5, rank_choices=(1, 3, 8, 40)), 2),
]


@pytest.mark.parametrize("name,kw,policy", SMALL, ids=[s[0] for s in SMALL])
def test_small_multi_bit_identical(rt, name, kw, policy):
    wl = _small_multi(kw["seed"], 3, **{k: v for k, v in kw.items() if k != "seed"})
    say(f"[gpu] apply_multi small {name}: 3 projections {wl.projections[0].d_in}x{wl.projections[0].d_out}")
    inst, ys = _multi_vs_single(rt, wl, policy=policy, exact=(name == "decode"))
    ref, _ = oracle_ref(wl, 2)
    margin_line(f"apply_multi small {name} proj 2 all rows", check_close(_bits(ys[2]), ref, wl.dtype, name))
    inst.close()


def test_multi_eight_projections(rt):
    """The most projections one call takes (8), both families."""
    wl = _small_multi(306, 8, dtype="bf16", n_adapters=30, d_in=768, d_out=1024, page_elems=256,
                      n_tokens=160, n_segments=3, rank_choices=(4, 16, 96), p_none=0.05)
    say("[gpu] apply_multi with 8 projections")
    inst, ys = _multi_vs_single(rt, wl)
    ref, _ = oracle_ref(wl, 7)
    margin_line("apply_multi 8 projections, proj 7 all rows", check_close(_bits(ys[7]), ref, wl.dtype, "p7"))
    inst.close()


def test_multi_single_projection(rt):
    wl = _small_multi(304, 1, dtype="f16", n_adapters=20, d_in=512, d_out=512, page_elems=256,
                      n_tokens=90, n_segments=2, rank_choices=(8, 16, 128))
    say("[gpu] apply_multi with one projection")
    inst, _ = _multi_vs_single(rt, wl)
    inst.close()


@pytest.mark.timeout(900)
def test_prefill_multi(rt):
    """The prefill batch's four projections in one launch (the step the benchmark times)."""
    wl = workloads.make("prefill_sgmv")
    say("[gpu] apply_multi prefill_sgmv q/k/v/o, building instance")
    inst, ys = _multi_vs_single(rt, wl)
    ev = sample_tokens(wl, 48)
    ref, _ = oracle_ref(wl, 3, ev)
    margin_line("apply_multi prefill_sgmv o sampled rows",
                check_close(_bits(ys[3])[ev], ref, wl.dtype, "prefill multi o"))
    inst.close()


@pytest.mark.timeout(900)
def test_mixed_multi(rt):
    """The mixed batch's four projections, both families, in one launch."""
    wl = workloads.make("mixed_13b")
    say("[gpu] apply_multi mixed_13b q/k/v/o, building instance")
    inst, ys = _multi_vs_single(rt, wl)
    ev = sample_tokens(wl, 48)
    ref, _ = oracle_ref(wl, 1, ev)
    margin_line("apply_multi mixed_13b k sampled rows",
                check_close(_bits(ys[1])[ev], ref, wl.dtype, "mixed multi k"))
    inst.close()


@pytest.mark.timeout(900)
def test_mlp_multi_rank_classes(rt):
    """gate and up (4096 -> 11008) together: enough tiles of both rank classes for a
    launch each, timed as one interval."""
    wl = workloads.make("mlp_asym")
    say("[gpu] apply_multi mlp_asym gate+up, building instance")
    inst, _ = _multi_vs_single(rt, wl, projs=[wl.proj("gate")[0], wl.proj("up")[0]])
    inst.close()


def test_multi_two_streams(rt):
    """slora_apply_multi calls on two workspaces and two streams, issued alternately with
    the host far ahead of the GPU: the library orders the launches across the streams,
    every output is the same bits as the per-projection reference and both workspaces
    report a clean status."""
    from heterogeneous_lora_amd import _lib
    wl = _small_multi(305, 4, dtype="f16", n_adapters=60, d_in=2048, d_out=2048, page_elems=1024,
                      n_tokens=400, n_segments=4, rank_choices=(8, 16, 64, 128), p_none=0.05)
    say("[gpu] apply_multi alternating over two streams, 4 projections")
    inst = rt.PagedLoRA(wl)
    calls = [inst.call(p) for p in range(4)]
    ins = [inst.inputs(p) for p in range(4)]
    single = []
    for c, (x, y0) in zip(calls, ins):
        y = y0.clone()
        inst.apply(c, x, y, inst.workspace(c))
        single.append(_bits(y))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [torch.zeros(_lib.workspace_size_multi(calls), dtype=torch.uint8, device=inst.device)
           for _ in range(2)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.cuda._sleep(20_000_000)  # bounded spin: the host runs ahead
    outs = []
    for i in range(8):
        k = i % 2
        with torch.cuda.stream(streams[k]):
            ys = [y0.clone() for _, y0 in ins]
            _lib.apply_multi(calls, [x.data_ptr() for x, _ in ins], [y.data_ptr() for y in ys],
                             wss[k].data_ptr(), wss[k].numel(), streams[k].cuda_stream)
        outs.append(ys)
    torch.cuda.synchronize()
    for k in range(2):
        assert _lib.workspace_status(wss[k].data_ptr(), streams[k].cuda_stream) == 0
    for i, ys in enumerate(outs):
        for p in range(4):
            _assert_same(_bits(ys[p]), single[p], wl.dtype, False, (i, p))
            assert np.array_equal(_bits(ys[p]), _bits(outs[0][p])), (i, p, "repeat")
    inst.close()
