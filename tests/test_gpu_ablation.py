"""The pages' ablation baselines through the HIP path, against the same oracle.

* slora_apply_gathered ("conventional batched matmul"): each request's adapter copied
  out of the pool into contiguous memory padded to the batch's largest rank, then one
  padded batched GEMM.
* adapters in a pool of their own, allocated in page order (each adapter contiguous),
  with no KV pages among them (S-LoRA without unified memory), computed by slora_apply.
"""

import numpy as np
import pytest

import workloads
from gpu_util import check_close, margin_line, oracle_ref, sample_tokens, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_lora_amd import _lib, runtime
    _lib.load()
    return runtime


def _gathered(rt, wl, proj=0, inst=None):
    inst = inst or rt.PagedLoRA(wl)
    call = inst.call(proj)
    x, y = inst.inputs(proj)
    ws = inst.gathered_workspace(call)
    inst.apply_gathered(call, x, y, ws)
    torch.cuda.synchronize()
    from heterogeneous_lora_amd import _lib
    assert _lib.workspace_status(ws.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    return y.cpu().numpy().view(np.uint16), inst


SMALL = [dict(seed=501), dict(seed=502, dtype="bf16"),
         dict(seed=503, d_in=1000, d_out=520, page_elems=64, n_tokens=70, n_segments=5,
              rank_choices=(0, 1, 3, 8, 16, 40)),
         dict(seed=504, dtype="bf16", d_in=520, d_out=1032, page_elems=512, n_tokens=41,
              n_segments=3, rank_choices=(8, 64, 128), n_adapters=4)]


@pytest.mark.parametrize("kw", SMALL, ids=[f"s{k['seed']}" for k in SMALL])
def test_gathered_small(rt, kw):
    wl = workloads.random_small(**kw)
    say(f"[gpu] gathered baseline {kw}")
    y, inst = _gathered(rt, wl)
    ref, _ = oracle_ref(wl, 0)
    margin_line(f"gathered s{kw['seed']}", check_close(y, ref, wl.dtype, f"gathered {kw}"))
    ids = np.concatenate([np.repeat(wl.seg_adapter, np.diff(wl.seg_offsets)), wl.token_adapter])
    idle = (ids < 0) | (wl.ranks[np.maximum(ids, 0)] == 0)
    assert np.array_equal(y[idle], wl.y0(0)[idle])
    inst.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode_7b", "mixed_13b"])
def test_gathered_large(rt, name):
    wl = workloads.make(name)
    say(f"[gpu] gathered baseline {name}")
    inst = rt.PagedLoRA(wl)
    y, _ = _gathered(rt, wl, inst=inst)
    ev = np.arange(wl.n_tokens) if wl.n_tokens <= 512 else sample_tokens(wl, 64)
    ref, _ = oracle_ref(wl, 0, ev, n_threads=16)
    margin_line(f"gathered {name} proj=q {ev.size} rows", check_close(y[ev], ref, wl.dtype, name))
    inst.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["decode_7b", "mixed_13b"])
def test_split_pool_contiguous_adapters(rt, name):
    """Adapters in an ordered pool of their own: every adapter's page-table entries are
    consecutive pages, and slora_apply gives the same bits as on the unified pool."""
    wl = workloads.make(name)
    say(f"[gpu] adapters in a pool of their own, {name}")
    split = rt.PagedLoRA(wl, ordered=True)
    pt = split.pt_dev[0].cpu().numpy()
    for a in split.adapters:
        b = int(split.base[0][a])
        p0 = wl.projections[0]
        n = int(wl.ranks[a]) * (-(-p0.d_in // wl.page_elems) + -(-p0.d_out // wl.page_elems))
        seg = pt[b:b + n]
        assert np.array_equal(seg, np.arange(seg[0], seg[0] + n)), a
    call = split.call(0)
    x, y = split.inputs(0)
    ws = split.workspace(call)
    split.apply(call, x, y, ws)
    torch.cuda.synchronize()
    ys = y.cpu().numpy().view(np.uint16)
    ev = np.arange(wl.n_tokens) if wl.n_tokens <= 512 else sample_tokens(wl, 64)
    ref, _ = oracle_ref(wl, 0, ev, n_threads=16)
    margin_line(f"split pool {name} proj=q {ev.size} rows", check_close(ys[ev], ref, wl.dtype, name))
    split.close()
    uni = rt.PagedLoRA(wl)
    call = uni.call(0)
    x, y = uni.inputs(0)
    ws = uni.workspace(call)
    uni.apply(call, x, y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(ys, y.cpu().numpy().view(np.uint16))  # placement never changes a bit
    uni.close()
