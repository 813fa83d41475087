"""slora_apply_noalloc (the allocation-free variant of slora_apply, whose workspace is
a static device array of the library) against slora_apply, through the C ABI.

Two calls in a row on one device, the second smaller than the first, so the second
runs on scratch that still holds the first call's words: once through the fused
decode launch (the 7B decode batch, then a third of its tokens) and once through
both kernel families (a batch of prefill segments and decode ids, then a smaller
one). Every output must equal slora_apply's bit for bit, and the scratch's give-up
status must read clean.
"""

import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import check_close, oracle_ref, say

torch = pytest.importorskip("torch")


def _sub(wl, keep):
    """The same workload restricted to per-token ids `keep` (no segments)."""
    return dataclasses.replace(wl, token_adapter=wl.token_adapter[keep].copy(), _cache={})


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call whose workspace would exceed the static array is refused before anything
    reaches a device (so this runs without a GPU)."""
    from heterogeneous_lora_amd import _lib
    wl = workloads.decode7b(0)
    n = 200_000  # 200,000 tokens x r_max 64 x 8 bytes of tagged v alone > 64 MiB
    call = _lib.Call(pool_ptr=0x7F0000000000, n_pages=wl.n_pages, page_elems=wl.page_elems,
                     dtype=wl.dtype, d_in=4096, d_out=4096, page_table_ptr=0x7F0000000000,
                     page_table_len=1, base=np.full(wl.n_adapters, -1, np.int64), rank=wl.ranks,
                     scale=wl.scales.astype(np.float32), r_max=64, n_tokens=n,
                     seg_offsets=np.zeros(1, np.int32), seg_adapter=np.zeros(0, np.int32),
                     token_adapter=np.full(n, -1, np.int32))
    with pytest.raises(_lib.SloraError) as e:
        _lib.apply_noalloc(call, 0x7F0000000000, 0x7F0000000000, 0)
    assert e.value.code == _lib.E_INVALID and "static scratch" in str(e.value)


def _pair(rt, inst, wl, x_np, y0_np, policy, what):
    """slora_apply and slora_apply_noalloc on the same inputs: (apply bits, noalloc bits)."""
    from heterogeneous_lora_amd import _lib
    call = inst.call(0, policy, wl=wl)
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).cuda()
    y_a = torch.from_numpy(np.ascontiguousarray(y0_np).view(np.int16)).cuda()
    y_n = y_a.clone()
    ws = inst.workspace(call)
    stream = torch.cuda.current_stream().cuda_stream
    say(f"[gpu] noalloc {what}: slora_apply, then slora_apply_noalloc ({wl.n_tokens} tokens)")
    _lib.apply(call, x.data_ptr(), y_a.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    _lib.apply_noalloc(call, x.data_ptr(), y_n.data_ptr(), stream)
    torch.cuda.synchronize()
    assert _lib.workspace_status(ws.data_ptr(), stream) == 0
    assert _lib.workspace_status(None, stream) == 0
    return y_a.cpu().numpy().view(np.uint16), y_n.cpu().numpy().view(np.uint16)


@pytest.mark.gpu
def test_noalloc_matches_apply_decode(rt_noalloc):
    rt = rt_noalloc
    wl = workloads.decode7b(0)
    inst = rt.PagedLoRA(wl)
    x, y0 = wl.x(0), wl.y0(0)
    ya, yn = _pair(rt, inst, wl, x, y0, 0, "decode_7b, 256 tokens")
    assert np.array_equal(ya, yn)
    ref, _ = oracle_ref(wl, 0)
    check_close(yn, ref, wl.dtype, "noalloc decode_7b")
    keep = np.arange(0, wl.n_tokens, 3)
    sub = _sub(wl, keep)
    ya, yn = _pair(rt, inst, sub, x[keep], y0[keep], 0, "decode_7b, every third token")
    assert np.array_equal(ya, yn)
    ref, _ = oracle_ref(sub, 0, x=x[keep], y0=y0[keep])
    check_close(yn, ref, wl.dtype, "noalloc decode_7b subset")
    inst.close()


@pytest.mark.gpu
def test_noalloc_matches_apply_mixed(rt_noalloc):
    rt = rt_noalloc
    big = workloads.random_small(211, d_in=1024, d_out=1536, page_elems=512, n_tokens=150,
                                 n_segments=4, rank_choices=(8, 16, 32, 100), n_pages=8192)
    small = workloads.random_small(212, d_in=1024, d_out=1536, page_elems=512, n_tokens=41,
                                   n_segments=2, rank_choices=(4, 16, 64), n_pages=4096)
    for wl, what in ((big, "mixed batch, 150 tokens"), (small, "mixed batch, 41 tokens")):
        inst = rt.PagedLoRA(wl)
        for policy in (0, 2):
            ya, yn = _pair(rt, inst, wl, wl.x(0), wl.y0(0), policy, f"{what}, policy {policy}")
            assert np.array_equal(ya, yn), (what, policy)
            ref, _ = oracle_ref(wl, 0)
            check_close(yn, ref, wl.dtype, f"noalloc {what}")
        inst.close()


@pytest.fixture(scope="module")
def rt_noalloc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_lora_amd import _lib, runtime
    _lib.load()
    return runtime
