"""ctypes binding of libslora.so: argument marshalling only.

Every function here has the name of the C entry point it calls (without the
`slora_` prefix) and does nothing but convert arguments and raise SloraError on a
negative return code. All work runs in the library's HIP kernels and host code;
there is no fallback of any kind: if libslora.so is missing the import fails.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libslora.so")

OK, E_INVALID, E_POOL_FULL, E_STATE, E_HIP = 0, -1, -2, -3, -4
F16, BF16 = 0, 1
POLICY_AUTO, POLICY_MBGMV, POLICY_SGMV = 0, 1, 2
DTYPES = {"f16": F16, "bf16": BF16}

_c_i32, _c_i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class SloraError(RuntimeError):
    def __init__(self, code: int, what: str, msg: str):
        super().__init__(f"{what} failed ({code}): {msg}")
        self.code = code


class Lora(ctypes.Structure):
    _fields_ = [("pool", _vp), ("n_pages", _c_i64), ("page_elems", _c_i32), ("dtype", _c_i32),
                ("d_in", _c_i32), ("d_out", _c_i32), ("page_table", _vp),
                ("page_table_len", _c_i64), ("n_adapters", _c_i32), ("base", _vp), ("rank", _vp),
                ("scale", _vp), ("r_max", _c_i32)]


class Routing(ctypes.Structure):
    _fields_ = [("n_tokens", _c_i32), ("n_segments", _c_i32), ("seg_offsets", _vp),
                ("seg_adapter", _vp), ("token_adapter", _vp), ("policy", _c_i32)]


class ResidencyStats(ctypes.Structure):
    _fields_ = [("resident", _c_i32), ("pinned", _c_i32), ("hits", _c_i64), ("misses", _c_i64),
                ("evictions", _c_i64), ("prefetches", _c_i64)]


class SchedConfig(ctypes.Structure):
    _fields_ = [("kv_pages_per_token", _c_i32), ("max_batch_tokens", _c_i32),
                ("max_running", _c_i32)]


class SchedBatch(ctypes.Structure):
    _fields_ = [("step", _c_i64), ("n_tokens", _c_i32), ("n_segments", _c_i32),
                ("seg_offsets", _vp), ("seg_adapter", _vp), ("token_adapter", _vp),
                ("seg_request", _vp), ("token_request", _vp),
                ("n_fetch", _c_i32), ("fetch", _vp), ("n_evicted", _c_i32), ("evicted", _vp),
                ("n_finished", _c_i32), ("finished", _vp), ("n_aborted", _c_i32), ("aborted", _vp),
                ("abort_reason", _vp), ("n_waiting", _c_i32), ("n_running", _c_i32),
                ("free_pages", _c_i64)]


ABORT_DEADLINE, ABORT_POOL_FULL = 1, 2

_lib = None


def load(path: str = LIB_PATH):
    """Load libslora.so. Raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with heterogeneous_lora_amd/build.py")
    # The library and torch must share one HIP runtime. torch ships its own copy of
    # libamdhip64; loading torch first makes the library bind to that copy (same soname)
    # instead of pulling a second runtime into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P, I = _vp, _c_i32
    sig = {
        "slora_last_error": ([], ctypes.c_char_p),
        "slora_abi_version": ([], I),
        "slora_pool_create": ([P, _c_i64, I, I, ctypes.c_uint64, P], I),
        "slora_pool_destroy": ([P], I),
        "slora_pool_info": ([P, P, P, P, P], I),
        "slora_pool_alloc_kv": ([P, I, P], I),
        "slora_pool_free_kv": ([P, P, I], I),
        "slora_pool_free": ([P, P, I], I),
        "slora_pool_n_free": ([P, P], I),
        "slora_pool_alloc_adapter": ([P, I, I, I, P, P], I),
        "slora_pool_free_adapter": ([P, I], I),
        "slora_pool_page_table": ([P, I, I, P, _c_i64, P, P, P], I),
        "slora_pool_owners": ([P, P], I),
        "slora_fetch_async": ([P, I, P, P, P, P], I),
        "slora_fetch_many_async": ([P, I, P, P, P, P, P], I),
        "slora_workspace_size": ([P, P, P], I),
        "slora_shrink": ([P, P, P, P, P, _c_i64, P], I),
        "slora_expand": ([P, P, P, P, P, _c_i64, P], I),
        "slora_apply": ([P, P, P, P, P, _c_i64, P], I),
        "slora_apply_noalloc": ([P, P, P, P, P], I),
        "slora_workspace_size_multi": ([I, P, P, P], I),
        "slora_apply_multi": ([I, P, P, P, P, P, _c_i64, P], I),
        "slora_gathered_workspace_size": ([P, P, P], I),
        "slora_apply_gathered": ([P, P, P, P, P, _c_i64, P], I),
        "slora_pool_create_ordered": ([P, _c_i64, I, I, P], I),
        "slora_plan_inspect": ([P, P, P, P, I, P], I),
        "slora_timing_enable": ([I], I),
        "slora_workspace_status": ([P, P, P], I),
        "slora_timing_read": ([I, P, P], I),
        "slora_timing_read_all": ([_c_i64, P, P, P], I),
        "slora_set_wait_limit": ([I], I),
        "slora_residency_create": ([P, I, P, P, P], I),
        "slora_residency_destroy": ([P], I),
        "slora_residency_acquire": ([P, I, I, P, P, I, P], I),
        "slora_residency_prefetch": ([P, I, I, P], I),
        "slora_residency_release": ([P, I], I),
        "slora_residency_info": ([P, P], I),
        "slora_residency_is_resident": ([P, I, P], I),
        "slora_sched_create": ([P, P, P, P], I),
        "slora_sched_destroy": ([P], I),
        "slora_sched_submit": ([P, _c_i64, I, I, I, I, _c_i64], I),
        "slora_sched_finish": ([P, _c_i64], I),
        "slora_sched_step": ([P, P], I),
        "slora_sched_request_pages": ([P, _c_i64, P, I, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != OK:
        raise SloraError(rc, what, load().slora_last_error().decode())


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def last_error() -> str:
    return load().slora_last_error().decode()


def abi_version() -> int:
    return load().slora_abi_version()


class Pool:
    """Owner of one slora_pool handle over caller-owned device memory."""

    def __init__(self, dev_ptr: int, n_pages: int, page_elems: int, dtype: str, seed: int,
                 ordered: bool = False):
        self._lib = load()
        h = ctypes.c_void_p()
        if ordered:  # pages handed out in ascending order (no shuffle)
            _check(self._lib.slora_pool_create_ordered(ctypes.c_void_p(dev_ptr), n_pages, page_elems,
                                                       DTYPES[dtype], ctypes.byref(h)), "pool_create_ordered")
        else:
            _check(self._lib.slora_pool_create(ctypes.c_void_p(dev_ptr), n_pages, page_elems,
                                               DTYPES[dtype], seed, ctypes.byref(h)), "pool_create")
        self.handle = h
        self.n_pages, self.page_elems, self.dtype = n_pages, page_elems, dtype

    def destroy(self):
        if self.handle:
            _check(self._lib.slora_pool_destroy(self.handle), "pool_destroy")
            self.handle = None

    def info(self):
        n, f, pe, dt = _c_i64(), _c_i64(), _c_i32(), _c_i32()
        _check(self._lib.slora_pool_info(self.handle, ctypes.byref(n), ctypes.byref(f),
                                         ctypes.byref(pe), ctypes.byref(dt)), "pool_info")
        return dict(n_pages=n.value, n_free=f.value, page_elems=pe.value, dtype=dt.value)

    def alloc_kv(self, n: int) -> np.ndarray:
        out = np.empty(n, np.int32)
        _check(self._lib.slora_pool_alloc_kv(self.handle, n, _p(out)), "pool_alloc_kv")
        return out

    def free_kv(self, ids: np.ndarray):
        ids = np.ascontiguousarray(ids, np.int32)
        _check(self._lib.slora_pool_free_kv(self.handle, _p(ids), ids.size), "pool_free_kv")

    def free(self, ids: np.ndarray):
        ids = np.ascontiguousarray(ids, np.int32)
        _check(self._lib.slora_pool_free(self.handle, _p(ids), ids.size), "pool_free")

    def n_free(self) -> int:
        n = _c_i64()
        _check(self._lib.slora_pool_n_free(self.handle, ctypes.byref(n)), "pool_n_free")
        return n.value

    def alloc_adapter(self, adapter_id: int, rank: int, d_in: Sequence[int], d_out: Sequence[int]):
        di = np.ascontiguousarray(d_in, np.int32)
        do = np.ascontiguousarray(d_out, np.int32)
        _check(self._lib.slora_pool_alloc_adapter(self.handle, adapter_id, rank, di.size, _p(di),
                                                  _p(do)), "pool_alloc_adapter")

    def free_adapter(self, adapter_id: int):
        _check(self._lib.slora_pool_free_adapter(self.handle, adapter_id), "pool_free_adapter")

    def page_table(self, proj: int, n_adapters: int):
        n = _c_i64()
        base = np.empty(max(n_adapters, 1), np.int64)
        rank = np.empty(max(n_adapters, 1), np.int32)
        _check(self._lib.slora_pool_page_table(self.handle, proj, n_adapters, None, 0,
                                               ctypes.byref(n), _p(base), _p(rank)), "page_table")
        pt = np.empty(max(n.value, 1), np.int32)
        _check(self._lib.slora_pool_page_table(self.handle, proj, n_adapters, _p(pt), pt.size,
                                               ctypes.byref(n), _p(base), _p(rank)), "page_table")
        return pt[:n.value], base[:n_adapters], rank[:n_adapters]

    def owners(self) -> np.ndarray:
        out = np.empty(self.n_pages, np.int32)
        _check(self._lib.slora_pool_owners(self.handle, _p(out)), "pool_owners")
        return out

    def fetch_async(self, adapter_id: int, host_at: Sequence[int], host_b: Sequence[int],
                    stream: int, event: Optional[int]):
        at = (ctypes.c_void_p * max(len(host_at), 1))(*host_at)
        b = (ctypes.c_void_p * max(len(host_b), 1))(*host_b)
        _check(self._lib.slora_fetch_async(self.handle, adapter_id, at, b, ctypes.c_void_p(stream),
                                           ctypes.c_void_p(event) if event else None),
               "fetch_async")

    def fetch_many_async(self, adapter_ids: Sequence[int], host_at: Sequence[Sequence[int]],
                         host_b: Sequence[Sequence[int]], stream: int, event: Optional[int]):
        """fetch_async for several adapters in one launch; host_at[i] / host_b[i] are
        adapter_ids[i]'s per-projection row pointers."""
        n = len(adapter_ids)
        if len(host_at) != n or len(host_b) != n:
            raise ValueError("fetch_many_async: one pointer list per adapter")
        ids = np.ascontiguousarray(adapter_ids, dtype=np.int32)

        def table(lists):
            # the per-adapter pointer arrays as rows of one uint64 block, and an array of
            # the rows' addresses (both kept alive by the caller's references)
            width = max([len(x) for x in lists] + [1])
            block = np.zeros((max(n, 1), width), np.uint64)
            for i, x in enumerate(lists):
                block[i, :len(x)] = x
            rows = block.ctypes.data + np.arange(max(n, 1), dtype=np.uint64) * np.uint64(width * 8)
            return block, np.ascontiguousarray(rows, dtype=np.uint64)

        blk_at, at = table(host_at)
        blk_b, b = table(host_b)
        _check(self._lib.slora_fetch_many_async(self.handle, n, _p(ids), _p(at), _p(b),
                                                ctypes.c_void_p(stream),
                                                ctypes.c_void_p(event) if event else None),
               "fetch_many_async")


class Residency:
    """slora_residency: LRU residency of the adapters of one pool (host bookkeeping)."""

    def __init__(self, pool: Pool, d_in: Sequence[int], d_out: Sequence[int]):
        self._lib = load()
        self.pool = pool
        di = np.ascontiguousarray(d_in, np.int32)
        do = np.ascontiguousarray(d_out, np.int32)
        h = ctypes.c_void_p()
        _check(self._lib.slora_residency_create(pool.handle, di.size, _p(di), _p(do), ctypes.byref(h)),
               "residency_create")
        self.handle = h

    def destroy(self):
        if self.handle:
            _check(self._lib.slora_residency_destroy(self.handle), "residency_destroy")
            self.handle = None

    def acquire(self, adapter_id: int, rank: int):
        """(needs_fetch, [evicted ids])."""
        nf, ne = _c_i32(), _c_i32()
        ev = np.zeros(4096, np.int32)
        _check(self._lib.slora_residency_acquire(self.handle, adapter_id, rank, ctypes.byref(nf), _p(ev),
                                                 ev.size, ctypes.byref(ne)), "residency_acquire")
        return bool(nf.value), [int(v) for v in ev[:ne.value]]

    def prefetch(self, adapter_id: int, rank: int) -> bool:
        nf = _c_i32()
        _check(self._lib.slora_residency_prefetch(self.handle, adapter_id, rank, ctypes.byref(nf)),
               "residency_prefetch")
        return bool(nf.value)

    def release(self, adapter_id: int):
        _check(self._lib.slora_residency_release(self.handle, adapter_id), "residency_release")

    def info(self) -> dict:
        st = ResidencyStats()
        _check(self._lib.slora_residency_info(self.handle, ctypes.byref(st)), "residency_info")
        return {f: getattr(st, f) for f, _ in ResidencyStats._fields_}

    def pins(self, adapter_id: int) -> int:
        """Pin count, -1 if not resident."""
        v = _c_i32()
        _check(self._lib.slora_residency_is_resident(self.handle, adapter_id, ctypes.byref(v)),
               "residency_is_resident")
        return v.value


def _arr(ptr, n, dtype):
    if n <= 0 or not ptr:
        return np.zeros(0, dtype)
    ct = ctypes.c_int64 if dtype == np.int64 else ctypes.c_int32
    return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ct)), shape=(n,)).copy()


class Scheduler:
    """slora_sched: FIFO continuous-batching admission over the unified pool."""

    def __init__(self, pool: Pool, residency: Optional[Residency], kv_pages_per_token: int,
                 max_batch_tokens: int, max_running: int):
        self._lib = load()
        self.pool, self.residency = pool, residency
        cfg = SchedConfig(kv_pages_per_token, max_batch_tokens, max_running)
        h = ctypes.c_void_p()
        _check(self._lib.slora_sched_create(pool.handle, residency.handle if residency else None,
                                            ctypes.byref(cfg), ctypes.byref(h)), "sched_create")
        self.handle = h

    def destroy(self):
        if self.handle:
            _check(self._lib.slora_sched_destroy(self.handle), "sched_destroy")
            self.handle = None

    def submit(self, request_id: int, adapter_id: int, rank: int, prompt_len: int,
               max_new_tokens: int, deadline_step: int = -1):
        _check(self._lib.slora_sched_submit(self.handle, request_id, adapter_id, rank, prompt_len,
                                            max_new_tokens, deadline_step), "sched_submit")

    def finish(self, request_id: int):
        _check(self._lib.slora_sched_finish(self.handle, request_id), "sched_finish")

    def step(self) -> dict:
        b = SchedBatch()
        _check(self._lib.slora_sched_step(self.handle, ctypes.byref(b)), "sched_step")
        S = b.n_segments
        so = _arr(b.seg_offsets, S + 1, np.int32)
        n_dec = b.n_tokens - int(so[-1])
        return dict(step=b.step, n_tokens=b.n_tokens, seg_offsets=so,
                    seg_adapter=_arr(b.seg_adapter, S, np.int32),
                    token_adapter=_arr(b.token_adapter, n_dec, np.int32),
                    seg_request=_arr(b.seg_request, S, np.int64),
                    token_request=_arr(b.token_request, n_dec, np.int64),
                    fetch=_arr(b.fetch, b.n_fetch, np.int32), evicted=_arr(b.evicted, b.n_evicted, np.int32),
                    finished=_arr(b.finished, b.n_finished, np.int64),
                    aborted=_arr(b.aborted, b.n_aborted, np.int64),
                    abort_reason=_arr(b.abort_reason, b.n_aborted, np.int32),
                    n_waiting=b.n_waiting, n_running=b.n_running, free_pages=b.free_pages)

    def request_pages(self, request_id: int) -> np.ndarray:
        n = _c_i32()
        buf = np.zeros(1 << 20, np.int32)
        _check(self._lib.slora_sched_request_pages(self.handle, request_id, _p(buf), buf.size,
                                                   ctypes.byref(n)), "sched_request_pages")
        return buf[:n.value].copy()


class Call:
    """Host-side arguments of one compute call (keeps the host arrays alive)."""

    def __init__(self, *, pool_ptr: int, n_pages: int, page_elems: int, dtype: str, d_in: int,
                 d_out: int, page_table_ptr: int, page_table_len: int, base: np.ndarray,
                 rank: np.ndarray, scale: np.ndarray, r_max: int, n_tokens: int,
                 seg_offsets: np.ndarray, seg_adapter: np.ndarray, token_adapter: np.ndarray,
                 policy: int = POLICY_AUTO):
        self.base = np.ascontiguousarray(base, np.int64)
        self.rank = np.ascontiguousarray(rank, np.int32)
        self.scale = np.ascontiguousarray(scale, np.float32)
        self.seg_offsets = np.ascontiguousarray(seg_offsets, np.int32)
        self.seg_adapter = np.ascontiguousarray(seg_adapter, np.int32)
        self.token_adapter = np.ascontiguousarray(token_adapter, np.int32)
        self.lora = Lora(pool=pool_ptr, n_pages=n_pages, page_elems=page_elems,
                         dtype=DTYPES[dtype], d_in=d_in, d_out=d_out, page_table=page_table_ptr,
                         page_table_len=page_table_len, n_adapters=self.rank.size,
                         base=self.base.ctypes.data, rank=self.rank.ctypes.data,
                         scale=self.scale.ctypes.data, r_max=r_max)
        self.routing = Routing(n_tokens=n_tokens, n_segments=self.seg_adapter.size,
                               seg_offsets=self.seg_offsets.ctypes.data,
                               seg_adapter=self.seg_adapter.ctypes.data,
                               token_adapter=self.token_adapter.ctypes.data, policy=policy)

    def set_policy(self, policy: int):
        self.routing.policy = policy


def workspace_size(call: Call) -> int:
    n = _c_i64()
    _check(load().slora_workspace_size(ctypes.byref(call.lora), ctypes.byref(call.routing),
                                       ctypes.byref(n)), "workspace_size")
    return n.value


def shrink(call: Call, x: int, v: int, ws: int, ws_bytes: int, stream: int):
    _check(load().slora_shrink(ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(x), _vp(v),
                               _vp(ws), ws_bytes, _vp(stream)), "shrink")


def expand(call: Call, v: int, y: int, ws: int, ws_bytes: int, stream: int):
    _check(load().slora_expand(ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(v), _vp(y),
                               _vp(ws), ws_bytes, _vp(stream)), "expand")


def apply(call: Call, x: int, y: int, ws: int, ws_bytes: int, stream: int):
    _check(load().slora_apply(ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(x), _vp(y),
                              _vp(ws), ws_bytes, _vp(stream)), "apply")


def gathered_workspace_size(call: Call) -> int:
    n = _c_i64()
    _check(load().slora_gathered_workspace_size(ctypes.byref(call.lora), ctypes.byref(call.routing),
                                                ctypes.byref(n)), "gathered_workspace_size")
    return n.value


def apply_gathered(call: Call, x: int, y: int, ws: int, ws_bytes: int, stream: int):
    _check(load().slora_apply_gathered(ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(x),
                                       _vp(y), _vp(ws), ws_bytes, _vp(stream)), "apply_gathered")


def apply_noalloc(call: Call, x: int, y: int, stream: int):
    _check(load().slora_apply_noalloc(ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(x),
                                      _vp(y), _vp(stream)), "apply_noalloc")


class MultiCall:
    """Host-side arguments of one slora_apply_multi: the projections' Call objects (their
    lora structs side by side, the routing of the first) and the x / y pointers."""

    def __init__(self, calls: Sequence[Call], xs: Sequence[int], ys: Sequence[int]):
        self.calls = list(calls)
        self.n = len(self.calls)
        self.loras = (Lora * max(self.n, 1))(*[c.lora for c in self.calls])
        self.xs = (_vp * max(self.n, 1))(*xs)
        self.ys = (_vp * max(self.n, 1))(*ys)


def workspace_size_multi(calls: Sequence[Call]) -> int:
    m = MultiCall(calls, [0] * len(calls), [0] * len(calls))
    n = _c_i64()
    _check(load().slora_workspace_size_multi(m.n, m.loras, ctypes.byref(calls[0].routing),
                                             ctypes.byref(n)), "workspace_size_multi")
    return n.value


def apply_multi(calls: Sequence[Call], xs: Sequence[int], ys: Sequence[int], ws: int, ws_bytes: int,
                stream: int):
    m = MultiCall(calls, xs, ys)
    _check(load().slora_apply_multi(m.n, m.loras, ctypes.byref(m.calls[0].routing), m.xs, m.ys,
                                    _vp(ws), ws_bytes, _vp(stream)), "apply_multi")


def bind_apply_multi(calls: Sequence[Call], xs: Sequence[int], ys: Sequence[int], ws: int,
                     ws_bytes: int, stream: int):
    """slora_apply_multi with its arguments converted once (see bind_apply)."""
    m = MultiCall(calls, xs, ys)
    f = load().slora_apply_multi
    args = (m.n, m.loras, ctypes.byref(m.calls[0].routing), m.xs, m.ys, _vp(ws), _c_i64(ws_bytes),
            _vp(stream))

    def run():
        rc = f(*args)
        if rc != OK:
            _check(rc, "apply_multi")

    run.call = m
    return run


def bind_apply(call: Call, x: int, y: int, ws: int, ws_bytes: int, stream: int,
               gathered: bool = False):
    """slora_apply (or slora_apply_gathered) with its arguments converted once: returns a
    no-argument callable for callers that repeat the same call (same buffers, new
    contents) many times."""
    f = load().slora_apply_gathered if gathered else load().slora_apply
    args = (ctypes.byref(call.lora), ctypes.byref(call.routing), _vp(x), _vp(y), _vp(ws),
            _c_i64(ws_bytes), _vp(stream))

    def run():
        rc = f(*args)
        if rc != OK:
            _check(rc, "apply")

    run.call = call  # the argument structs must outlive the callable
    return run


KERNELS = ["mbgmv_shrink", "mbgmv_expand", "sgmv_shrink", "sgmv_expand", "mbgmv_fused", "gather",
           "fetch", "sgmv_fused", "mixed_fused", "multi_fused"]


def timing_enable(on: bool):
    _check(load().slora_timing_enable(1 if on else 0), "timing_enable")


def timing_read():
    """{kernel name: (launches, total ms)} since timing_enable; clears the counters."""
    n = len(KERNELS)
    launches = np.zeros(n, np.int64)
    ms = np.zeros(n, np.float64)
    _check(load().slora_timing_read(n, _p(launches), _p(ms)), "timing_read")
    return {k: (int(launches[i]), float(ms[i])) for i, k in enumerate(KERNELS)}


def timing_read_all(cap: int = 1 << 16):
    """Every timed launch since the last read: (kernel names [n], durations in ms [n]);
    clears them."""
    kernel = np.zeros(cap, np.int32)
    ms = np.zeros(cap, np.float64)
    n = _c_i64()
    _check(load().slora_timing_read_all(cap, _p(kernel), _p(ms), ctypes.byref(n)), "timing_read_all")
    return [KERNELS[k] for k in kernel[:n.value]], ms[:n.value].copy()


def set_wait_limit(polls: int):
    """Bound of the decode launches' wait for v, in polls (0 = the default, 2^20)."""
    _check(load().slora_set_wait_limit(polls), "set_wait_limit")


def workspace_status(ws: Optional[int], stream: int) -> int:
    """0 if every fused call on this workspace since the last status read ran clean;
    1 if a wait gave up in one of them. Synchronizes the stream; clears the flag.
    ws None: the current device's static scratch of apply_noalloc."""
    st = _c_i32()
    _check(load().slora_workspace_status(_vp(ws), _vp(stream), ctypes.byref(st)), "workspace_status")
    return st.value


def plan_inspect(call: Call):
    """(groups [n x 5] int32: family, first slot, count, pt_base, rank; tokens int32)."""
    lib = load()
    n = _c_i32()
    cap = max(call.routing.n_tokens, 1)
    info = np.empty(5 * cap, np.int32)
    toks = np.empty(cap, np.int32)
    _check(lib.slora_plan_inspect(ctypes.byref(call.lora), ctypes.byref(call.routing),
                                  ctypes.byref(n), _p(info), cap, _p(toks)), "plan_inspect")
    g = info[:5 * n.value].reshape(n.value, 5)
    used = int(g[:, 2].sum()) if n.value else 0
    return g, toks[:used]
