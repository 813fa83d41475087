"""Device-memory and stream plumbing around libslora for one workload instance.

PyTorch only allocates device and pinned host memory and provides streams and
events; every step of the LoRA path (allocation bookkeeping, fetch, planning,
shrink, expand) runs in libslora. Used by the tests, the smoke check and the
benchmark.
"""

from __future__ import annotations

from dataclasses import replace as dataclass_replace
from typing import Dict, List, Optional

import numpy as np
import torch

from . import _lib

SENTINEL_I16 = {"f16": 0x7E00, "bf16": 0x7FC0}  # quiet NaN bit patterns (both < 2^15)


def _dev_i16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device, non_blocking=False)


class HostStore:
    """Adapter weights of one projection set in one pinned host buffer (16-byte aligned rows)."""

    def __init__(self, wl, adapters):
        self.offsets: Dict[tuple, int] = {}
        total = 0
        for a in adapters:
            r = int(wl.ranks[a])
            for p, pr in enumerate(wl.projections):
                for half, L in ((0, pr.d_in), (1, pr.d_out)):
                    self.offsets[(a, p, half)] = total
                    total += ((r * L * 2 + 255) // 256) * 256
        self.buf = torch.empty(max(total, 256), dtype=torch.uint8, pin_memory=True)
        host = self.buf.numpy()
        for a in adapters:
            for p in range(len(wl.projections)):
                at, b = wl.adapter(int(a), p)
                for half, arr in ((0, at), (1, b)):
                    o = self.offsets[(a, p, half)]
                    raw = np.ascontiguousarray(arr).view(np.uint8).ravel()
                    host[o:o + raw.size] = raw
        self.base_ptr = self.buf.data_ptr()

    def ptrs(self, a, n_proj):
        return ([self.base_ptr + self.offsets[(a, p, 0)] for p in range(n_proj)],
                [self.base_ptr + self.offsets[(a, p, 1)] for p in range(n_proj)])


class PagedLoRA:
    """One workload on one GPU: pool, resident adapters, page tables, inputs, workspace."""

    def __init__(self, wl, device: str = "cuda", adapters: Optional[List[int]] = None,
                 fill_kv: bool = True, sentinel: bool = True, pool_seed: Optional[int] = None,
                 store: Optional[HostStore] = None, ordered: bool = False,
                 n_pages: Optional[int] = None):
        """ordered: a pool of its own for the adapters, pages handed out in order (each
        adapter contiguous), no KV pages in it (the split-memory ablation); n_pages then
        defaults to the adapters' pages plus the workload's spare."""
        self.wl = wl
        self.device = torch.device(device)
        P = wl.page_elems
        self.adapters = [int(a) for a in (wl.active_adapters() if adapters is None else adapters)]
        if ordered:
            fill_kv = False
            if n_pages is None:
                n_pages = sum(wl.adapter_pages(a) for a in self.adapters) + 64
        self.n_pages = wl.n_pages if n_pages is None else n_pages
        self.pool_t = torch.empty(self.n_pages * P, dtype=torch.int16, device=self.device)
        if sentinel:
            self.pool_t.fill_(SENTINEL_I16[wl.dtype])
        self.pool = _lib.Pool(self.pool_t.data_ptr(), self.n_pages, P, wl.dtype,
                              wl.pool_seed if pool_seed is None else pool_seed, ordered=ordered)
        d_in = [p.d_in for p in wl.projections]
        d_out = [p.d_out for p in wl.projections]
        for a in self.adapters:
            self.pool.alloc_adapter(a, int(wl.ranks[a]), d_in, d_out)
        self.kv_pages = np.zeros(0, np.int32)
        if fill_kv:
            self._fill_kv()
        self.store = store if store is not None else HostStore(wl, self.adapters)
        self.fetch_ms = self.fetch()
        self.pt_dev, self.pt_len, self.base, self.rank = [], [], [], []
        for p in range(len(wl.projections)):
            pt, base, rank = self.pool.page_table(p, wl.n_adapters)
            self.pt_len.append(int(pt.size))
            self.pt_dev.append(torch.from_numpy(np.ascontiguousarray(pt)).to(self.device)
                               if pt.size else torch.zeros(1, dtype=torch.int32, device=self.device))
            self.base.append(base)
            self.rank.append(rank)
        self.r_max = int(max([int(wl.ranks[a]) for a in self.adapters] + [0]))
        self.r_max = max(self.r_max, 1)

    def _fill_kv(self):
        free = self.pool.info()["n_free"]
        lens = self.wl.kv_seq_lens
        got = []
        if lens.size:
            for L in lens:  # one K and one V page per token, until the pool is full
                n = int(min(2 * int(L), free))
                if n <= 0:
                    break
                got.append(self.pool.alloc_kv(n))
                free -= n
        elif free > 0:
            got.append(self.pool.alloc_kv(free))
        self.kv_pages = np.concatenate(got) if got else np.zeros(0, np.int32)

    def fetch(self, adapters: Optional[List[int]] = None) -> float:
        """Fetch adapters on a side stream; the current stream waits for the done event.
        Returns the fetch time in ms (events on the side stream; waits for it)."""
        side = torch.cuda.Stream(device=self.device)
        done = torch.cuda.Event(enable_timing=True)
        start = torch.cuda.Event(enable_timing=True)
        side.wait_stream(torch.cuda.current_stream(self.device))
        start.record(side)
        done.record(side)  # creates the event so its handle can be passed down
        n_proj = len(self.wl.projections)
        todo = self.adapters if adapters is None else adapters
        rows = [self.store.ptrs(a, n_proj) for a in todo]
        self.pool.fetch_many_async(todo, [r[0] for r in rows], [r[1] for r in rows],
                                   side.cuda_stream, done.cuda_event)
        torch.cuda.current_stream(self.device).wait_event(done)
        self._fetch_done = done
        done.synchronize()
        return start.elapsed_time(done)

    def call(self, proj: int, policy: int = _lib.POLICY_AUTO, wl=None) -> _lib.Call:
        wl = wl or self.wl
        p = wl.projections[proj]
        return _lib.Call(pool_ptr=self.pool_t.data_ptr(), n_pages=self.n_pages,
                         page_elems=wl.page_elems, dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out,
                         page_table_ptr=self.pt_dev[proj].data_ptr(),
                         page_table_len=self.pt_len[proj], base=self.base[proj], rank=wl.ranks,
                         scale=wl.scales.astype(np.float32), r_max=self.r_max,
                         n_tokens=wl.n_tokens, seg_offsets=wl.seg_offsets,
                         seg_adapter=wl.seg_adapter, token_adapter=wl.token_adapter,
                         policy=policy)

    def inputs(self, proj: int):
        """(x, y) device tensors for a projection; y holds y0."""
        return _dev_i16(self.wl.x(proj), self.device), _dev_i16(self.wl.y0(proj), self.device)

    def workspace(self, call: _lib.Call) -> torch.Tensor:
        """Device workspace for calls like `call` (zero-filled once, as the library requires)."""
        return torch.zeros(_lib.workspace_size(call), dtype=torch.uint8, device=self.device)

    def gathered_workspace(self, call: _lib.Call) -> torch.Tensor:
        return torch.zeros(_lib.gathered_workspace_size(call), dtype=torch.uint8, device=self.device)

    def apply_gathered(self, call, x, y, ws, stream=None):
        s = stream or torch.cuda.current_stream(self.device)
        _lib.apply_gathered(call, x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream)

    def apply(self, call: _lib.Call, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
              stream: Optional[torch.cuda.Stream] = None):
        s = stream or torch.cuda.current_stream(self.device)
        _lib.apply(call, x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream)

    def bind_apply(self, call: _lib.Call, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor,
                   stream: Optional[torch.cuda.Stream] = None, gathered: bool = False):
        """apply() (or apply_gathered()) with its arguments marshalled once (a callable
        with no arguments)."""
        s = stream or torch.cuda.current_stream(self.device)
        return _lib.bind_apply(call, x.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                               s.cuda_stream, gathered=gathered)

    def multi_workspace(self, calls) -> torch.Tensor:
        """Device workspace for apply_multi over `calls` (zero-filled once)."""
        return torch.zeros(_lib.workspace_size_multi(calls), dtype=torch.uint8, device=self.device)

    def bind_apply_multi(self, calls, xs, ys, ws: torch.Tensor,
                         stream: Optional[torch.cuda.Stream] = None):
        """slora_apply_multi over several projections' calls, marshalled once."""
        s = stream or torch.cuda.current_stream(self.device)
        return _lib.bind_apply_multi(calls, [x.data_ptr() for x in xs], [y.data_ptr() for y in ys],
                                     ws.data_ptr(), ws.numel(), s.cuda_stream)

    def shrink(self, call, x, v, ws, stream=None):
        s = stream or torch.cuda.current_stream(self.device)
        _lib.shrink(call, x.data_ptr(), v.data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream)

    def expand(self, call, v, y, ws, stream=None):
        s = stream or torch.cuda.current_stream(self.device)
        _lib.expand(call, v.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream)

    def close(self):
        torch.cuda.synchronize(self.device)
        self.pool.destroy()


class ServingLoop:
    """Continuous batching of one projection over a unified pool: slora_sched admits
    requests FIFO by free pages, slora_residency keeps adapters resident (LRU eviction),
    adapters a step needs are fetched on a side stream from the host store, and the
    step's batch (new prompts as segments, one decode token per running request) runs
    through slora_apply on the compute stream once the fetch event has fired.

    Every adapter the workload defines is in the host store; only the pool's pages limit
    how many are resident at once. The weights, x and y0 of a step are seeded synthetic
    data (the same generators the tests and the oracle use)."""

    def __init__(self, wl, n_pages: int, kv_pages_per_token: int = 2, max_batch_tokens: int = 4096,
                 max_running: int = 512, proj: int = 0, device: str = "cuda", seed: int = 0):
        self.wl, self.proj, self.device = wl, proj, torch.device(device)
        p = wl.projections[proj]
        self.d_in, self.d_out = p.d_in, p.d_out
        self.n_pages = n_pages
        P = wl.page_elems
        self.pool_t = torch.full((n_pages * P,), SENTINEL_I16[wl.dtype], dtype=torch.int16,
                                 device=self.device)
        self.pool = _lib.Pool(self.pool_t.data_ptr(), n_pages, P, wl.dtype, seed)
        self.res = _lib.Residency(self.pool, [p.d_in], [p.d_out])
        self.sched = _lib.Scheduler(self.pool, self.res, kv_pages_per_token, max_batch_tokens,
                                    max_running)
        # the projection alone (its weights are drawn as projection 0 of this workload)
        self.one = dataclass_replace(wl, projections=[p], _cache={})
        self.store = HostStore(self.one, list(range(wl.n_adapters)))
        self.side = torch.cuda.Stream(device=self.device)
        self.stream = torch.cuda.current_stream(self.device)
        self.scales = wl.scales.astype(np.float32)
        self.r_max = max(int(wl.ranks.max()), 1)
        self.fetch_bytes = 0
        self.steps_run = 0

    def submit(self, request_id, adapter_id, prompt_len, max_new_tokens, deadline_step=-1):
        r = int(self.wl.ranks[adapter_id]) if adapter_id >= 0 else 0
        self.sched.submit(request_id, adapter_id, r, prompt_len, max_new_tokens, deadline_step)

    def step(self, seed: int):
        """Plan one step, fetch what it needs, run its batch. Returns (batch dict, x, y0, y)
        as host arrays (uint16 bits) for checking, or the batch alone when it is empty."""
        b = self.sched.step()
        if b["fetch"].size:
            done = torch.cuda.Event()
            self.side.wait_stream(self.stream)
            ids = [int(a) for a in b["fetch"]]
            rows = [self.store.ptrs(a, 1) for a in ids]
            self.pool.fetch_many_async(ids, [r[0] for r in rows], [r[1] for r in rows],
                                       self.side.cuda_stream, None)
            self.fetch_bytes += sum(int(self.wl.ranks[a]) * (self.d_in + self.d_out) * 2 for a in ids)
            done.record(self.side)
            self.stream.wait_event(done)
        if b["n_tokens"] == 0:
            return b, None, None, None
        pt, base, rank = self.pool.page_table(0, self.wl.n_adapters)
        pt_dev = torch.from_numpy(np.ascontiguousarray(pt)).to(self.device) if pt.size else \
            torch.zeros(1, dtype=torch.int32, device=self.device)
        T = b["n_tokens"]
        rng_x = np.random.default_rng([seed, 1])
        rng_y = np.random.default_rng([seed, 2])
        from workloads import normal_bits
        x = normal_bits(rng_x, (T, self.d_in), 1.0, self.wl.dtype)
        y0 = normal_bits(rng_y, (T, self.d_out), 1.0, self.wl.dtype)
        call = _lib.Call(pool_ptr=self.pool_t.data_ptr(), n_pages=self.n_pages,
                         page_elems=self.wl.page_elems, dtype=self.wl.dtype, d_in=self.d_in,
                         d_out=self.d_out, page_table_ptr=pt_dev.data_ptr(), page_table_len=pt.size,
                         base=base, rank=self.wl.ranks, scale=self.scales, r_max=self.r_max,
                         n_tokens=T, seg_offsets=b["seg_offsets"], seg_adapter=b["seg_adapter"],
                         token_adapter=b["token_adapter"])
        xd = _dev_i16(x, self.device)
        yd = _dev_i16(y0, self.device)
        ws = torch.zeros(_lib.workspace_size(call), dtype=torch.uint8, device=self.device)
        _lib.apply(call, xd.data_ptr(), yd.data_ptr(), ws.data_ptr(), ws.numel(), self.stream.cuda_stream)
        status = _lib.workspace_status(ws.data_ptr(), self.stream.cuda_stream)
        if status:
            raise RuntimeError(f"step {b['step']}: a decode launch gave up waiting")
        self.steps_run += 1
        return b, x, y0, yd.cpu().numpy().view(np.uint16)

    def close(self):
        torch.cuda.synchronize(self.device)
        self.sched.destroy()
        self.res.destroy()
        self.pool.destroy()
