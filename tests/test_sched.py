"""Adapter residency (LRU over the unified pool) and continuous-batching admission
(CPU only: host bookkeeping, no device memory is touched).

Both are checked step by step against independent Python models of the rules the
header states, on seeded random traces, and against invariants: pages are conserved
(free + KV + adapter pages = pool size at every step), no page has two owners, every
running request holds exactly (prompt + decoded tokens) x kv_pages_per_token KV pages,
admission is FIFO within the token budget, requests past their deadline never run, and
every step's batch is a valid routing for the compute calls.
"""

from collections import OrderedDict

import numpy as np
import pytest

from heterogeneous_lora_amd import _lib

FAKE_DEV = 0x7F0000000000  # never dereferenced by host code
D_IN, D_OUT, P = [128, 64], [64, 200], 64  # pages per rank row: (2 + 1) + (1 + 4) = 8


def pages_of(rank):
    return rank * sum(-(-a // P) + -(-b // P) for a, b in zip(D_IN, D_OUT))


def _pool(n_pages, seed=5):
    return _lib.Pool(FAKE_DEV, n_pages, P, "f16", seed)


# ------------------------------------------------------------------ residency

class LruModel:
    """The residency rules: pins per adapter; an acquire of a non-resident adapter evicts
    unpinned adapters, least recently used first, until the free pages hold it (nothing
    at all if even every unpinned adapter would not be enough); a prefetch only uses
    free pages. A use (acquire) refreshes recency; an unpinned adapter's recency is its
    last use or, for a prefetch, the prefetch."""

    def __init__(self, n_pages):
        self.free = n_pages
        self.res = {}  # id -> [rank, pins]
        self.lru = OrderedDict()  # unpinned, oldest first

    def acquire(self, a, r):
        if a in self.res:
            if self.res[a][1] == 0:
                del self.lru[a]
            self.res[a][1] += 1
            return False, []
        need = pages_of(r)
        have, victims = self.free, []
        for v in self.lru:
            if have >= need:
                break
            victims.append(v)
            have += pages_of(self.res[v][0])
        if have < need:
            raise MemoryError
        for v in victims:
            self.free += pages_of(self.res[v][0])
            del self.lru[v]
            del self.res[v]
        self.free -= need
        self.res[a] = [r, 1]
        return True, victims

    def prefetch(self, a, r):
        if a in self.res or self.free < pages_of(r):
            return False
        self.free -= pages_of(r)
        self.res[a] = [r, 0]
        self.lru[a] = None
        return True

    def release(self, a):
        self.res[a][1] -= 1
        if self.res[a][1] == 0:
            self.lru[a] = None  # most recent at the end (released in use order is not needed)


def test_residency_lru_order_and_pins():
    pool = _pool(8 * 16)  # room for 16 rank rows
    res = _lib.Residency(pool, D_IN, D_OUT)
    for a in (1, 2, 3):
        assert res.acquire(a, 4) == (True, [])  # 3 x 32 pages
    assert res.acquire(2, 4) == (False, []) and res.pins(2) == 2
    for a in (1, 3, 2, 2):
        res.release(a)
    # unpinned by recency of use: 1 (oldest use), 3, 2 (used last)
    fetch, ev = res.acquire(9, 8)  # 64 pages: 32 free + adapter 1's 32
    assert fetch and ev == [1] and res.pins(1) == -1
    fetch, ev = res.acquire(10, 4)  # 32 more: evicts 3 next
    assert fetch and ev == [3]
    # pinned adapters (9, 10) are never evicted: 2 is all that is left to evict
    with pytest.raises(_lib.SloraError) as e:
        res.acquire(11, 16)
    assert e.value.code == _lib.E_POOL_FULL and res.pins(2) == 0  # nothing evicted
    with pytest.raises(_lib.SloraError) as e:
        res.acquire(9, 4)  # resident with another rank
    assert e.value.code == _lib.E_INVALID
    with pytest.raises(_lib.SloraError) as e:
        res.release(2)  # not pinned
    assert e.value.code == _lib.E_STATE
    st = res.info()
    assert (st["resident"], st["pinned"], st["misses"], st["hits"], st["evictions"]) == (3, 2, 5, 1, 2)
    own = pool.owners()
    for a, r in ((2, 4), (9, 8), (10, 4)):
        assert (own == a).sum() == pages_of(r)
    assert (own >= 0).sum() + pool.n_free() == pool.n_pages
    res.destroy()
    pool.destroy()


def test_residency_prefetch_uses_free_pages_only():
    pool = _pool(8 * 12)
    res = _lib.Residency(pool, D_IN, D_OUT)
    assert res.acquire(1, 8) == (True, [])  # 64 of 96 pages
    assert res.prefetch(2, 4)  # 32 free: fits
    assert not res.prefetch(3, 1) and res.pins(3) == -1  # no free page left; evicts nothing
    assert res.pins(2) == 0  # prefetched, not pinned
    assert not res.prefetch(2, 4)  # already resident
    res.release(1)
    fetch, ev = res.acquire(4, 8)  # evicts 2 (prefetched earlier) before 1 (released later)
    assert fetch and ev == [2, 1]
    res.destroy()
    pool.destroy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_residency_matches_model_on_random_trace(seed):
    rng = np.random.default_rng(seed)
    n_pages = 8 * 64
    pool = _pool(n_pages, seed)
    res = _lib.Residency(pool, D_IN, D_OUT)
    model = LruModel(n_pages)
    ranks = {a: int(rng.choice([1, 2, 4, 8, 16])) for a in range(40)}
    pinned = []
    for it in range(600):
        op = rng.random()
        if op < 0.5 or not pinned:
            a = int(rng.integers(40))
            try:
                want = model.acquire(a, ranks[a])
            except MemoryError:
                with pytest.raises(_lib.SloraError) as e:
                    res.acquire(a, ranks[a])
                assert e.value.code == _lib.E_POOL_FULL
                continue
            assert res.acquire(a, ranks[a]) == want, it
            pinned.append(a)
        elif op < 0.85:
            a = pinned.pop(int(rng.integers(len(pinned))))
            model.release(a)
            res.release(a)
        else:
            a = int(rng.integers(40))
            assert res.prefetch(a, ranks[a]) == model.prefetch(a, ranks[a]), it
        own = pool.owners()
        assert pool.n_free() == model.free
        for a, (r, pins) in model.res.items():
            assert res.pins(a) == pins and (own == a).sum() == pages_of(r)
        assert ((own >= 0).sum() == sum(pages_of(r) for r, _ in model.res.values()))
    res.destroy()
    pool.destroy()


# ------------------------------------------------------------------ admission

class SchedModel:
    """The admission rules of the header, written independently: returns each step's
    (segments as (request, adapter, prompt), decode (request, adapter) list, finished,
    aborted with reasons). Adapters are not modelled here (no residency)."""

    def __init__(self, n_free, ppt, budget, max_running):
        self.free, self.ppt, self.budget, self.max_running = n_free, ppt, budget, max_running
        self.queue, self.running, self.step_no = [], [], 0

    def submit(self, rid, adapter, prompt, max_new, deadline):
        self.queue.append(dict(id=rid, adapter=adapter, prompt=prompt, max_new=max_new,
                               deadline=deadline, gen=0, kv=0))

    def step(self):
        self.step_no += 1
        now = self.step_no
        finished, aborted = [], []
        keep = []
        for q in self.running:
            if q["gen"] >= q["max_new"]:
                finished.append(q["id"])
                self.free += q["kv"]
            elif q["deadline"] >= 0 and now > q["deadline"]:
                aborted.append((q["id"], 1))
                self.free += q["kv"]
            else:
                keep.append(q)
        self.running = keep
        live = []
        for q in self.queue:
            if q["deadline"] >= 0 and now > q["deadline"]:
                aborted.append((q["id"], 1))
            else:
                live.append(q)
        self.queue = live
        while self.running and self.free < len(self.running) * self.ppt:
            q = self.running.pop()
            aborted.append((q["id"], 2))
            self.free += q["kv"]
        decode = []
        for q in self.running:
            q["kv"] += self.ppt
            self.free -= self.ppt
            q["gen"] += 1
            decode.append((q["id"], q["adapter"]))
        tokens = len(decode)
        segs, admitted = [], []
        while self.queue and len(self.running) + len(admitted) < self.max_running:
            q = self.queue[0]
            if tokens + q["prompt"] > self.budget or self.free < q["prompt"] * self.ppt:
                break
            self.queue.pop(0)
            q["kv"] = q["prompt"] * self.ppt
            self.free -= q["kv"]
            q["gen"] = 1
            tokens += q["prompt"]
            segs.append((q["id"], q["adapter"], q["prompt"]))
            admitted.append(q)
        self.running += admitted
        return segs, decode, finished, aborted


def _check_batch(b, model_out):
    segs, decode, finished, aborted = model_out
    so = b["seg_offsets"]
    assert list(b["seg_request"]) == [s[0] for s in segs]
    assert list(b["seg_adapter"]) == [s[1] for s in segs]
    assert list(np.diff(so)) == [s[2] for s in segs] and so[0] == 0
    assert list(b["token_request"]) == [d[0] for d in decode]
    assert list(b["token_adapter"]) == [d[1] for d in decode]
    assert b["n_tokens"] == int(so[-1]) + len(decode)
    assert sorted(b["finished"]) == sorted(finished)
    assert sorted(zip(b["aborted"], b["abort_reason"])) == sorted(aborted)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_sched_matches_model_and_conserves_pages(seed):
    rng = np.random.default_rng(100 + seed)
    n_pages, ppt, budget, max_running = 3000, 2, 400, 48
    pool = _pool(n_pages, seed)
    sched = _lib.Scheduler(pool, None, ppt, budget, max_running)
    model = SchedModel(n_pages, ppt, budget, max_running)
    rid = 0
    held = {}
    for step in range(150):
        for _ in range(int(rng.poisson(3))):
            prompt = int(rng.integers(1, 120))
            max_new = int(rng.integers(1, 40))
            deadline = int(step + 1 + rng.integers(2, 60)) if rng.random() < 0.3 else -1
            adapter = int(rng.integers(-1, 20))
            sched.submit(rid, adapter, 0 if adapter < 0 else 8, prompt, max_new, deadline)
            model.submit(rid, adapter, prompt, max_new, deadline)
            rid += 1
        b = sched.step()
        _check_batch(b, model.step())
        assert b["n_tokens"] <= budget and b["n_running"] <= max_running
        # pages: every running request holds (prompt + decoded) x ppt pages of its own
        own = pool.owners()
        assert (own == -2).sum() == n_pages - pool.n_free() == n_pages - model.free
        held = {q["id"]: q for q in model.running}
        pages = set()
        for q in model.running:
            mine = sched.request_pages(q["id"])
            assert mine.size == q["kv"] and (own[mine] == -2).all()
            assert pages.isdisjoint(mine.tolist())
            pages.update(mine.tolist())
        # nothing past its deadline runs
        for r in list(b["token_request"]) + list(b["seg_request"]):
            d = held[int(r)]["deadline"]
            assert d < 0 or b["step"] <= d
    sched.destroy()
    assert pool.n_free() == n_pages  # destroy returned every running request's pages
    pool.destroy()


def test_sched_finish_fifo_and_pool_full_abort():
    pool = _pool(200)
    sched = _lib.Scheduler(pool, None, 2, 64, 8)
    sched.submit(1, 3, 8, 30, 5)     # 60 pages
    sched.submit(2, 4, 8, 40, 50)    # 80 pages; budget 64 tokens: waits for the next step
    sched.submit(3, 4, 8, 10, 50)    # behind 2 (FIFO: not admitted before it)
    b = sched.step()
    assert list(b["seg_request"]) == [1] and b["n_tokens"] == 30
    b = sched.step()
    assert list(b["seg_request"]) == [2, 3] and list(b["token_request"]) == [1]
    sched.finish(3)  # an end-of-sequence token: pages back at once
    assert pool.n_free() == 200 - 62 - 80
    # 1 produces 5 tokens (prefill + 4 decodes), then leaves
    for _ in range(3):
        b = sched.step()
    assert list(b["token_request"]) == [1, 2]
    b = sched.step()
    assert list(b["finished"]) == [1] and list(b["token_request"]) == [2]
    # fill the pool: the newest running request is aborted when its next token does not fit
    sched.submit(7, -1, 0, 20, 1000)
    sched.submit(8, -1, 0, 20, 1000)
    got = {}
    for _ in range(40):
        b = sched.step()
        for r, why in zip(b["aborted"], b["abort_reason"]):
            got[int(r)] = int(why)
        if got:
            break
    assert got == {8: _lib.ABORT_POOL_FULL}
    with pytest.raises(_lib.SloraError) as e:
        sched.finish(8)  # gone already
    assert e.value.code == _lib.E_STATE
    with pytest.raises(_lib.SloraError) as e:
        sched.submit(2, 0, 8, 5, 5)  # id still running
    assert e.value.code == _lib.E_STATE
    sched.destroy()
    pool.destroy()


def test_sched_with_residency_pins_fetches_and_evicts():
    """Adapters of admitted requests are pinned while they run, fetched when they were not
    resident, and evicted (least recently used, unpinned) when a new request needs room;
    every step's batch is a valid routing for the compute calls (checked by the planner)."""
    n_pages = 8 * 40 + 400  # adapters of up to 40 rank rows, plus KV room
    pool = _pool(n_pages)
    res = _lib.Residency(pool, D_IN, D_OUT)
    sched = _lib.Scheduler(pool, res, 2, 256, 16)
    rng = np.random.default_rng(7)
    ranks = {a: int(rng.choice([4, 8, 16])) for a in range(30)}
    fetched, evicted_total = set(), 0
    rid = 0
    for step in range(120):
        for _ in range(int(rng.poisson(1.5))):
            a = int(rng.integers(30))
            sched.submit(rid, a, ranks[a], int(rng.integers(1, 40)), int(rng.integers(1, 12)))
            rid += 1
        b = sched.step()
        for a in b["evicted"]:
            fetched.discard(int(a))
            evicted_total += 1
        for a in b["fetch"]:
            assert res.pins(int(a)) >= 1
            fetched.add(int(a))
        used = set(int(a) for a in b["seg_adapter"]) | set(int(a) for a in b["token_adapter"])
        for a in used:
            assert res.pins(a) >= 1 and a in fetched  # pinned and fetched before use
        own = pool.owners()
        assert (own >= 0).sum() + (own == -2).sum() + pool.n_free() == n_pages
        if b["n_tokens"]:
            d_in, d_out = D_IN[0], D_OUT[0]
            pt, base, rank = pool.page_table(0, 30)
            call = _lib.Call(pool_ptr=FAKE_DEV, n_pages=n_pages, page_elems=P, dtype="f16", d_in=d_in,
                             d_out=d_out, page_table_ptr=FAKE_DEV, page_table_len=pt.size, base=base,
                             rank=np.array([ranks[a] for a in range(30)], np.int32),
                             scale=np.ones(30, np.float32), r_max=16, n_tokens=b["n_tokens"],
                             seg_offsets=b["seg_offsets"], seg_adapter=b["seg_adapter"],
                             token_adapter=b["token_adapter"])
            groups, toks = _lib.plan_inspect(call)
            assert np.array_equal(np.sort(toks), np.arange(b["n_tokens"]))
    assert evicted_total > 0 and res.info()["misses"] > 30
    sched.destroy()
    assert res.info()["pinned"] == 0
    res.destroy()
    pool.destroy()


def test_ordered_pool_hands_out_pages_in_order():
    """The pool of the split-memory ablation: no shuffle, so one adapter's pages are
    consecutive, and a scheduler can take KV pages from one pool while its residency
    manager keeps adapters in another."""
    apool = _lib.Pool(FAKE_DEV, 1000, P, "f16", 0, ordered=True)
    apool.alloc_adapter(3, 4, D_IN, D_OUT)
    apool.alloc_adapter(1, 2, D_IN, D_OUT)
    for proj in (0, 1):
        pt, base, rank = apool.page_table(proj, 4)
        per_row = -(-D_IN[proj] // P) + -(-D_OUT[proj] // P)
        for a in (1, 3):  # each adapter's pages of a projection are consecutive
            seg = pt[base[a]:base[a] + rank[a] * per_row]
            assert np.array_equal(seg, np.arange(seg[0], seg[0] + seg.size))
    own = apool.owners()
    assert (own[:32] == 3).all() and (own[32:48] == 1).all() and (own[48:] == -1).all()
    kv = _pool(400)
    res = _lib.Residency(apool, D_IN, D_OUT)
    sched = _lib.Scheduler(kv, res, 2, 128, 8)
    sched.submit(0, 7, 8, 50, 3)
    b = sched.step()
    assert list(b["fetch"]) == [7] and res.pins(7) == 1
    assert kv.n_free() == 400 - 100 and (kv.owners() == -2).sum() == 100
    assert (apool.owners() == 7).sum() == pages_of(8)
    sched.destroy()
    res.destroy()
    kv.destroy()
    apool.destroy()


def test_capacity_ablation_runs_on_the_host():
    """bench.py's unified-against-split simulation: both configurations serve the same
    trace; every token served is a prefill or a decode token."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    d = bench.capacity_ablation(steps=40, fractions=(0.5,))
    assert set(d["results"]) == {"unified", "split adapters 50%"}
    for r in d["results"].values():
        assert r["tokens"] == r["prefill_tokens"] + r["decode_tokens"] > 0
