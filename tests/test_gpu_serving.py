"""Continuous batching through the HIP path: the scheduler admits requests over a pool
that cannot hold every adapter at once, the residency manager evicts and the runtime
fetches adapters on a side stream between steps, and every step's outputs (new prompts
and decode tokens together) are checked against the oracle on every row."""

import dataclasses

import numpy as np
import pytest

import workloads
from gpu_util import check_close, margin_line, oracle_ref, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _serving_workload():
    wl = workloads.random_small(401, dtype="f16", n_adapters=48, d_in=1024, d_out=1536,
                                page_elems=512, n_tokens=1, n_segments=0, rank_choices=(8, 16, 32, 64))
    return wl


@pytest.mark.timeout(600)
def test_serving_loop_with_evictions_matches_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from heterogeneous_lora_amd import _lib, runtime
    _lib.load()
    wl = _serving_workload()
    per_rank_row = 2 + 3  # pages of one rank row: A^T 1024 / 512, B 1536 / 512
    all_pages = int(wl.ranks.sum()) * per_rank_row
    n_pages = all_pages // 3 + 2000  # about a third of the adapters, plus KV room
    loop = runtime.ServingLoop(wl, n_pages=n_pages, kv_pages_per_token=2, max_batch_tokens=384,
                               max_running=64, device="cuda")
    rng = np.random.default_rng(3)
    p = np.arange(1, wl.n_adapters + 1, dtype=np.float64) ** -0.8
    p /= p.sum()
    rid = 0
    checked = evicted = fetched = 0
    worst = 0.0
    for step in range(40):
        for _ in range(int(rng.poisson(4))):
            a = int(rng.choice(wl.n_adapters, p=p))
            loop.submit(rid, a, int(rng.integers(4, 64)), int(rng.integers(1, 16)))
            rid += 1
        b, x, y0, y = loop.step(seed=step)
        evicted += b["evicted"].size
        fetched += b["fetch"].size
        if x is None:
            continue
        say(f"[gpu] serving step {b['step']}: {b['n_tokens']} tokens, {len(b['seg_adapter'])} prompts, "
            f"{b['token_adapter'].size} decode, fetched {b['fetch'].size}, evicted {b['evicted'].size}")
        batch_wl = dataclasses.replace(loop.one, seg_offsets=b["seg_offsets"],
                                       seg_adapter=b["seg_adapter"], token_adapter=b["token_adapter"],
                                       _cache={})
        ref, _ = oracle_ref(batch_wl, 0, x=x, y0=y0)
        worst = max(worst, check_close(y, ref, wl.dtype, f"serving step {b['step']}"))
        checked += 1
    margin_line(f"serving loop, {checked} steps with evictions", worst)
    assert checked >= 30 and evicted > 0 and fetched > wl.n_adapters // 3
    loop.close()
