"""The seeded synthetic inputs: deterministic per seed (their digests are stored in
tests/golden/workload_hashes.json, written by make_workload_hashes.py from the
workloads module alone), and shaped as the input recipe states (token counts, length
and rank ranges, routing skew, value scales)."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import workloads  # noqa: E402
from make_workload_hashes import fingerprint  # noqa: E402


def decode(bits, dtype):
    bits = np.asarray(bits).view(np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_generators_match_stored_digests():
    with open(os.path.join(HERE, "golden", "workload_hashes.json")) as f:
        want = json.load(f)
    assert set(want) == set(workloads.CONFIGS)
    for name in workloads.CONFIGS:
        assert fingerprint(workloads.make(name)) == want[name], name


def test_seeds_are_independent_streams():
    a, b = workloads.make("decode_7b", 0), workloads.make("decode_7b", 1)
    assert not np.array_equal(a.token_adapter, b.token_adapter)
    assert not np.array_equal(a.x(0)[:4], b.x(0)[:4])
    # x and y0 of different projections come from different streams
    p = workloads.make("prefill_sgmv")
    assert not np.array_equal(p.x(0)[:4], p.x(1)[:4])


def test_recipe_shapes_and_ranges():
    d = workloads.make("decode_7b")
    assert d.n_tokens == 256 and d.n_segments == 0 and d.projections[0].d_in == 4096
    assert set(np.unique(d.ranks)) <= {8, 16, 32, 64}
    assert len(d.active_adapters()) == 126  # Zipf(1.0) over 1000 ids, 256 draws
    counts = np.bincount(d.token_adapter, minlength=d.n_adapters)
    assert counts[0] == counts.max() and counts[0] >= 20  # the head of the Zipf law is hot
    p = workloads.make("prefill_sgmv")
    lens = np.diff(p.seg_offsets)
    assert p.n_segments == 64 and lens.min() >= 8 and lens.max() <= 512 and p.n_tokens == 18571
    assert len(p.projections) == 4 and p.dtype == "bf16"
    m = workloads.make("mixed_13b")
    lens = np.diff(m.seg_offsets)
    assert m.n_segments == 48 and lens.min() >= 16 and lens.max() <= 256
    assert m.token_adapter.size == 512 and set(np.unique(m.ranks)) <= {8, 16, 32, 64, 128}
    assert m.kv_seq_lens.size == 560 and m.kv_seq_lens.min() >= 64 and m.kv_seq_lens.max() <= 2048
    mlp = workloads.make("mlp_asym")
    assert mlp.n_tokens == 4096 and mlp.token_adapter.min() >= 0 and mlp.token_adapter.max() < 500
    assert [(q.d_in, q.d_out) for q in mlp.projections] == [(4096, 11008), (4096, 11008), (11008, 4096)]
    # scale = 16 / rank for every adapter of rank > 0
    for wl in (d, p, m, mlp):
        assert np.allclose(wl.scales, 16.0 / wl.ranks)


def test_value_scales():
    """Weights N(0, 0.02) and x, y0 N(0, 1), after the cast to the workload's type."""
    for name in ("decode_7b", "prefill_sgmv"):
        wl = workloads.make(name)
        a = int(wl.active_adapters()[0])
        at, b = wl.adapter(a, 0)
        for w in (at, b):
            v = decode(w, wl.dtype)
            assert abs(v.mean()) < 0.002 and 0.018 < v.std() < 0.022, name
        x = decode(wl.x(0)[:64], wl.dtype)
        y0 = decode(wl.y0(0)[:64], wl.dtype)
        for v in (x, y0):
            assert abs(v.mean()) < 0.02 and 0.98 < v.std() < 1.02, name
