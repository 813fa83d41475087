"""Writes workload_hashes.json: SHA-256 digests of the seeded synthetic inputs (routing,
ranks, KV lengths, the first rows of x and y0, one adapter's weights) of every named
workload, so that a change to a generator shows up as a failing test. Calls only the
workloads module (no library, no oracle).

    python3 tests/golden/make_workload_hashes.py
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import workloads  # noqa: E402


def digest(a) -> str:
    a = np.ascontiguousarray(a)
    return hashlib.sha256(a.dtype.str.encode() + str(a.shape).encode() + a.tobytes()).hexdigest()


def fingerprint(wl) -> dict:
    a0 = int(wl.active_adapters()[0])
    at, b = wl.adapter(a0, 0)
    return {
        "ranks": digest(wl.ranks), "seg_offsets": digest(wl.seg_offsets),
        "seg_adapter": digest(wl.seg_adapter), "token_adapter": digest(wl.token_adapter),
        "kv_seq_lens": digest(wl.kv_seq_lens), "scales": digest(wl.scales),
        "x0_rows64": digest(wl.x(0)[:64]), "y0_0_rows64": digest(wl.y0(0)[:64]),
        "adapter_first_active": a0, "adapter_at": digest(at), "adapter_b": digest(b),
    }


def main():
    out = {name: fingerprint(workloads.make(name)) for name in workloads.CONFIGS}
    with open(os.path.join(HERE, "workload_hashes.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
