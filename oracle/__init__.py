"""CPU oracle for heterogeneous batched LoRA (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. The GPU library never imports, links or calls it, and it imports nothing
from the GPU library.

`lora(...)` wraps `oracle_lora` in oracle.c: an fp64 loop over tokens that gathers
adapter rows through a page table, as the S-LoRA pages describe the computation
("Makale Bulteni - S-LoRA", section "Iddia ve Gerceklik"; the S-LoRA overview,
sections "1. Unified Paging" and "2. Heterogeneous Batching").

`build_pool(...)` is the oracle's own paged layout: it places the rows of the
adapters it is given on randomly permuted pages of a private pool image, fills
every unused page and every page tail with a NaN sentinel, and returns the page
table. It shares nothing with the GPU library's allocator; the two paths only
need to agree on the result, which does not depend on where pages sit.

Every function here is pinned by tests/test_oracle_pins.py against closed forms
(numpy dense products), special cases and invariants; see that file.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

SENTINEL = {"f16": 0x7E00, "bf16": 0x7FC0}  # quiet NaN bit patterns
DTYPE_CODE = {"f16": 0, "bf16": 1}


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile oracle.c with gcc (-O2, IEEE semantics kept: no -ffast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    P = ctypes.c_void_p
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_bfloat16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bfloat16_to_double.restype = ctypes.c_double
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_lora.argtypes = [i32, i32, i32, i64, P, P, P, i64, i32, P, i64, i32, P, P, P,
                                i32, P, P, P, i64, P, P, P, i32, i32]
    lib.oracle_lora.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None):
    """Load liboracle.so, building it first when it is missing."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def decode(bits: np.ndarray, dtype: str, lib=None) -> np.ndarray:
    """fp16/bf16 bit patterns -> float64 through the oracle's own decoders (slow, elementwise)."""
    lib = lib or load()
    f = lib.oracle_half_to_double if dtype == "f16" else lib.oracle_bfloat16_to_double
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(b)) for b in flat], dtype=np.float64).reshape(np.shape(bits))


class OracleError(RuntimeError):
    pass


def lora(*, dtype: str, d_in: int, d_out: int, x: np.ndarray, y0: np.ndarray,
         pool: np.ndarray, page_elems: int, page_table: np.ndarray, base: np.ndarray,
         rank: np.ndarray, scale: np.ndarray, seg_offsets: np.ndarray, seg_adapter: np.ndarray,
         token_adapter: np.ndarray, eval_tokens: Optional[np.ndarray] = None,
         r_max: Optional[int] = None, want_v: bool = False, n_threads: int = 1,
         lib=None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Run the oracle. Returns (y_ref [n_eval x d_out] float64, v_ref or None)."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y0 = np.ascontiguousarray(y0, dtype=np.uint16)
    pool = np.ascontiguousarray(pool, dtype=np.uint16)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    base = np.ascontiguousarray(base, dtype=np.int64)
    rank = np.ascontiguousarray(rank, dtype=np.int32)
    scale = np.ascontiguousarray(scale, dtype=np.float64)
    so = np.ascontiguousarray(seg_offsets, dtype=np.int32)
    sa = np.ascontiguousarray(seg_adapter, dtype=np.int32)
    ta = np.ascontiguousarray(token_adapter, dtype=np.int32)
    n_tokens = x.shape[0]
    if x.shape != (n_tokens, d_in) or y0.shape != (n_tokens, d_out):
        raise ValueError("x / y0 shape")
    if eval_tokens is not None:
        ev = np.ascontiguousarray(eval_tokens, dtype=np.int64)
        n_eval = ev.shape[0]
    else:
        ev, n_eval = None, n_tokens
    if r_max is None:
        r_max = int(rank.max()) if rank.size else 0
    y_ref = np.empty((n_eval, d_out), dtype=np.float64)
    v_ref = np.empty((n_eval, max(r_max, 1)), dtype=np.float64) if want_v else None
    n_pages = pool.size // page_elems
    rc = lib.oracle_lora(DTYPE_CODE[dtype], d_in, d_out, n_tokens, _ptr(x), _ptr(y0), _ptr(pool),
                         n_pages, page_elems, _ptr(pt), pt.size, rank.size, _ptr(base),
                         _ptr(rank), _ptr(scale), sa.size, _ptr(so), _ptr(sa), _ptr(ta), n_eval,
                         _ptr(ev), _ptr(y_ref), _ptr(v_ref), r_max, n_threads)
    if rc != 0:
        raise OracleError(f"oracle_lora returned {rc}")
    if v_ref is not None:
        v_ref = v_ref[:, :r_max]
    return y_ref, v_ref


def build_pool(adapters: Dict[int, Tuple[np.ndarray, np.ndarray]], n_adapters: int,
               d_in: int, d_out: int, page_elems: int, dtype: str,
               rng: np.random.Generator, spare_pages: int = 7
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Lay adapters out on randomly permuted pages of a private pool image.

    adapters: {id: (AT [r x d_in], B [r x d_out])} uint16 bits.
    Returns (pool uint16 [n_pages * P], page_table int32, base int64 [n_adapters], -1 = absent).
    """
    P = page_elems
    cA, cB = -(-d_in // P), -(-d_out // P)
    base = np.full(n_adapters, -1, dtype=np.int64)
    rows = []  # (logical entry, source row) in page-table order
    entry = 0
    for a in sorted(adapters):
        at, b = adapters[a]
        r = at.shape[0]
        if at.shape != (r, d_in) or b.shape != (r, d_out):
            raise ValueError("adapter shape")
        base[a] = entry
        for k in range(r):
            for c in range(cA):
                rows.append(at[k, c * P:(c + 1) * P])
        for k in range(r):
            for c in range(cB):
                rows.append(b[k, c * P:(c + 1) * P])
        entry += r * (cA + cB)
    n_pages = entry + spare_pages
    perm = rng.permutation(n_pages).astype(np.int32)
    pool = np.full((n_pages, P), SENTINEL[dtype], dtype=np.uint16)
    pt = perm[:entry].copy()
    for e, chunk in enumerate(rows):
        pool[pt[e], :chunk.shape[0]] = chunk
    return pool.reshape(-1), pt, base


def reference(wl, proj: int, eval_tokens: Optional[Sequence[int]] = None, *,
              n_threads: int = 1, perm_seed: int = 12345, want_v: bool = False,
              x: Optional[np.ndarray] = None, y0: Optional[np.ndarray] = None,
              r_max: Optional[int] = None):
    """Oracle output for projection `proj` of a workload (duck-typed, see workloads.Workload).

    Only the adapters used by the evaluated tokens are placed in the oracle's pool.
    """
    p = wl.projections[proj]
    x = wl.x(proj) if x is None else x
    y0 = wl.y0(proj) if y0 is None else y0
    so, sa, ta = wl.seg_offsets, wl.seg_adapter, wl.token_adapter
    T = x.shape[0]
    ev = np.arange(T, dtype=np.int64) if eval_tokens is None else np.asarray(eval_tokens, np.int64)
    # adapters the evaluated tokens need (segment membership by offsets)
    seg_end = int(so[-1])
    need = set()
    for t in ev:
        if t < seg_end:
            s = int(np.searchsorted(so, t, side="right") - 1)
            a = int(sa[s])
        else:
            a = int(ta[t - seg_end])
        if a >= 0 and int(wl.ranks[a]) > 0:
            need.add(a)
    adapters = {a: wl.adapter(a, proj) for a in sorted(need)}
    pool, pt, base = build_pool(adapters, wl.n_adapters, p.d_in, p.d_out, wl.page_elems,
                                wl.dtype, np.random.default_rng(perm_seed))
    if r_max is None:
        r_max = int(wl.ranks.max()) if wl.ranks.size else 0
    return lora(dtype=wl.dtype, d_in=p.d_in, d_out=p.d_out, x=x, y0=y0, pool=pool,
                page_elems=wl.page_elems, page_table=pt, base=base, rank=wl.ranks,
                scale=wl.scales, seg_offsets=so, seg_adapter=sa, token_adapter=ta,
                eval_tokens=None if eval_tokens is None else ev, r_max=r_max,
                want_v=want_v, n_threads=n_threads)
