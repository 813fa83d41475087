"""Helpers for the GPU tests: run the HIP path through libslora, compare with the oracle."""

import sys

import numpy as np

import oracle
import workloads

TOL = 5e-3  # max|y - y_ref| <= TOL * max(1, ||y_ref||_inf), fp16/bf16 in, fp32 accumulation


def decode(bits, dtype):
    bits = np.asarray(bits).view(np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check_close(y_gpu_bits, y_ref, dtype, what=""):
    y = decode(y_gpu_bits, dtype)
    assert y.shape == y_ref.shape, (y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite GPU output at {np.argwhere(~np.isfinite(y))[:5]}"
    scale = max(1.0, float(np.max(np.abs(y_ref))))
    err = float(np.max(np.abs(y - y_ref)))
    assert err <= TOL * scale, f"{what}: max err {err:.3e} > {TOL} * {scale:.3f}"
    return err / scale


def assert_same_to_rounding(got, want, dtype, what=""):
    """Two GPU results of one computation whose fp32 sums were grouped differently, as
    storage-type bit patterns, element by element:
    |got - want| <= ulp(want) + 2^-12 * max(1, max|want|). The grouping moves an fp32 sum
    by a relative 2^-22 or so; v entries that the segment expand reads rounded to the
    storage type can round the other way, which moves y by about 1e-5 at the workloads'
    value scales (far below 2^-12); y's own rounding can then land one unit away. A wrong
    row, column or projection moves an output by the size of the LoRA term (~5e-2) and
    fails."""
    g, w = decode(got, dtype), decode(want, dtype)
    wb = np.asarray(want).view(np.uint16)
    nxt = ((wb & 0x8000) | ((wb & 0x7FFF) + 1)).astype(np.uint16)  # next value away from 0
    ulp = np.abs(decode(nxt, dtype) - w)
    bound = ulp + 2.0 ** -12 * max(1.0, float(np.abs(w).max(initial=0.0)))
    excess = np.abs(g - w) - bound
    assert float(excess.max(initial=-1.0)) <= 0.0, (what, float(np.abs(g - w).max()),
                                                     int((np.asarray(got) != np.asarray(want)).sum()))


def margin_line(what, rel):
    """One greppable line per parity check: max|y - y_ref| / max(1, ||y_ref||_inf) and the
    tolerance, so the margins of every workload and routing policy are on record."""
    say(f"[margin] {what}: max_err/scale={rel:.3e} tol={TOL:.0e} ratio={rel / TOL:.3f}")


def full_rows_rel(y_gpu_bits, wl, proj, dtype, what, chunk=2048, n_threads=16):
    """Every output row against the oracle, in chunks of rows to bound host memory.
    The tolerance is the global one: max over all rows of |y - y_ref| against
    TOL * max(1, max over all rows of |y_ref|)."""
    T = wl.n_tokens
    err, ref_max = 0.0, 0.0
    for c0 in range(0, T, chunk):
        ev = np.arange(c0, min(T, c0 + chunk), dtype=np.int64)
        ref, _ = oracle.reference(wl, proj, ev, n_threads=n_threads)
        y = decode(y_gpu_bits[ev], dtype)
        assert np.all(np.isfinite(y)), f"{what}: non-finite GPU output in rows {c0}.."
        err = max(err, float(np.max(np.abs(y - ref))))
        ref_max = max(ref_max, float(np.max(np.abs(ref))))
    scale = max(1.0, ref_max)
    assert err <= TOL * scale, f"{what}: max err {err:.3e} > {TOL} * {scale:.3f}"
    return err / scale


def sample_tokens(wl, n, seed=0):
    """Evaluation rows: ends of every segment (ragged tails), both ends of the batch, random rest."""
    T = wl.n_tokens
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    so = wl.seg_offsets
    for s in range(len(wl.seg_adapter)):
        if so[s + 1] > so[s]:
            pick.update([int(so[s]), int(so[s + 1]) - 1])
    pick.update(int(t) for t in rng.choice(T, size=min(n, T), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


class CodedWorkload(workloads.Workload):
    """Adapter weights replaced by exact small-integer codes (probe tests).

    Element j of A^T row k of adapter a, projection p, is code(a, p, k, j); B rows
    use a second code. |codes| <= 120, exact in fp16 and bf16.
    """

    @staticmethod
    def code(a, p, k, j, half):
        return ((a * 37 + p * 11 + k * 7 + j * 3 + half * 5) % 241) - 120

    def adapter(self, adapter_id, proj):
        p = self.projections[proj]
        r = int(self.ranks[adapter_id])
        k = np.arange(r)[:, None]
        at = self.code(adapter_id, proj, k, np.arange(p.d_in)[None, :], 0).astype(np.float32)
        b = self.code(adapter_id, proj, k, np.arange(p.d_out)[None, :], 1).astype(np.float32)
        return workloads.to_bits(at, self.dtype), workloads.to_bits(b, self.dtype)


def coded(wl):
    c = CodedWorkload(**{f: getattr(wl, f) for f in wl.__dataclass_fields__ if f != "_cache"})
    return c


def oracle_ref(wl, proj, eval_tokens=None, want_v=False, x=None, y0=None, n_threads=8):
    return oracle.reference(wl, proj, eval_tokens, want_v=want_v, x=x, y0=y0, n_threads=n_threads)
