"""Comparison of HIP outputs with the fp64 oracle.

Two bounds, both required:

* elementwise ``|gpu - ref| <= atol + rtol * |ref|``: atol 2e-2 / rtol 1e-2
  for a bf16 pool (the bounds test_verify_splitkv.py uses against its
  single-pass baseline, ATOL / RTOL), atol 3e-2 for an fp8 pool (the extra
  room the E4M3 query rounding and the 8-bit value rows take);
* relative L2 over the compared values, ``||gpu - ref||_2 <= 1e-2 *
  ||ref||_2``.  At long context the outputs are averages of thousands of
  unit-variance values, so their magnitude is ~1e-2 and the absolute bound
  alone would accept an all-zero output.  The relative bound follows from
  the arithmetic: the bf16 output store rounds each value to within 2^-9 of
  itself, the bf16 partial outputs and bf16 probabilities add at most two more
  such roundings, so the path's relative error stays below 3 * 2^-9 ~ 6e-3.

``tests/test_parity_checker.py`` pins the checker on the CPU: the oracle's own
output rounded to bf16 passes; an all-zero output, a halved output and the
output of a batch with one range dropped fail.
"""
import numpy as np

BF16_TOL = dict(atol=2e-2, rtol=1e-2, rel_l2=1e-2)
FP8_TOL = dict(atol=3e-2, rtol=1e-2, rel_l2=1e-2)


def compare(got: np.ndarray, ref: np.ndarray, tol):
    """(elementwise ok, relative-L2 ok, max abs err, relative L2 err)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    elem_ok = bool(np.isfinite(got).all()) and not (err > tol["atol"] + tol["rtol"] * np.abs(ref)).any()
    nref = float(np.linalg.norm(ref))
    nerr = float(np.linalg.norm(got - ref)) if np.isfinite(got).all() else float("inf")
    rel = nerr / nref if nref > 0 else (0.0 if nerr == 0 else float("inf"))
    # an all-zero reference (rows that see no key) must be matched exactly
    l2_ok = nerr <= tol["rel_l2"] * nref if nref > 0 else nerr == 0
    return elem_ok, l2_ok, (float(err.max()) if err.size else 0.0), rel


def assert_close(gpu, ref: np.ndarray, tol, what="", mask=None):
    """Check a GPU tensor against the oracle's array; returns the max abs err."""
    g = gpu.float().cpu().double().numpy() if hasattr(gpu, "cpu") else np.asarray(gpu, np.float64)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    assert np.isfinite(g).all(), what + ": non-finite GPU output"
    elem_ok, l2_ok, worst, rel = compare(g, ref, tol)
    print("%s: max abs err %.3e, relative L2 err %.3e over %d values" % (what, worst, rel, g.size),
          flush=True)
    if not elem_ok:
        err = np.abs(g - ref)
        bad = err > tol["atol"] + tol["rtol"] * np.abs(ref)
        raise AssertionError("%s: %d/%d values out of tolerance, max abs err %.3e"
                             % (what, int(bad.sum()), bad.size, worst))
    assert l2_ok, "%s: relative L2 error %.3e above %.1e" % (what, rel, tol["rel_l2"])
    return worst
