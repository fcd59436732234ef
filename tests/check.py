"""Comparison helpers for GPU results against the oracle.

Tolerance (bf16 output, fp32 accumulation in a different order than the
oracle's exact fp64 sums): |d - ref| <= 8e-3 * |ref| + 1e-3 * max|ref|, with
ref the oracle's bf16 value and max|ref| taken over the compared elements.
Adjacent bf16 values are at most 2^-7 |ref| apart, so one-ulp disagreements
always pass; the absolute term covers cancellation near zero.
"""
import numpy as np

REL = 8e-3
ABS_OF_MAX = 1e-3
SENTINEL = 0x7FA5   # a bf16 NaN payload no kernel writes


def bf16_to_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tolerance_report(d_bits, ref_bits):
    d = bf16_to_f64(d_bits).ravel()
    r = bf16_to_f64(ref_bits).ravel()
    nan_r, nan_d = np.isnan(r), np.isnan(d)
    finite = ~nan_r & ~nan_d
    maxref = np.abs(r[finite]).max() if finite.any() else 0.0
    tol = REL * np.abs(r) + ABS_OF_MAX * maxref
    err = np.abs(d - r)
    bad = (nan_r != nan_d) | (finite & (err > tol))
    ulp = np.abs(np.asarray(d_bits).astype(np.int64).ravel() - np.asarray(ref_bits).astype(np.int64).ravel())
    return dict(n=int(d.size), bad=int(bad.sum()), max_err_over_tol=float(np.max(err[finite] / tol[finite])) if finite.any() else 0.0,
                exact=int((ulp == 0).sum()), le1ulp=int((ulp <= 1).sum()), maxref=float(maxref),
                first_bad=(np.nonzero(bad)[0][:5].tolist()))


def assert_close(d_bits, ref_bits, what=""):
    rep = tolerance_report(d_bits, ref_bits)
    assert rep["bad"] == 0, "%s: %d of %d elements out of tolerance: %s" % (what, rep["bad"], rep["n"], rep)
    return rep
