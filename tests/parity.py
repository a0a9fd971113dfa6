"""Comparison helpers for the GPU parity tests (oracle vs HIP library)."""
from __future__ import annotations

import numpy as np

import oracle

REL = 2.0 ** -7      # one bf16 ulp, relative
ABS_RMS = 1e-3       # times rms(ref) over the call's valid outputs


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


def gpu_bits(t) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def within_tolerance(got_bits: np.ndarray, ref_bits: np.ndarray, mask=None, rms_ref=None):
    """|gpu - ref| <= 2^-7 |ref| + 1e-3 rms(ref), per element, over `mask` (all if None).
    Returns (ok, report)."""
    g = bits_to_f64(got_bits)
    r = bits_to_f64(ref_bits)
    if mask is not None:
        g, r = g[mask], r[mask]
    if rms_ref is None:
        rms_ref = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    lim = REL * np.abs(r) + ABS_RMS * rms_ref
    bad = ~(err <= lim)
    eq = float(np.mean(g == r)) if r.size else 1.0
    rep = dict(n=int(r.size), bad=int(bad.sum()), bit_equal=eq,
               max_err_over_lim=float(np.max(err / np.maximum(lim, 1e-300))) if r.size else 0.0,
               rms_ref=rms_ref)
    return (not bad.any()), rep


def assert_close(got_bits, ref_bits, mask=None, rms_ref=None, what=""):
    ok, rep = within_tolerance(got_bits, ref_bits, mask, rms_ref)
    assert ok, "%s: %s" % (what, rep)
    return rep


def assert_bit_exact(got_bits, ref_bits, mask=None, what=""):
    g = got_bits if mask is None else got_bits[mask]
    r = ref_bits if mask is None else ref_bits[mask]
    neq = int(np.sum(g != r))
    assert neq == 0, "%s: %d of %d outputs differ in bits" % (what, neq, r.size)


# ---- full-output reports ---------------------------------------------------------------------

ULP_BUCKETS = ((0, 0, "0"), (1, 1, "1"), (2, 2, "2"), (3, 3, "3"), (4, 7, "4-7"), (8, 15, "8-15"),
               (16, 1 << 30, "16+"))


def ulp_distance(got_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 units in the last place between finite bf16 bit patterns: the patterns
    mapped to a monotonic integer line (sign-magnitude to two's complement, +0 and -0 both 0)."""
    def line(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int32)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(line(got_bits) - line(ref_bits))


def full_report(got_bits, ref_bits, mask=None) -> dict:
    """Over every valid output (mask; all if None): count, share of bit-equal outputs, the bf16
    ulp-distance histogram, the worst error as a fraction of the tolerance and rms(ref)."""
    g = got_bits if mask is None else got_bits[mask]
    r = ref_bits if mask is None else ref_bits[mask]
    ok, rep = within_tolerance(g, r)
    d = ulp_distance(g, r)
    rep["ulp_histogram"] = {name: int(np.sum((d >= lo) & (d <= hi))) for lo, hi, name in ULP_BUCKETS}
    rep["within_tolerance"] = ok
    return rep


def record(name: str, rep: dict) -> None:
    """Print a full-output report; with FP8GEMM_PARITY_REPORT=<path> also append it there as a
    JSON line (for the design notes)."""
    import json
    import os
    line = dict(case=name, **rep)
    print("parity", json.dumps(line), flush=True)
    path = os.environ.get("FP8GEMM_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(line) + "\n")


def assert_close_full(got_bits, ref_bits, mask=None, what=""):
    """assert_close over every valid output of a call (rms over all of them), and record the
    full-output report."""
    rep = full_report(got_bits, ref_bits, mask)
    record(what, rep)
    assert rep["within_tolerance"], "%s: %s" % (what, rep)
    return rep
