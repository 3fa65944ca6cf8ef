"""Helpers for the GPU parity tests: device copies and the tolerances.

Tolerances (written out here, used by every GPU test):
  fp32 path:  |gpu - oracle| <= 1e-5 * |oracle| + 1e-5 * rms(oracle), element-wise
              (relative 1e-5; the rms term keeps outputs near zero from
              demanding more than float32 can hold);
  bf16 value: |gpu - oracle| <= 1e-2 absolute (unit-scale data, fp32 accumulation);
  bf16 projection output: |gpu - oracle| <= 2^-7 * |oracle| + 1e-5 (one bf16
              unit in the last place: fp32 accumulation may move a value
              across a rounding boundary of the final bf16 rounding);
  integers (hit counts, pair lists): bit-exact;
  scatter-accumulated sums (value gradients, summed with float32 atomics
              in no fixed order over up to ~10^3 contributions per element):
              |gpu - oracle| <= 1e-5 * (m + rms(m)), m = the element's sum of
              its contributions' magnitudes.  Float32 summation error is
              relative to what is summed, not to the possibly cancelled total;
              the rms term plays the part it plays in the fp32 bar: each
              contribution alpha * w * g carries an absolute error of about
              3e-8 * alpha * |g| from the float32 interpolation weight, so an
              element fed only by a few small-weight corners cannot meet a
              bound relative to its own small sum.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


def announce(msg):
    """Name the case on the real stderr before a GPU step (survives capture)."""
    sys.__stderr__.write(f"[gpu case] {msg}\n")
    sys.__stderr__.flush()


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_fp32_close(got, ref, what):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = np.abs(got - ref)
    tol = 1e-5 * np.abs(ref) + 1e-5 * rms
    bad = err > tol
    nrm = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} elements beyond 1e-5 rel; max err "
                           f"{err.max():.3g} at ref {ref[np.argmax(err)]:.4g}; rms {rms:.3g}; normwise {nrm:.3g}")
    return nrm


def assert_abs_close(got, ref, atol, what):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    assert not (err > atol).any(), f"{what}: max abs err {err.max():.3g} > {atol}"
    return float(err.max()) if err.size else 0.0


def assert_bf16_ulp_close(got_bits, ref, what):
    got = bf16_bits_to_f64(got_bits).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    err = np.abs(got - ref)
    tol = 2.0 ** -7 * np.abs(ref) + 1e-5
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())}/{bad.size} beyond one bf16 ulp; max err {err.max():.3g}"


def assert_sum_close(got, ref, abs_sum, what):
    """Scatter-accumulated sums: |got - ref| <= 1e-5 * (abs_sum + rms(abs_sum))
    element-wise, abs_sum = the sum of the magnitudes of each element's
    contributions; elements with no contribution must be exactly zero."""
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    abs_sum = np.asarray(abs_sum, np.float64).reshape(-1)
    assert got.shape == ref.shape == abs_sum.shape, (what, got.shape, ref.shape, abs_sum.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    assert not got[abs_sum == 0].any(), f"{what}: nonzero where nothing contributes"
    rms = float(np.sqrt(np.mean(abs_sum ** 2))) if abs_sum.size else 0.0
    tol = 1e-5 * (abs_sum + rms)
    bad = err > tol
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} elements beyond the bar (worst err/tol "
                           f"{worst:.3g}; rms of the magnitudes {rms:.3g})")
    return worst


def oracle_by_rows(fn, rows, threads=None):
    """The oracle over many rows at once: fn(chunk) -> array [len(chunk), ...]
    for contiguous chunks of `rows`, run on the host's cores (ctypes releases
    the interpreter lock while the C oracle runs), stacked in row order."""
    n = threads or min(16, len(os.sched_getaffinity(0)))
    rows = np.asarray(rows, np.int64)
    chunks = [c for c in np.array_split(rows, 4 * n) if len(c)]
    with ThreadPoolExecutor(n) as ex:
        return np.concatenate(list(ex.map(fn, chunks)))
