"""Helpers shared by the GPU parity tests (marshalling and comparison only)."""
import os

import numpy as np

ATOL = 2e-3  # attention output tolerance (max-abs) against the oracle
RTOL = 1e-2  # and relative part: |gpu - oracle| <= ATOL + RTOL * |oracle|
LSE_ATOL = 2e-3


def sweep_count(n):
    """Case count of a seeded random-shape test: n, times the integer in the
    environment variable MPFA_SWEEP_SCALE when it is set (the first n cases
    stay the same, more are drawn after them)."""
    return n * max(1, int(os.environ.get("MPFA_SWEEP_SCALE", "1")))


def say(msg):
    print(msg, flush=True)


def dev(x, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t.to(dtype) if dtype is not None else t


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    if t.dtype == torch.int16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def assert_close(name, got, ref, atol=ATOL, rtol=RTOL, slack=None):
    """|got - ref| <= atol + rtol |ref| (+ slack: the oracle's per-element bound
    on what an equally valid rounding of a P^ value lying on an E4M3 midpoint
    can change, zero almost everywhere)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite GPU values"
    err = np.abs(got - ref)
    tol = atol + rtol * np.abs(ref)
    if slack is not None:
        slack = np.asarray(slack, dtype=np.float64).reshape(got.shape)
        say(f"  {name}: {int((slack > 0).any(axis=-1).sum())} rows hold a P^ rounding on an E4M3 "
            f"midpoint (slack up to {slack.max():.2e})")
        tol = tol + slack
    bad = err > tol
    rel = err / np.maximum(np.abs(ref), 1e-30)
    say(f"  {name}: max_abs={err.max():.3e} max_rel(|ref|>1e-3)="
        f"{rel[np.abs(ref) > 1e-3].max() if (np.abs(ref) > 1e-3).any() else 0:.3e} "
        f"violations={int(bad.sum())}/{bad.size}")
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{name}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={ref[i]!r}")


def assert_bytes_equal(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    diff = got != ref
    say(f"  {name}: {int(diff.sum())} mismatches of {diff.size}")
    if diff.any():
        i = np.argwhere(diff)[0]
        raise AssertionError(f"{name}: {int(diff.sum())} mismatches; first at {tuple(i)}: "
                             f"gpu={got[tuple(i)]!r} oracle={ref[tuple(i)]!r}")
