"""Helpers for the GPU parity tests: move seeded inputs to the device, compare
against the oracle, and report the worst element."""
import sys

import numpy as np

# Tolerances (max abs error vs the float64 oracle on identical input values).
TOL = {"f32": {"o": 1e-5, "lse": 1e-5}, "bf16": {"o": 1e-2, "lse": 1e-3}}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: values are already bf16-representable
    return t.cuda()


def worst(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"non-finite output at {np.argwhere(~np.isfinite(got))[:5].tolist()}"
    err = np.abs(got - want)
    i = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else ()
    return (float(err.max()) if err.size else 0.0), i


def assert_close(name, got, want, tol):
    e, i = worst(got, want)
    g = np.asarray(got)[i] if np.asarray(got).size else None
    w = np.asarray(want)[i] if np.asarray(want).size else None
    say(f"{name}: max|err|={e:.3e} at {tuple(int(x) for x in i)} (got {g}, want {w}), tol {tol:g}")
    assert e <= tol, f"{name}: max abs error {e:.3e} > {tol:g} at {i}: got {g}, want {w}"


# Both workgroup shapes of the bf16 block kernel (4 waves; 8 waves in ping-pong).
SHAPES = (4, 8)



_REF_CACHE = {}


def full_ref(key, q, k, v, scale):
    """The float64 oracle's full attention of q against k, v (every element), computed once per
    key for the whole test session: the full-size workloads are checked element by element by
    several tests, and the 32k ring-4 share alone costs the oracle about 20 s of host time."""
    import oracle
    if key not in _REF_CACHE:
        _REF_CACHE[key] = oracle.attention(q, k, v, scale)
    return _REF_CACHE[key]
