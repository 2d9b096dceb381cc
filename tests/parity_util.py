"""Shared helpers for the GPU parity tests (comparison gates, row sampling)."""

import numpy as np
import torch

# Tolerances. fp32 inputs: max-abs 1e-5. bf16 inputs with fp32 accumulation:
# max-abs 2e-2 and mean-abs 2e-3 against the fp64 oracle evaluated on the
# bf16-rounded inputs; in addition (outputs can be small, e.g. pointwise
# attention divides by S) a relative gate: ||gpu - ref||_2 / ||ref||_2 <= 1e-2
# and max-abs <= 2e-2 * max|ref|.
F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_L2 = 1e-2
BF16_REL_MAX = 2e-2


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(got, ref, dtype: str, what: str = ""):
    """Assert the gates for ``dtype`` ("f32" or "bf16") and return the errors."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    err = dict(max_abs=float(d.max(initial=0.0)), mean_abs=float(d.mean()) if d.size else 0.0)
    nref = float(np.linalg.norm(ref))
    err["rel_l2"] = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
    if dtype == "f32":
        assert err["max_abs"] <= F32_MAX_ABS, f"{what}: {err}"
    else:
        assert err["max_abs"] <= BF16_MAX_ABS, f"{what}: {err}"
        assert err["mean_abs"] <= BF16_MEAN_ABS, f"{what}: {err}"
        if nref > 0:
            assert err["rel_l2"] <= BF16_REL_L2, f"{what}: {err}"
            assert err["max_abs"] <= BF16_REL_MAX * float(np.abs(ref).max()) + 1e-6, f"{what}: {err}"
    return err


def check_close_grad(got, ref, what: str = ""):
    """bf16 gates for gradients. A gradient entry sums up to S terms (dK, dV
    over queries, dQ over keys) whose weights (P, dS) are rounded to bf16
    (round to nearest even: relative error at most 2^-9) for the matrix
    cores, so its error is about 2^-9 of its size and its size grows with S.
    The gates are therefore relative: rel-L2 <= 1e-2 (about 5x the rounding
    alone) and max-abs <= 2e-2 * max(1, max|ref|); for gradients of size at
    most 1 the second is the forward's max-abs gate."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    d = np.abs(got - ref)
    err = dict(max_abs=float(d.max(initial=0.0)), mean_abs=float(d.mean()) if d.size else 0.0)
    nref = float(np.linalg.norm(ref))
    err["rel_l2"] = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
    amax = float(np.abs(ref).max(initial=0.0))
    assert err["max_abs"] <= BF16_MAX_ABS * max(1.0, amax), f"{what}: {err}"
    if nref > 0:
        assert err["rel_l2"] <= BF16_REL_L2, f"{what}: {err}"
    else:
        assert err["max_abs"] == 0.0, f"{what}: {err}"
    return err


def sample_rows(rng, B, H, S, n, extra=()):
    """(b, h, q) triples: n random ones plus the first and last rows and any
    ``extra`` query positions, on random (b, h)."""
    out = set()
    for qpos in (0, S - 1, *extra):
        out.add((int(rng.integers(B)), int(rng.integers(H)), int(qpos)))
    while len(out) < n + 2 + len(extra):
        out.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(S))))
    return sorted(out)
