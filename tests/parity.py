"""Shared helpers of the GPU parity tests (compare against the CPU oracle).

Tolerances (per output, error scale S = sum_k |x w| + |residual|):
  * path 0 (f32 GEMV) and path 1 (split-f16 matrix cores): |gpu - ref| <= 1e-5 S
  * path 2 (f16 matrix cores): |gpu - ref| <= 2e-3 S and, per output row with
    a non-zero reference, cosine(gpu, ref) >= 0.99999 in float64.

Fused gate/up + SwiGLU (``check_swiglu``): with g and u each within the
path's tol * S of the exact projections, the output is within tol * E of the
exact silu(g) * u, E = 1.1 Sg (|u| + tol Su) + |silu(g)| Su (the oracle's
gate_up_swiglu_error_scale; 1.1 bounds silu's slope).  The f32 epilogue adds
a few roundings (exp, divide, multiply: under 1e-6 of the f32 result, whose
size is at most |ref| + tol * E), so the bar is
|gpu - ref| <= tol * E * (1 + 1e-6) + 1e-6 |ref|, plus the row cosine on path 2.
"""

import numpy as np

TOL = {0: 1e-5, 1: 1e-5, 2: 2e-3}
COS_MIN = 0.99999


def check(gpu, ref, s, path, label=""):
    """Return (ok, message).  ``gpu`` f32, ``ref``/``s`` float64, same shape."""
    gpu64 = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
    if not np.all(np.isfinite(gpu64)):
        return False, "%s: non-finite outputs" % label
    err = np.abs(gpu64 - ref)
    tol = TOL[path]
    bad = err > tol * s
    worst = float(np.max(err / np.maximum(s, 1e-300))) if err.size else 0.0
    if bad.any():
        idx = np.argwhere(bad)[0]
        return False, ("%s: %d of %d outputs exceed %g*S (worst err/S %.3g; first at %s: gpu %r "
                       "ref %r S %r)" % (label, int(bad.sum()), bad.size, tol, worst, tuple(idx),
                                         gpu64[tuple(idx)], ref[tuple(idx)], s[tuple(idx)]))
    if path == 2 and ref.ndim == 2:
        num = np.sum(gpu64 * ref, axis=1)
        den = np.linalg.norm(gpu64, axis=1) * np.linalg.norm(ref, axis=1)
        rows = np.linalg.norm(ref, axis=1) > 0
        cos = num[rows] / np.maximum(den[rows], 1e-300)
        if cos.size and cos.min() < COS_MIN:
            return False, "%s: row cosine %.8f < %g" % (label, float(cos.min()), COS_MIN)
    return True, "%s: ok (worst err/S %.3g)" % (label, worst)


SWIGLU_F32_REL = 1e-6


def check_swiglu(gpu, ref, e, path, label=""):
    """Return (ok, message) for the fused gate/up + SwiGLU output; ``e`` is the
    oracle's error scale computed with this path's tolerance."""
    gpu64 = np.asarray(gpu, dtype=np.float64).reshape(ref.shape)
    if not np.all(np.isfinite(gpu64)):
        return False, "%s: non-finite outputs" % label
    err = np.abs(gpu64 - ref)
    bound = TOL[path] * e * (1 + SWIGLU_F32_REL) + SWIGLU_F32_REL * np.abs(ref)
    bad = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    if bad.any():
        idx = np.argwhere(bad)[0]
        return False, ("%s: %d of %d outputs exceed the bound (worst err/bound %.3g; first at "
                       "%s: gpu %r ref %r bound %r)" % (label, int(bad.sum()), bad.size, worst,
                                                         tuple(idx), gpu64[tuple(idx)],
                                                         ref[tuple(idx)], bound[tuple(idx)]))
    if path == 2 and ref.ndim == 2 and ref.shape[1] > 1:
        num = np.sum(gpu64 * ref, axis=1)
        den = np.linalg.norm(gpu64, axis=1) * np.linalg.norm(ref, axis=1)
        rows = np.linalg.norm(ref, axis=1) > 0
        cos = num[rows] / np.maximum(den[rows], 1e-300)
        if cos.size and cos.min() < COS_MIN:
            return False, "%s: row cosine %.8f < %g" % (label, float(cos.min()), COS_MIN)
    return True, "%s: ok (worst err/bound %.3g)" % (label, worst)
