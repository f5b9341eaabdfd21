"""Shared helpers for the GPU parity tests (comparison rule, the oracle's own activations)."""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-5


def n_terms(qtype: int, idim: int) -> int:
    """Scale-group terms per output: id/32 (Q4_K sub-blocks, Q4_0 / Q8_0 blocks) or id/16 (Q6_K groups)."""
    return idim // 16 if qtype in (2, 3) else idim // 32


def assert_close(got, ref, mag, qtype: int, idim: int, what: str = ""):
    """|g - o| <= 1e-5 * max(|o|, A / sqrt(n)) elementwise, A = sum of |term|.

    The floor A/sqrt(n) is the typical size of a sum of n terms of random sign; it
    keeps outputs that nearly cancel from failing on f32 rounding noise alone."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.asarray(mag, np.float64)
    tol = REL_TOL * np.maximum(np.abs(ref), mag / np.sqrt(n_terms(qtype, idim)))
    err = np.abs(got - ref)
    bad = err > tol
    if bad.any():
        k = int(np.argmax(err - tol))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at flat {k}: "
                             f"got {got.flat[k]!r} ref {ref.flat[k]!r} err {err.flat[k]:.3e} tol {tol.flat[k]:.3e}")
    rel = err / np.maximum(np.abs(ref), 1e-300)
    return float(np.max(err / np.maximum(tol, 1e-300))), float(np.max(rel))


def oracle_activations(quantize, x, gpu, what: str = ""):
    """The oracle's own quantization of x (quantize: the oracle's per-32 or Q8_K
    quantizer), checked bit-equal to the GPU's activation tensors `gpu`.  The
    reference computations take the oracle's arrays, so no oracle input comes from
    the GPU path."""
    ref = quantize(x)
    for name, g, r in zip(("q", "d", "s"), gpu, ref):
        g = g.cpu().numpy() if hasattr(g, "cpu") else np.asarray(g)
        same = g.dtype == r.dtype and g.shape == r.shape and np.array_equal(g.view(np.uint8), r.view(np.uint8))
        assert same, f"{what}: activation {name} differs from the oracle's"
    return ref
