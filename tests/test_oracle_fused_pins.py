"""Pins for the oracle's producer-side steps (RMS norm, residual add + RMS norm,
silu(g) * u) that feed the quantizer.

Page: "The quantized GEMM" (mojo-dllm kernels page), The GPU path, "Fused
elementwise kernels": each norm and the FFN activation end in the quantizer; the
fused kernels compute the same float expressions in the same order as the chain.
The pages give neither the norm's formula nor its order; the readings (fixed sum
order in f32; silu * u in f64 with one rounding) are checked here against what the
mathematics fixes:

* the sum order, on a row worked by hand (golden): a single running sum, or any
  other order, gives a different last bit;
* the f64 value of the plain definition x / sqrt(mean(x^2) + eps) * w, within the
  error bound of the f32 operations (a wrong mean, a misplaced eps, a wrong weight
  index all exceed it);
* exact special cases: constant rows give +-1, power-of-two scaling of the row
  leaves the norm unchanged, scaling w scales y, a zero row with eps > 0 gives 0;
* silu at points where e^-g is known in closed form (ln 3, -ln 3, ln 7), its
  asymptote g * u, silu(g) - silu(-g) = g, silu(0) = 0, exact scaling in u;
* planted mistakes (OQ_MUTATE 6..9) must fail at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24


def _golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rows[k.strip()] = v.strip()
    return rows


# ---------------------------------------------------------------- pin checks
# Each returns None when the pin holds, else a message.

def pin_rms_sum_order_golden():
    g = _golden("rmsnorm_sum_order.txt")
    n = int(g["n"])
    x = np.zeros((1, n), np.float32)
    x[0, 0] = 4096.0
    x[0, 4:n:4] = 1.0
    y = oracle.rmsnorm(x, np.ones(n, np.float32), 0.0)
    ss = np.float32(float(g["ss"]))
    mean = ss / np.float32(n)
    if float(mean) != float(g["mean"]):
        return "golden file inconsistent"
    r = np.float32(1.0) / np.sqrt(mean)
    want0 = np.float32(4096.0) * r
    if y[0, 0] != want0 or y[0, 4] != r or np.any(y[0, 1:4] != 0):
        return f"sum order: y0 {y[0, 0]!r} != {want0!r} or y4 {y[0, 4]!r} != {r!r}"
    return None


def _rms_f64(x, w, eps):
    x64 = x.astype(np.float64)
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    return x64 / np.sqrt(ms + eps) * w.astype(np.float64)


def pin_rms_f64_bound(cases=((3, 4096, 1e-5), (2, 1056, 0.5), (4, 2048, 1e-6), (1, 32, 0.25))):
    for seed, (nt, n, eps) in enumerate(cases):
        x = synth.activations(nt, n, seed=60 + seed, outlier_frac=0.01)
        w = (1.0 + 0.1 * synth.activations(1, n, seed=70 + seed)[0]).astype(np.float32)
        y = oracle.rmsnorm(x, w, eps).astype(np.float64)
        ref = _rms_f64(x, w, eps)
        # first-order bound of the f32 evaluation: n/256 fused adds per lane, 8 tree
        # levels, the mean, + eps, sqrt (halves), reciprocal, two multiplies
        c = 1.1 * ((n / 256 + 10) / 2 + 4)
        bad = np.abs(y - ref) > c * U * np.abs(ref) + 1e-37
        if np.any(bad):
            k = np.argmax(np.abs(y - ref) / (np.abs(ref) + 1e-30))
            return f"rmsnorm n={n} eps={eps}: |y - f64| too large at {np.unravel_index(k, y.shape)}"
    return None


def pin_rms_exact_cases():
    n = 2080
    w1 = np.ones(n, np.float32)
    for c in (1.0, -8.0, 0.0625, 2.0 ** 20):
        y = oracle.rmsnorm(np.full((1, n), c, np.float32), w1, 0.0)
        if not np.all(y == np.float32(math.copysign(1.0, c))):
            return f"constant row {c} must normalize to +-1"
    x = synth.activations(2, n, seed=80)
    w = synth.activations(1, n, seed=81)[0]
    y = oracle.rmsnorm(x, w, 0.0)
    for k in (-5, 3):
        if not np.array_equal(oracle.rmsnorm(x * np.float32(2.0 ** k), w, 0.0), y):
            return f"norm must be invariant under x -> 2^{k} x"
    if not np.array_equal(oracle.rmsnorm(x, w * np.float32(4.0), 0.0), y * np.float32(4.0)):
        return "y must scale exactly with w"
    if not np.all(oracle.rmsnorm(np.zeros((1, n), np.float32), w, 1e-6) == 0.0):
        return "zero row with eps > 0 must give 0"
    return None


def pin_add_rmsnorm():
    nt, n, eps = 3, 1024, 1e-5
    h = synth.activations(nt, n, seed=82)
    o = synth.activations(nt, n, seed=83)
    w = synth.activations(1, n, seed=84)[0]
    hn, y = oracle.add_rmsnorm(h, o, w, eps)
    if not np.array_equal(hn, h + o):
        return "residual update must be h + o in f32"
    if not np.array_equal(y, oracle.rmsnorm(h + o, w, eps)):
        return "add_rmsnorm must normalize h + o"
    return None


def _silu_taylor(g32, a, sig):
    """silu(g) for g = a + delta (a with sigmoid(a) = sig known exactly), to second
    order in delta: sigma(a + delta) = sig + sig(1 - sig) delta + ..."""
    g = float(g32)
    dl = g - a
    s1 = sig * (1 - sig)
    s2 = s1 * (1 - 2 * sig) / 2
    return g * (sig + s1 * dl + s2 * dl * dl)


def pin_silu_closed_forms():
    pts = [(math.log(3.0), 0.75), (-math.log(3.0), 0.25), (math.log(7.0), 0.875),
           (math.log(1.0 / 7.0), 0.125), (0.0, 0.5)]
    g = np.array([np.float32(a) for a, _ in pts], np.float32)
    y = oracle.silu_mul(g, np.ones_like(g))
    for k, (a, sig) in enumerate(pts):
        want = _silu_taylor(g[k], a, sig)
        if abs(float(y[k]) - want) > U * abs(want) + 1e-45:
            return f"silu({g[k]}) = {y[k]} != {want}"
    return None


def pin_silu_identities():
    g = synth.activations(1, 4096, seed=85)[0] * np.float32(4.0)
    one = np.ones_like(g)
    yp, yn = oracle.silu_mul(g, one), oracle.silu_mul(-g, one)
    err = np.abs(yp.astype(np.float64) - yn.astype(np.float64) - g.astype(np.float64))
    if np.any(err > U * (np.abs(yp) + np.abs(yn)).astype(np.float64) + 1e-45):
        return "silu(g) - silu(-g) must equal g"
    big = np.array([40.0, 57.25, 1e6, 3e30], np.float32)
    u = np.array([1.5, -3.0, 1e-3, 7.0], np.float32)
    if not np.array_equal(oracle.silu_mul(big, u), (big.astype(np.float64) * u).astype(np.float32)):
        return "silu(g) * u must equal g * u for large g"
    if not np.all(oracle.silu_mul(np.zeros(4, np.float32), u) == 0.0):
        return "silu(0) must be 0"
    u2 = synth.activations(1, 4096, seed=86)[0]
    if not np.array_equal(oracle.silu_mul(g, u2 * np.float32(8.0)), oracle.silu_mul(g, u2) * np.float32(8.0)):
        return "silu(g) * u must scale exactly with u"
    return None


FUSED_PINS = [pin_rms_sum_order_golden, pin_rms_f64_bound, pin_rms_exact_cases, pin_add_rmsnorm,
              pin_silu_closed_forms, pin_silu_identities]


# ---------------------------------------------------------------- tests

@pytest.mark.parametrize("pin", FUSED_PINS, ids=[p.__name__ for p in FUSED_PINS])
def test_fused_pin(pin):
    msg = pin()
    assert msg is None, msg


@pytest.mark.parametrize("mutation", [6, 7, 8, 9])
def test_planted_fused_mistakes_are_caught(mutation, tmp_path):
    """RMS mean over n - 1, eps after the square root, one running sum of squares,
    silu with exp(+g): each must fail at least one pin."""
    path = oracle.build(out=str(tmp_path / f"liboracle_m{mutation}.so"), mutate=mutation)
    with oracle.use(path):
        failures = [m for m in (p() for p in FUSED_PINS) if m is not None]
    assert failures, f"mutation {mutation} passed every pin"
    assert all(p() is None for p in FUSED_PINS)
