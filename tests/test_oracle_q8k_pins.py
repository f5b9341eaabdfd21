"""Pins for the oracle's Q8_K path (activations with one scale per 256 values and
16-value code sums), checked against what the pages and plain mathematics fix.

Page: "The quantized GEMM" (mojo-dllm kernels page), "Activations: int8 with a
scale per 256" and "The zero points do not touch the inner loop": one f32 scale per
256 activations, the sum of each 16-value group kept, and the Q4_K min term
dmin * m times the sub-block's activation sum taken from those sums.

* crafted blocks worked by hand (golden): scale, rounding mode, group sums;
* invariants: the largest magnitude maps to +-127, the rounding bound, sign
  symmetry, power-of-two scaling, group sums equal the code sums;
* the fold identity: the oracle equals the f64 product of the dequantized weights
  (independent element-indexed decoder) with dx * qx, to f64 rounding -- the group
  sums are exact, so no stored rounding enters;
* the activation-quantization bound against the f64 product with x itself;
* planted mistakes (scale from the first 32 values; min term from half the sums)
  must fail a pin.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q4, Q6, Q5 = oracle.TYPE_Q4_K, oracle.TYPE_Q6_K, oracle.TYPE_Q5_K


def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "quantize_q8k_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rows[k.strip()] = v.split()
    return rows


def _golden_blocks():
    a = np.where(np.arange(256) % 2 == 0, 2.5, -2.5).astype(np.float32)
    a[0] = 127.0
    b = np.where(np.arange(256) < 128, 1.25, 0.75).astype(np.float32)
    b[255] = -63.5
    c = np.zeros(256, np.float32)
    return np.stack([a, b, c])


def pin_q8k_golden():
    g = _golden()
    q, d, bs = oracle.quantize_q8k(_golden_blocks())
    for k, name in enumerate("ABC"):
        if float(d[k, 0]) != float(g[f"{name}.d"][0]):
            return f"block {name}: d {d[k, 0]} != {g[name + '.d'][0]}"
        want = [float(v) for v in g[f"{name}.bsum"]]
        if list(bs[k]) != want:
            return f"block {name}: group sums {list(bs[k])} != {want}"
    return None


def _fold_case(qtype, od, idim, nt, seed):
    W = synth.weights(qtype, od, idim, seed=seed)
    x = synth.activations(nt, idim, seed=seed, outlier_frac=0.02)
    q, d, bs = oracle.quantize_q8k(x)
    out, mag = oracle.matmul_q8k(qtype, W, q, d, bs, od)
    Wd = bf.dequant(qtype, W, od, idim)
    xd = np.repeat(d.astype(np.float64), 256, axis=1) * q.astype(np.float64)
    return W, x, (q, d, bs), out, mag, Wd, xd


def pin_q8k_fold_identity():
    for qtype in (Q4, Q6, Q5):
        for seed in (1, 2):
            _, _, _, out, mag, Wd, xd = _fold_case(qtype, 6, 768, 3, 20 + seed)
            ref = xd @ Wd.T
            err = np.abs(out.astype(np.float64) - ref)
            if not np.all(err <= 2.0 ** -24 * np.abs(ref) + 1e-12 * mag):
                return f"type {qtype}: Q8_K fold identity fails by {float(np.max(err)):.3e}"
    return None


def pin_q8k_quantization_bound():
    for qtype in (Q4, Q6, Q5):
        _, x, (q, d, bs), out, mag, Wd, _ = _fold_case(qtype, 5, 1024, 4, 30)
        exact = x.astype(np.float64) @ Wd.T
        absW = np.abs(Wd).reshape(Wd.shape[0], -1, 256).sum(axis=2)
        act = (d.astype(np.float64) * (0.5 + 2.0 ** -17)) @ absW.T
        bound = act + 2.0 ** -24 * np.abs(out) + 1e-12 * mag
        if not np.all(np.abs(out.astype(np.float64) - exact) <= bound):
            return f"type {qtype}: error exceeds the activation quantization bound"
    return None


Q8K_PINS = [pin_q8k_golden, pin_q8k_fold_identity, pin_q8k_quantization_bound]


@pytest.mark.parametrize("pin", Q8K_PINS, ids=[p.__name__ for p in Q8K_PINS])
def test_q8k_pin(pin):
    msg = pin()
    assert msg is None, msg


@pytest.mark.parametrize("seed,scale", [(1, 1.0), (2, 1e-3), (3, 50.0)])
def test_q8k_invariants(seed, scale):
    x = (synth.activations(3, 1024, seed=seed, outlier_frac=0.01) * np.float32(scale)).astype(np.float32)
    q, d, bs = oracle.quantize_q8k(x)
    xb = x.reshape(3, 4, 256)
    qb = q.reshape(3, 4, 256).astype(np.int32)
    k = np.argmax(np.abs(xb), axis=2)
    qmax = np.take_along_axis(qb, k[..., None], axis=2)[..., 0]
    xmax = np.take_along_axis(xb, k[..., None], axis=2)[..., 0]
    assert np.all(qmax == np.where(xmax > 0, 127, -127)) and np.all(np.abs(qb) <= 127)
    err = np.abs(xb.astype(np.float64) - d.reshape(3, 4, 1).astype(np.float64) * qb)
    assert np.all(err <= d.reshape(3, 4, 1).astype(np.float64) * (0.5 + 2.0 ** -17))
    assert np.array_equal(bs, q.reshape(3, -1, 16).astype(np.int32).sum(axis=2).astype(np.float32))
    qn, dn, bn = oracle.quantize_q8k(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d) and np.array_equal(bn, -bs)
    if scale >= 1.0:
        q2, d2, b2 = oracle.quantize_q8k((x * np.float32(0.25)).astype(np.float32))
        assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(0.25)) and np.array_equal(b2, bs)


def test_q8k_points_match_full():
    od, idim, nt = 7, 512, 3
    for qtype in (Q4, Q6, Q5):
        W, _, (q, d, bs), out, mag, _, _ = _fold_case(qtype, od, idim, nt, 40)
        t = np.array([0, 2, 1], np.int32)
        r = np.array([6, 0, 3], np.int32)
        po, pm = oracle.matmul_q8k_points(qtype, W, q, d, bs, od, t, r)
        assert np.array_equal(po, out[t, r]) and np.array_equal(pm, mag[t, r])


@pytest.mark.parametrize("qtype", [Q4, Q6, Q5])
def test_q8k_superblock_sums_brute_force(qtype):
    """The integer stage from the element-indexed decoder and plain Python sums."""
    od, idim, nt = 3, 512, 2
    W, _, (q, d, bs), *_ = _fold_case(qtype, od, idim, nt, 50)
    S = oracle.q8k_superblock_sums(qtype, W, q, bs, od)
    bb = {Q4: 144, Q6: 210, Q5: 176}[qtype]
    Wb = W.reshape(od, idim // 256, bb)
    for t in range(nt):
        for r in range(od):
            for b in range(idim // 256):
                blk = Wb[r, b]
                qx = q[t, 256 * b: 256 * b + 256].astype(np.int64)
                if qtype in (Q4, Q5):
                    code = bf.q4k_code if qtype == Q4 else bf.q5k_code
                    codes = np.array([code(blk, e) for e in range(256)], np.int64)
                    scm = [bf.q4k_field(blk, j) for j in range(8)]
                    s1 = sum(scm[j][0] * int(np.dot(codes[32 * j: 32 * j + 32], qx[32 * j: 32 * j + 32]))
                             for j in range(8))
                    s2 = sum(scm[j][1] * int(bs[t, 16 * b + 2 * j] + bs[t, 16 * b + 2 * j + 1]) for j in range(8))
                else:
                    codes = np.array([bf.q6k_code(blk, e) for e in range(256)], np.int64)
                    sc = blk[192:208].view(np.int8).astype(np.int64)
                    s1 = sum(int(sc[g]) * int(np.dot(codes[16 * g: 16 * g + 16] - 32, qx[16 * g: 16 * g + 16]))
                             for g in range(16))
                    s2 = 0
                assert (S[t, r, b, 0], S[t, r, b, 1]) == (s1, s2), (t, r, b)


@pytest.mark.parametrize("mutation", [10, 11])
def test_planted_q8k_mistakes_are_caught(mutation, tmp_path):
    path = oracle.build(out=str(tmp_path / f"liboracle_m{mutation}.so"), mutate=mutation)
    with oracle.use(path):
        failures = [m for m in (p() for p in Q8K_PINS) if m is not None]
    assert failures, f"mutation {mutation} passed every pin"
    assert all(p() is None for p in Q8K_PINS)
