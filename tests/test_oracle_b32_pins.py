"""Pins for the oracle's 32-weight block formats Q4_0 and Q8_0, checked against
what the pages and plain arithmetic fix.

Pages: "03 - Reading minfer's kernels I -- elementwise, dequant, embedding", section
3.2 (the Q4_0 block: f16 scale, 16 bytes of nibbles, element l in the low and
element l + 16 in the high nibble of byte l, value d * (nibble - 8)); "04 - Reading
minfer's kernels II", section 3.4 (the Q4_0 x q8 dot: d8 * d4 * (dot - 8 * sx), the
offset folded through the activation sum).  Q8_0's layout is a reading (f16 d then
32 int8 codes).

* blocks worked by hand (golden): field positions, nibble order, the offset 8;
* the decoder against an independent element-indexed decoder (tests/bruteforce.py);
* integer dots by brute force; the fold identity against the f64 product of the
  dequantized weights with dx * qx; the activation-quantization bound;
* planted mistakes (offset dropped, nibbles read interleaved) must fail a pin.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q40, Q80 = oracle.TYPE_Q4_0, oracle.TYPE_Q8_0


def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "block32_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rows[k.strip()] = v.split()
    return rows


def _group_from(qtype, block_bytes):
    """A group of eight copies of one block (the oracle reads groups of eight)."""
    return np.tile(np.array(block_bytes, np.uint8), 8)


def pin_golden_blocks():
    g = _golden()
    for name, qtype in (("A", Q40), ("B", Q80)):
        blk = [int(b, 16) for b in g[f"{name}.bytes"]]
        d, codes = oracle.decode_group32(qtype, _group_from(qtype, blk))
        w = d[0] * codes[:32]
        want = np.array([float(v) for v in g[f"{name}.w"]])
        if not np.array_equal(w, want):
            return f"block {name}: {list(w)} != {list(want)}"
    return None


def pin_decoder_brute_force():
    for qtype in (Q40, Q80):
        W = synth.weights(qtype, 3, 512, seed=70 + qtype)
        gb = 144 if qtype == Q40 else 272
        for gi in range(6):
            grp = W[gb * gi: gb * gi + gb]
            d, codes = oracle.decode_group32(qtype, grp)
            got = np.repeat(d, 32) * codes
            ref = np.array([bf.b32_weight(qtype, grp, e) for e in range(256)])
            if not np.array_equal(got, ref):
                return f"type {qtype} group {gi}: decoder differs from the element rule"
    return None


def _case(qtype, od, idim, nt, seed):
    W = synth.weights(qtype, od, idim, seed=seed)
    x = synth.activations(nt, idim, seed=seed, outlier_frac=0.02)
    out, mag, (q, d, s) = oracle.matmul(qtype, W, x, od)
    Wd = bf.b32_dequant(qtype, W, od, idim)
    return W, x, q, d, out, mag, Wd


def pin_fold_identity():
    for qtype in (Q40, Q80):
        W, x, q, d, out, mag, Wd = _case(qtype, 4, 512, 3, 80 + qtype)
        xd = np.repeat(d.astype(np.float64), 32, axis=1) * q.astype(np.float64)
        ref = xd @ Wd.T
        if not np.all(np.abs(out.astype(np.float64) - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-12 * mag):
            return f"type {qtype}: fold identity fails"
    return None


def pin_group_dots():
    for qtype in (Q40, Q80):
        od, idim, nt = 2, 512, 2
        W, x, q, d, *_ = _case(qtype, od, idim, nt, 90 + qtype)
        S = oracle.subblock_dots(qtype, W, q, od)
        gb = 144 if qtype == Q40 else 272
        G = W.reshape(od, idim // 256, gb)
        for t in range(nt):
            for r in range(od):
                for b in range(idim // 256):
                    for j in range(8):
                        want = sum(bf.b32_code(qtype, G[r, b], 32 * j + l) * int(q[t, 256 * b + 32 * j + l])
                                   for l in range(32))
                        if S[t, r, b, j] != want:
                            return f"type {qtype}: dot ({t},{r},{b},{j}) {S[t, r, b, j]} != {want}"
    return None


B32_PINS = [pin_golden_blocks, pin_decoder_brute_force, pin_fold_identity, pin_group_dots]


@pytest.mark.parametrize("pin", B32_PINS, ids=[p.__name__ for p in B32_PINS])
def test_b32_pin(pin):
    msg = pin()
    assert msg is None, msg


@pytest.mark.parametrize("qtype", [Q40, Q80])
def test_b32_quantization_bound(qtype):
    W, x, q, d, out, mag, Wd = _case(qtype, 5, 1024, 4, 100 + qtype)
    exact = x.astype(np.float64) @ Wd.T
    absW = np.abs(Wd).reshape(Wd.shape[0], -1, 32).sum(axis=2)
    act = (d.astype(np.float64) * (0.5 + 2.0 ** -17)) @ absW.T
    assert np.all(np.abs(out.astype(np.float64) - exact) <= act + 2.0 ** -24 * np.abs(out) + 1e-12 * mag)


@pytest.mark.parametrize("mutation", [12, 13])
def test_planted_b32_mistakes_are_caught(mutation, tmp_path):
    path = oracle.build(out=str(tmp_path / f"liboracle_m{mutation}.so"), mutate=mutation)
    with oracle.use(path):
        failures = [m for m in (p() for p in B32_PINS) if m is not None]
    assert failures, f"mutation {mutation} passed every pin"
    assert all(p() is None for p in B32_PINS)
