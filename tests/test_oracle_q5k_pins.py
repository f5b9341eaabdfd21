"""Pins for the oracle's Q5_K reading (the public block layout; the pages name the
type only, so this reading is pinned by internal consistency, a block worked by
hand from the reading, and special cases -- parity unpinned by the pages).

* the hand-worked block (golden): field positions, the fifth bit, code = nibble + 16 bit;
* the decoder against an independent element-indexed decoder (tests/bruteforce.py);
* the fold identity against the f64 product of the dequantized weights with dx * qx
  (within the rounding of the stored activation sums), integer dots by brute force;
* with every high bit zero, Q5_K gives exactly the Q4_K result of the same scales and
  nibbles;
* a planted mistake (high bit dropped) must fail a pin.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q5, Q4 = oracle.TYPE_Q5_K, oracle.TYPE_Q4_K


def _golden_block():
    rows = {}
    with open(os.path.join(GOLDEN, "q5k_block_worked.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rows[k.strip()] = v.split()
    blk = np.zeros(176, np.uint8)
    blk[:16] = [int(b, 16) for b in rows["bytes"]]
    blk[16:48] = int(rows["high"][0], 16)
    blk[48:80] = int(rows["chunk0"][0], 16)
    want = []
    for item in rows["w"]:
        v, n = item.split("x")
        want += [float(v)] * int(n)
    return blk, np.array(want)


def pin_q5k_golden():
    blk, want = _golden_block()
    dec = oracle.decode_block(Q5, blk)
    w = dec["d"] * np.repeat(dec["sc"], 32) * dec["codes"] - dec["dmin"] * np.repeat(dec["m"], 32)
    if not np.array_equal(w, want):
        return "hand-worked Q5_K block decodes differently"
    return None


def pin_q5k_brute_force():
    W = synth.weights(Q5, 3, 512, seed=110).reshape(-1, 176)
    for b in range(W.shape[0]):
        dec = oracle.decode_block(Q5, W[b])
        if list(dec["codes"]) != [bf.q5k_code(W[b], e) for e in range(256)]:
            return f"block {b}: codes differ from the element rule"
    return None


def pin_q5k_fold_identity():
    od, idim, nt = 4, 512, 3
    W = synth.weights(Q5, od, idim, seed=111)
    x = synth.activations(nt, idim, seed=111, outlier_frac=0.02)
    out, mag, (q, d, s) = oracle.matmul(Q5, W, x, od)
    Wd = bf.dequant(Q5, W, od, idim)
    ref = (np.repeat(d.astype(np.float64), 32, axis=1) * q.astype(np.float64)) @ Wd.T
    # the min term uses the stored s = f32(d * sum q): allow its rounding
    if not np.all(np.abs(out - ref) <= 2.0 ** -22 * (np.abs(ref) + mag) + 1e-12):
        return "Q5_K fold identity fails"
    S = oracle.subblock_dots(Q5, W, q, od)
    G = W.reshape(od, idim // 256, 176)
    for t in range(nt):
        for r in range(od):
            for b in range(idim // 256):
                for j in range(8):
                    want = sum(bf.q5k_code(G[r, b], 32 * j + l) * int(q[t, 256 * b + 32 * j + l]) for l in range(32))
                    if S[t, r, b, j] != want:
                        return "Q5_K integer dots differ from brute force"
    return None


def pin_q5k_no_high_bits_is_q4k():
    W5 = synth.weights(Q5, 5, 768, seed=112).reshape(-1, 176).copy()
    W5[:, 16:48] = 0
    W4 = np.concatenate([W5[:, :16], W5[:, 48:]], axis=1).reshape(-1)
    x = synth.activations(2, 768, seed=113)
    if not np.array_equal(oracle.matmul(Q5, W5.reshape(-1), x, 5)[0], oracle.matmul(Q4, W4, x, 5)[0]):
        return "Q5_K without high bits must equal Q4_K"
    return None


Q5K_PINS = [pin_q5k_golden, pin_q5k_brute_force, pin_q5k_fold_identity, pin_q5k_no_high_bits_is_q4k]


@pytest.mark.parametrize("pin", Q5K_PINS, ids=[p.__name__ for p in Q5K_PINS])
def test_q5k_pin(pin):
    msg = pin()
    assert msg is None, msg


def test_planted_q5k_mistake_is_caught(tmp_path):
    path = oracle.build(out=str(tmp_path / "liboracle_m14.so"), mutate=14)
    with oracle.use(path):
        failures = [m for m in (p() for p in Q5K_PINS) if m is not None]
    assert failures
    assert all(p() is None for p in Q5K_PINS)
