"""The vectorised dequantizer (tests/dequant_np.py) against the element-by-element
decoder (tests/bruteforce.py) on random blocks of every weight layout: the two are
written independently from the byte layouts, so they must agree exactly."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import bruteforce as bf
from tests import dequant_np as dq


def _random_bytes(n, seed):
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def _fix_f16(W, qtype, od, idim):
    """Replace the f16 fields of random bytes by finite values (random bytes can
    make infinities and NaNs, which the two decoders would both propagate)."""
    B = W.reshape(od, -1, dq.BLOCK[qtype]).copy()
    if qtype in (1, 6):
        fields = [0, 2]
    elif qtype == 2:
        fields = [208]
    elif qtype == 4:
        fields = [18 * j for j in range(8)]
    else:
        fields = [34 * j for j in range(8)]
    for f in fields:
        B[..., f + 1] &= 0x3F   # exponent below the top of the range: finite
    return B.reshape(-1)


@pytest.mark.parametrize("qtype", [1, 2, 6])
@pytest.mark.parametrize("source", ["synth", "random"])
def test_k_quants_match_bruteforce(qtype, source):
    od, idim = 3, 512
    if source == "synth":
        W = synth.weights(qtype, od, idim, seed=5)
    else:
        W = _fix_f16(_random_bytes(od * 2 * dq.BLOCK[qtype], 6), qtype, od, idim)
    ref = bf.dequant(qtype, W, od, idim)
    got, mins = dq.dequant_rows(qtype, W, od, idim)
    assert np.array_equal(got, ref)
    if qtype in (1, 6):
        # mins: dmin * m_j, the value each sub-block subtracts
        B = W.reshape(od, 2, dq.BLOCK[qtype])
        for r in range(od):
            for b in range(2):
                dmin = bf.f16(int(B[r, b, 2]), int(B[r, b, 3]))
                for j in range(8):
                    assert mins[r, 8 * b + j] == dmin * bf.q4k_field(B[r, b], j)[1]


@pytest.mark.parametrize("qtype", [4, 5])
@pytest.mark.parametrize("source", ["synth", "random"])
def test_block32_match_bruteforce(qtype, source):
    od, idim = 3, 512
    if source == "synth":
        W = synth.weights(qtype, od, idim, seed=7)
    else:
        W = _fix_f16(_random_bytes(od * 2 * dq.BLOCK[qtype], 8), qtype, od, idim)
    assert np.array_equal(dq.dequant_rows(qtype, W, od, idim)[0], bf.b32_dequant(qtype, W, od, idim))


def test_padded_q6k_equals_unpadded():
    od, idim = 4, 768
    W = synth.weights(2, od, idim, seed=9).reshape(od, 3, 210)
    P = np.full((od, 3, 224), 0xA7, np.uint8)
    P[..., :210] = W
    assert np.array_equal(dq.dequant_rows(3, P.reshape(-1), od, idim)[0],
                          dq.dequant_rows(2, W.reshape(-1), od, idim)[0])


def test_row_selection():
    od, idim = 9, 256
    W = synth.weights(1, od, idim, seed=11)
    full, fm = dq.dequant_rows(1, W, od, idim)
    part, pm = dq.dequant_rows(1, W, od, idim, rows=[8, 0, 4])
    assert np.array_equal(part, full[[8, 0, 4]]) and np.array_equal(pm, fm[[8, 0, 4]])
