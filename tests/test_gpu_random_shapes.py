"""GPU parity on seeded random shapes: every weight type through qmm_matmul.

The hand-picked shape lists of the other parity tests cover the tile edges they were
written for; these cases add shapes drawn at random from a fixed seed -- odd row
counts, token counts on both sides of the vector / matrix switch and up to several
hundred, K from one super-block to 16 -- each against the oracle to the same bar
(f32 outputs within 1e-5 of max(|oracle|, A/sqrt(n))).  Padded Q6_K weights give
the unpadded result bit for bit.  The draw keeps nt * od * id below 3e8 so the
oracle finishes each case in about a second or less.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
DEV = "cuda:0"
TYPES = (qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q4_0, qmm.QMM_TYPE_Q8_0, qmm.QMM_TYPE_Q5_K)
BUDGET = 3e8


def _cases(n=24, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        qt = TYPES[i % len(TYPES)]
        nt = int(rng.choice([rng.integers(1, 9), rng.integers(9, 160), rng.integers(160, 700)]))
        idim = 256 * int(rng.integers(1, 17))
        od = int(rng.integers(1, 3000))
        od = max(1, min(od, int(BUDGET // (nt * idim))))
        out.append((qt, nt, od, idim, 7000 + i))
    return out


CASES = _cases()


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_case_draw_is_varied():
    kinds = {nt <= 8 for _, nt, _, _, _ in CASES}
    assert kinds == {True, False}
    assert {qt for qt, *_ in CASES} == set(TYPES)
    assert any(od % 32 for _, _, od, _, _ in CASES) and any(nt % 32 for _, nt, _, _, _ in CASES)


@pytest.mark.parametrize("qtype,nt,od,idim,seed", CASES)
def test_random_shape_parity(qtype, nt, od, idim, seed):
    print(f"random shape: type={qtype} nt={nt} od={od} id={idim} seed={seed}", flush=True)
    W = synth.weights(qtype, od, idim, seed=seed)
    x = synth.activations(nt, idim, seed=seed + 1, outlier_frac=0.01)
    ref, mag, _ = oracle.matmul(qtype, W, x, od)
    Wt, xt = _up(W), _up(x)
    out = qmm.qmm_matmul(qtype, Wt, xt, od)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, mag, qtype, idim, f"type {qtype} nt {nt} od {od} id {idim}")
    if qtype == qmm.QMM_TYPE_Q6_K:
        o2 = qmm.qmm_matmul(qmm.QMM_TYPE_Q6_K_P224, qmm.qmm_pad_q6k(Wt), xt, od)
        torch.cuda.synchronize()
        assert torch.equal(o2.view(torch.int32), out.view(torch.int32))
