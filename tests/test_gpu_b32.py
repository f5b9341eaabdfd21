"""GPU parity of the 32-weight block formats Q4_0 and Q8_0, through the C ABI.

Pages: "03 - Reading minfer's kernels I", section 3.2 (the Q4_0 block) and "04 -
Reading minfer's kernels II", section 3.4 (the Q4_0 x q8 decode dot, the offset
folded through the activation sum).  Q8_0's layout is a reading (f16 d, 32 int8).

* the per-block integer dots of both kernels are bit-exact against the oracle;
* f32 outputs within |g - o| <= 1e-5 * max(|o|, A / sqrt(n)) of the oracle's
  exact f64 combine, for the vector kernel at nt = 1..8 and every matrix-kernel
  tile shape, over several tiles and ragged tails in every dimension;
* the nt dispatch (qmm_matmul on f32 activations) on both sides of the switch;
* full size: 12288 x 4096 at nt = 1 and nt = 512 (sampled outputs).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._parity import assert_close, oracle_activations

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
Q40, Q80 = qmm.QMM_TYPE_Q4_0, qmm.QMM_TYPE_Q8_0
DEV = "cuda:0"
KINDS_MMQ = [qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK]


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = [(1, 5, 256), (3, 33, 768), (8, 70, 2304), (2, 64, 4096), (9, 65, 512), (40, 97, 768),
         (64, 128, 1024), (100, 257, 2048)]


@pytest.mark.parametrize("qtype", [Q40, Q80], ids=["Q4_0", "Q8_0"])
@pytest.mark.parametrize("nt,od,idim", CASES, ids=[f"{a}x{b}x{c}" for a, b, c in CASES])
def test_b32_parity(qtype, nt, od, idim):
    _say(f"type {qtype} nt={nt} od={od} id={idim}")
    W = synth.weights(qtype, od, idim, seed=3000 + od + qtype)
    x = synth.activations(nt, idim, seed=3100 + nt, outlier_frac=0.01)
    Wt = _up(W)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8(qtype, W, qn, dn, sn, od)
    ref_S = oracle.subblock_dots(qtype, W, qn, od)
    kinds = ([qmm.QMM_KIND_MMVQ] if nt <= 8 else []) + [qmm.QMM_KIND_MMQ]
    for kind in kinds:
        S = qmm.qmm_group_dots(kind, qtype, Wt, q, od)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), ref_S), f"kind {kind}: integer dots differ"
    for kind in kinds + KINDS_MMQ:
        out = qmm.qmm_matmul_q8_kind(kind, qtype, Wt, q, d, s, od)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, mag, qtype, idim, f"kind {kind}")
    # the whole path from f32 activations, through the dispatch
    out = qmm.qmm_matmul(qtype, Wt, _up(x), od)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, mag, qtype, idim, "qmm_matmul")


@pytest.mark.parametrize("qtype", [Q40, Q80], ids=["Q4_0", "Q8_0"])
@pytest.mark.parametrize("nt", [1, 4, 512])
def test_b32_full_size(qtype, nt):
    od, idim = 12288, 4096
    _say(f"type {qtype} full size nt={nt}")
    W = synth.weights(qtype, od, idim, seed=3200 + qtype)
    x = synth.activations(nt, idim, seed=3300 + nt, outlier_frac=0.01)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    out = qmm.qmm_matmul_q8(qtype, _up(W), q, d, s, od).cpu().numpy()
    rng = np.random.default_rng(nt + qtype)
    ts = np.unique(np.concatenate([rng.choice(nt, min(nt, 16), replace=False), [0, nt - 1]]))
    rs = np.unique(np.concatenate([rng.choice(od, 160, replace=False), [0, od - 1]]))
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8_points(qtype, W, qn, dn, sn, od, tt, rr)
    assert_close(out[tt, rr], ref, mag, qtype, idim, f"full size nt={nt}")
