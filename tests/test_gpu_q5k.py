"""GPU parity of Q5_K weights, through the C ABI.

Q5_K is read as the public 176-byte layout (the pages name the type only): Q4_K's
header and codes with a fifth code bit from 32 bytes of high bits.

* the per-sub-block integer dots of both kernels are bit-exact against the oracle;
* f32 outputs within |g - o| <= 1e-5 * max(|o|, A / sqrt(n)) for the vector kernel
  at nt = 1..8 and every matrix-kernel tile shape, several tiles and ragged tails;
* with all high bits zero the Q5_K outputs equal the Q4_K kernel's on the same
  header and nibbles bit for bit (same arithmetic, same order);
* full size: 12288 x 4096 at nt = 1, 3, 4, 6, 8 (the vector kernel, with the tokens'
  activations loaded in batches from nt = 3) and nt = 512 (sampled outputs).
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
Q5, Q4 = qmm.QMM_TYPE_Q5_K, qmm.QMM_TYPE_Q4_K
DEV = "cuda:0"
KINDS_MMQ = [qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK]


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = [(1, 5, 256), (3, 33, 768), (8, 70, 2304), (9, 65, 512), (40, 97, 768), (100, 257, 2048)]


@pytest.mark.parametrize("nt,od,idim", CASES, ids=[f"{a}x{b}x{c}" for a, b, c in CASES])
def test_q5k_parity(nt, od, idim):
    print(f"Q5_K nt={nt} od={od} id={idim}", flush=True)
    W = synth.weights(Q5, od, idim, seed=5000 + od)
    x = synth.activations(nt, idim, seed=5100 + nt, outlier_frac=0.01)
    Wt = _up(W)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8(Q5, W, qn, dn, sn, od)
    ref_S = oracle.subblock_dots(Q5, W, qn, od)
    kinds = ([qmm.QMM_KIND_MMVQ] if nt <= 8 else []) + [qmm.QMM_KIND_MMQ]
    for kind in kinds:
        S = qmm.qmm_group_dots(kind, Q5, Wt, q, od)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), ref_S), f"kind {kind}: integer dots differ"
    for kind in kinds + KINDS_MMQ:
        out = qmm.qmm_matmul_q8_kind(kind, Q5, Wt, q, d, s, od)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, mag, Q5, idim, f"kind {kind}")
    # zero high bits: the same matrix as Q4_K, bit for bit through the same kernel body
    # (the Q5_K matrix kernel is the Q4_K one of the 64 x 64 tiles with a fifth code
    # bit; the default Q4_K matrix kernel on 128 x 64 tiles is another body)
    W0 = W.reshape(-1, 176).copy()
    W0[:, 16:48] = 0
    W4 = np.concatenate([W0[:, :16], W0[:, 48:]], axis=1).reshape(-1)
    for kind in [k if k != qmm.QMM_KIND_MMQ else qmm.QMM_KIND_MMQ_64X64 for k in kinds]:
        a = qmm.qmm_matmul_q8_kind(kind, Q5, _up(W0.reshape(-1)), q, d, s, od)
        b = qmm.qmm_matmul_q8_kind(kind, Q4, _up(W4), q, d, s, od)
        torch.cuda.synchronize()
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), f"kind {kind}"


@pytest.mark.parametrize("nt", [1, 3, 4, 6, 8, 512])
def test_q5k_full_size(nt):
    od, idim = 12288, 4096
    W = synth.weights(Q5, od, idim, seed=5200)
    x = synth.activations(nt, idim, seed=5300 + nt, outlier_frac=0.01)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    out = qmm.qmm_matmul_q8(Q5, _up(W), q, d, s, od).cpu().numpy()
    rng = np.random.default_rng(nt)
    ts = np.unique(np.concatenate([rng.choice(nt, min(nt, 16), replace=False), [0, nt - 1]]))
    rs = np.unique(np.concatenate([rng.choice(od, 160, replace=False), [0, od - 1]]))
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8_points(Q5, W, qn, dn, sn, od, tt, rr)
    assert_close(out[tt, rr], ref, mag, Q5, idim, f"full size nt={nt}")
