"""GPU parity of the padded Q6_K layout (QMM_TYPE_Q6_K_P224), through the C ABI.

Page: "The quantized GEMM" (mojo-dllm kernels page), The GPU path, "Weights stay in
GGUF blocks": the upload pads each 210-byte Q6_K block to 224 bytes so every
16-byte piece is aligned and the kernels load 16 bytes at a time.

* qmm_pad_q6k writes exactly the source block bytes and zero pad;
* the padded path runs the same arithmetic in the same order as the unpadded one,
  so every output is bit-identical to QMM_TYPE_Q6_K's, for the vector kernel
  (nt = 1..8) and every matrix-kernel tile shape; the per-group integer dots are
  bit-exact against the oracle; outputs are within tolerance of the oracle;
* full size: the 32000 x 4096 output head at nt = 1, 5 and 8, 12288 x 4096 at nt = 7
  and 4096 x 4096 at nt = 8 (the vector kernel with and without token batches),
  and the diffusion-LM down projection 4096 x 12288 at L = 256.
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
Q6, P6 = qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q6_K_P224
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _np_pad(W):
    b = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1, 210)
    out = np.zeros((b.shape[0], 224), np.uint8)
    out[:, :210] = b
    return out.reshape(-1)


@pytest.mark.parametrize("nblocks", [1, 3, 1000, 65537])
def test_pad_q6k_bytes(nblocks):
    W = synth.weights(Q6, nblocks, 256, seed=2000 + nblocks)
    src = torch.zeros(W.size + 16, dtype=torch.uint8, device=DEV)
    src[2:2 + W.size] = _up(W)   # a 2-byte offset source: any alignment is allowed
    got = qmm.qmm_pad_q6k(src[2:2 + W.size])
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), _np_pad(W))


CASES = [(1, 7, 256), (3, 64, 512), (8, 100, 2304), (9, 33, 768), (64, 257, 1024), (130, 96, 4096)]


@pytest.mark.parametrize("nt,od,idim", CASES, ids=[f"{a}x{b}x{c}" for a, b, c in CASES])
def test_padded_equals_unpadded(nt, od, idim):
    _say(f"padded Q6_K nt={nt} od={od} id={idim}")
    W = synth.weights(Q6, od, idim, seed=2100 + od)
    Wt = _up(W)
    Wp = qmm.qmm_pad_q6k(Wt)
    x = synth.activations(nt, idim, seed=2200 + nt, outlier_frac=0.01)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    kinds = [qmm.QMM_KIND_MMQ, qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK]
    if nt <= 8:
        kinds = [qmm.QMM_KIND_MMVQ] + kinds
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8(oracle.TYPE_Q6_K_P224, _np_pad(W), qn, dn, sn, od)
    for kind in kinds:
        a = qmm.qmm_matmul_q8_kind(kind, Q6, Wt, q, d, s, od)
        b = qmm.qmm_matmul_q8_kind(kind, P6, Wp, q, d, s, od)
        torch.cuda.synchronize()
        an, bn = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(an.view(np.uint32), bn.view(np.uint32)), f"kind {kind}: padded differs"
        assert_close(bn, ref, mag, P6, idim, f"kind {kind} vs oracle")
    for kind in ([qmm.QMM_KIND_MMVQ] if nt <= 8 else []) + [qmm.QMM_KIND_MMQ]:
        S = qmm.qmm_group_dots(kind, P6, Wp, q, od)
        torch.cuda.synchronize()
        ref_S = oracle.subblock_dots(oracle.TYPE_Q6_K_P224, _np_pad(W), qn, od)
        assert np.array_equal(S.cpu().numpy(), ref_S), f"kind {kind}: group dots"


@pytest.mark.parametrize("od,idim,nt", [(32000, 4096, 1), (4096, 12288, 256), (32000, 4096, 5), (32000, 4096, 8),
                                        (12288, 4096, 7), (4096, 4096, 8)])
def test_padded_full_size(od, idim, nt):
    _say(f"padded Q6_K full size od={od} id={idim} nt={nt}")
    W = synth.weights(Q6, od, idim, seed=2300 + nt)
    Wt = _up(W)
    Wp = qmm.qmm_pad_q6k(Wt)
    x = synth.activations(nt, idim, seed=2400 + nt)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    a = qmm.qmm_matmul_q8(Q6, Wt, q, d, s, od)
    b = qmm.qmm_matmul_q8(P6, Wp, q, d, s, od)
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))
    rng = np.random.default_rng(od)
    rs = np.unique(np.concatenate([rng.choice(od, 200, replace=False), [0, od - 1]])).astype(np.int32)
    ts = np.arange(nt, dtype=np.int32) if nt <= 8 else np.array([0, 7, 100, nt - 1], np.int32)
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    ref, mag = oracle.matmul_q8_points(oracle.TYPE_Q6_K_P224, _np_pad(W), qn, dn, sn, od, tt, rr)
    assert_close(b.cpu().numpy()[tt, rr], ref, mag, P6, idim, "padded full size")
