"""qmm_matmul_noalloc (the entry point for callers that cannot allocate) against
qmm_matmul, through the C ABI with raw device pointers.

Two calls in a row on the shared scratch, the second smaller than the first, then a
third of another weight type: each output equals, bit for bit, qmm_matmul's with a
caller workspace of the same size (the same launches), and both are within the
oracle parity tolerance.  A call too large for the scratch is refused before any
device work and leaves the output untouched.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._parity import assert_close

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(qtype, W, x, od):
    """(noalloc output, qmm_matmul output with a workspace of the scratch's size) on
    the host, both through the raw C ABI."""
    L = qmm.lib()
    nt, idim = x.shape
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    Wg, xg = _up(W), _up(x)
    out_n = torch.full((nt, od), float("nan"), dtype=torch.float32, device=DEV)
    out_w = torch.full((nt, od), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(qmm.QMM_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
    rc = L.qmm_matmul_noalloc(qtype, _ptr(Wg), _ptr(xg), nt, od, idim, _ptr(out_n), st)
    assert rc == qmm.QMM_OK, qmm.strerror(rc)
    rc = L.qmm_matmul(qtype, _ptr(Wg), _ptr(xg), nt, od, idim, _ptr(out_w), _ptr(ws), ws.numel(), st)
    assert rc == qmm.QMM_OK, qmm.strerror(rc)
    torch.cuda.synchronize()
    return out_n.cpu().numpy(), out_w.cpu().numpy()


def _check_oracle(qtype, W, x, od, got, full, seed):
    nt, idim = x.shape
    q, d, s = oracle.quantize(x)
    if full:
        ref, mag = oracle.matmul_q8(qtype, W, q, d, s, od)
        assert_close(got, ref, mag, qtype, idim, "noalloc vs oracle")
        return
    rng = np.random.default_rng(seed)
    ts = np.unique(np.concatenate([rng.choice(nt, 12, replace=False), [0, nt - 1]]))
    rs = np.unique(np.concatenate([rng.choice(od, 64, replace=False), [0, od - 1]]))
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    ref, mag = oracle.matmul_q8_points(qtype, W, q, d, s, od, tt, rr)
    assert_close(got[tt, rr], ref, mag, qtype, idim, "noalloc vs oracle (sampled)")


# a large call (stream-K where qmm_matmul takes it), then a smaller one, then another type
CALLS = [
    ("Q4_K 4096x12288 nt=512", qmm.QMM_TYPE_Q4_K, 4096, 12288, 512, 0.01, False),
    ("Q4_K 1024x4096 nt=3", qmm.QMM_TYPE_Q4_K, 1024, 4096, 3, 0.0, True),
    ("Q6_K 300x1024 nt=40", qmm.QMM_TYPE_Q6_K, 300, 1024, 40, 0.0, True),
]


def test_noalloc_matches_matmul_on_consecutive_calls():
    for seed, (label, qtype, od, idim, nt, outl, full) in enumerate(CALLS):
        print(f"case noalloc {label}", flush=True)
        W = synth.weights(qtype, od, idim, seed=500 + seed)
        x = synth.activations(nt, idim, seed=600 + seed, outlier_frac=outl)
        got, ref_ws = _both(qtype, W, x, od)
        assert np.array_equal(got.view(np.uint32), ref_ws.view(np.uint32)), f"{label}: differs from qmm_matmul"
        _check_oracle(qtype, W, x, od, got, full, seed)


def test_noalloc_refuses_calls_beyond_its_scratch():
    L = qmm.lib()
    nt, idim, od = 2048, 12288, 256
    W = _up(synth.weights(qmm.QMM_TYPE_Q4_K, od, idim, seed=7))
    x = torch.zeros((nt, idim), dtype=torch.float32, device=DEV)
    out = torch.full((nt, od), 3.0, dtype=torch.float32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.qmm_matmul_noalloc(qmm.QMM_TYPE_Q4_K, _ptr(W), _ptr(x), nt, od, idim, _ptr(out), st)
    assert rc == qmm.QMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a refused call must not touch the output"
