"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: quantized activations (q, d, s) and the per-scale-group int32 dots of
both kernels.  f32 outputs: within 1e-5 of max(|oracle|, A/sqrt(n)) (tests/_parity.py).
Shapes span several tiles and ragged tails in od, nt and super-block count.
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
Q4, Q6 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _say(*a):
    print(*a, flush=True)


def test_mfma_tile_layout():
    """Pins the MFMA operand/result lane mappings the MMQ kernels assume: the int8
    32x32x32 tile, the f32 pair of outer products and the f32 K=2 product."""
    rng = np.random.default_rng(0)
    for trial in range(3):
        A = rng.integers(-128, 128, (32, 32), dtype=np.int8)
        B = rng.integers(-128, 128, (32, 32), dtype=np.int8)
        if trial == 2:
            A[:] = 0
            A[np.arange(32), np.arange(32)] = 1   # identity: C = B exactly
        C = qmm.qmm_mfma_tile_check(1, _up(A), _up(B))
        torch.cuda.synchronize()
        want = B.astype(np.int64) @ A.astype(np.int64).T
        assert np.array_equal(C.cpu().numpy().astype(np.int64), want)
    # small integers keep every f32 product and sum exact
    a = rng.integers(-50, 50, (2, 32)).astype(np.float32)
    b = rng.integers(-50, 50, (2, 32)).astype(np.float32)
    C2 = qmm.qmm_mfma_tile_check(2, _up(a), _up(b))
    C3 = qmm.qmm_mfma_tile_check(3, _up(a), _up(b))
    torch.cuda.synchronize()
    want2 = np.stack([np.outer(b[k], a[k]) for k in range(2)])      # [k][token][row]
    want3 = b.T @ a                                                # [token][row]
    assert np.array_equal(C2.cpu().numpy(), want2)
    assert np.array_equal(C3.cpu().numpy(), want3)


QUANT_CASES = [(1, 32, 0), (1, 96, 1), (3, 256, 2), (7, 4096, 3), (64, 768, 4), (129, 2048, 5), (512, 4096, 6)]


@pytest.mark.parametrize("nt,idim,seed", QUANT_CASES)
def test_quantize_bitexact(nt, idim, seed):
    _say(f"quantize nt={nt} id={idim} seed={seed}")
    scale = [1.0, 1e-3, 3e3, 1.0, 1e-20, 1.0, 1.0][seed]
    x = (synth.activations(nt, idim, seed=seed, outlier_frac=0.01) * np.float32(scale)).astype(np.float32)
    if idim >= 64:
        x[0, 32:64] = 0.0          # an all-zero block
    if nt > 1:
        x[1, :32] = np.float32(1.5)  # ties on the scale grid
    rq, rd, rs = oracle.quantize(x)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quantize_golden_ties_on_gpu():
    import os
    from tests.test_oracle_pins import _read_golden
    g = _read_golden("quantize_ties.txt")
    x = np.array([[float(v) for v in g[f"{n}.x"]] for n in "ABC"], np.float32).reshape(1, 96)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    torch.cuda.synchronize()
    want_q = np.array([[int(v) for n in "ABC" for v in g[f"{n}.q"]]], np.int8)
    assert np.array_equal(q.cpu().numpy(), want_q)
    assert list(d.cpu().numpy()[0]) == [float(g[f"{n}.d"][0]) for n in "ABC"]
    assert list(s.cpu().numpy()[0]) == [float(g[f"{n}.s"][0]) for n in "ABC"]


DOT_CASES = [
    (Q4, 1, 5, 256), (Q4, 3, 33, 768), (Q4, 8, 70, 2304), (Q4, 9, 65, 512), (Q4, 40, 97, 768),
    (Q6, 1, 5, 256), (Q6, 4, 33, 768), (Q6, 8, 70, 2304), (Q6, 9, 65, 512), (Q6, 70, 130, 512),
]


@pytest.mark.parametrize("qtype,nt,od,idim", DOT_CASES)
def test_group_dots_bitexact(qtype, nt, od, idim):
    _say(f"group dots type={qtype} nt={nt} od={od} id={idim}")
    W = synth.weights(qtype, od, idim, seed=nt + od)
    x = synth.activations(nt, idim, seed=nt + od + 1, outlier_frac=0.02)
    rq, _, _ = oracle.quantize(x)
    ref = oracle.subblock_dots(qtype, W, rq, od)
    Wt, qt = _up(W), _up(rq)
    kinds = [qmm.QMM_KIND_MMQ] + ([qmm.QMM_KIND_MMVQ] if nt <= 8 else [])
    for kind in kinds:
        S = qmm.qmm_group_dots(kind, qtype, Wt, qt, od)
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), ref), f"kind {kind}"


MATMUL_CASES = []
for _qt in (Q4, Q6):
    for _nt in (1, 2, 3, 4, 5, 6, 7, 8, 9, 13, 64, 100):
        for _od, _id in ((1, 256), (7, 768), (64, 512), (100, 2304), (257, 1024)):
            if _nt * _od * _id <= 100 * 257 * 2304:
                MATMUL_CASES.append((_qt, _nt, _od, _id))


@pytest.mark.parametrize("qtype,nt,od,idim", MATMUL_CASES)
def test_matmul_parity(qtype, nt, od, idim):
    _say(f"matmul type={qtype} nt={nt} od={od} id={idim}")
    W = synth.weights(qtype, od, idim, seed=1000 + nt)
    x = synth.activations(nt, idim, seed=2000 + od, outlier_frac=0.01)
    ref, mag, (rq, rd, rs) = oracle.matmul(qtype, W, x, od)
    Wt, xt = _up(W), _up(x)
    out = qmm.qmm_matmul(qtype, Wt, xt, od)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, mag, qtype, idim, f"qmm_matmul {qtype} {nt} {od} {idim}")
    # both kernels on the same quantized input where both apply
    if nt <= 8:
        for kind in (qmm.QMM_KIND_MMVQ, qmm.QMM_KIND_MMQ):
            o2 = qmm.qmm_matmul_q8_kind(kind, qtype, Wt, _up(rq), _up(rd), _up(rs), od)
            torch.cuda.synchronize()
            assert_close(o2.cpu().numpy(), ref, mag, qtype, idim, f"kind {kind}")


TILE_CASES = [(qt, nt, od, idim) for qt in (Q4, Q6)
              for nt, od, idim in ((9, 65, 256), (40, 130, 768), (100, 257, 2304), (64, 128, 512), (70, 33, 4608))]


@pytest.mark.parametrize("qtype,nt,od,idim", TILE_CASES)
def test_mmq_every_tile_shape(qtype, nt, od, idim):
    """Each MMQ tile shape, forced, on ragged tiles and odd super-block counts (1,
    3, 9, 2, 18: the split over K then has a group with nothing left to add)."""
    _say(f"mmq tiles type={qtype} nt={nt} od={od} id={idim}")
    W = synth.weights(qtype, od, idim, seed=3000 + nt)
    x = synth.activations(nt, idim, seed=4000 + od, outlier_frac=0.01)
    rq, rd, rs = oracle.quantize(x)
    ref, mag = oracle.matmul_q8(qtype, W, rq, rd, rs, od)
    args = (_up(W), _up(rq), _up(rd), _up(rs), od)
    kinds = [qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK]
    if qtype == Q4:
        kinds += [qmm.QMM_KIND_MMQ_WAVE32X64, qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK]
    for kind in kinds:
        o = qmm.qmm_matmul_q8_kind(kind, qtype, *args)
        torch.cuda.synchronize()
        assert_close(o.cpu().numpy(), ref, mag, qtype, idim, f"kind {kind}")
    # the split adds its partial sums in a fixed order: the same bits every run
    o1 = qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_64X64_SPLITK, qtype, *args)
    o2 = qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_64X64_SPLITK, qtype, *args)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def test_dispatch_boundary():
    """On a small matrix: nt = 8 runs MMVQ; nt = 9..16 run the small-batch kernel
    (Q4_K) or MMVQ on token slices of 8 (Q6_K); Q4_K at 17..48 tokens the
    small-batch kernel on token slices of 16; nt = 49 (Q4_K) and 17 (Q6_K) run MMQ.
    Every call matches the oracle; the Q6_K sliced call gives the same bits as its
    slices called alone, and a Q4_K small-batch call the same bits as the
    small-batch kernel on its tokens alone."""
    assert qmm.qmm_dispatch_kind(Q4, 8, 64, 512) == qmm.QMM_KIND_MMVQ
    assert qmm.qmm_dispatch_kind(Q4, 9, 64, 512) == qmm.QMM_KIND_SKINNY
    assert qmm.qmm_dispatch_kind(Q4, 16, 64, 512) == qmm.QMM_KIND_SKINNY
    assert qmm.qmm_dispatch_kind(Q4, 17, 64, 512) == qmm.QMM_KIND_SKINNY
    assert qmm.qmm_dispatch_kind(Q4, 48, 64, 512) == qmm.QMM_KIND_SKINNY
    assert qmm.qmm_dispatch_kind(Q4, 49, 64, 512) == qmm.QMM_KIND_MMQ
    assert qmm.qmm_dispatch_kind(Q6, 9, 64, 512) == qmm.QMM_KIND_MMVQ
    assert qmm.qmm_dispatch_kind(Q6, 17, 64, 512) == qmm.QMM_KIND_MMQ
    od, idim = 96, 1024
    for qtype in (Q4, Q6):
        W = synth.weights(qtype, od, idim, seed=5)
        x = synth.activations(49, idim, seed=5)
        ref, mag, _ = oracle.matmul(qtype, W, x, od)
        Wt = _up(W)
        for nt in (8, 9, 13, 16, 17, 33, 48, 49):
            o = qmm.qmm_matmul(qtype, Wt, _up(x[:nt]), od)
            torch.cuda.synchronize()
            assert_close(o.cpu().numpy(), ref[:nt], mag[:nt], qtype, idim, f"nt={nt}")
        q, d, s = qmm.qmm_quantize_act(_up(x[:13]))
        whole = qmm.qmm_matmul_q8(qtype, Wt, q, d, s, od)
        if qtype == Q4:
            k7 = qmm.QMM_KIND_SKINNY
            a = qmm.qmm_matmul_q8_kind(k7, qtype, Wt, q[:8].contiguous(), d[:8].contiguous(), s[:8].contiguous(), od)
            b = qmm.qmm_matmul_q8_kind(k7, qtype, Wt, q[8:].contiguous(), d[8:].contiguous(), s[8:].contiguous(), od)
        else:
            a = qmm.qmm_matmul_q8(qtype, Wt, q[:8].contiguous(), d[:8].contiguous(), s[:8].contiguous(), od)
            b = qmm.qmm_matmul_q8(qtype, Wt, q[8:].contiguous(), d[8:].contiguous(), s[8:].contiguous(), od)
        torch.cuda.synchronize()
        assert torch.equal(whole.view(torch.int32), torch.cat([a, b]).view(torch.int32))


def test_special_inputs():
    """Zero activations give exactly zero; Q6_K codes all 32 give exactly zero."""
    od, idim = 40, 512
    W = synth.weights(Q4, od, idim, seed=9)
    z = np.zeros((10, idim), np.float32)
    out = qmm.qmm_matmul(Q4, _up(W), _up(z), od)
    W6 = synth.weights(Q6, od, idim, seed=9).reshape(-1, 210).copy()
    W6[:, 0:128] = 0
    W6[:, 128:192] = 0xAA
    x = synth.activations(10, idim, seed=9)
    o6a = qmm.qmm_matmul(Q6, _up(W6.reshape(-1)), _up(x[:3]), od)
    o6b = qmm.qmm_matmul(Q6, _up(W6.reshape(-1)), _up(x), od)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)
    assert np.all(o6a.cpu().numpy() == 0.0) and np.all(o6b.cpu().numpy() == 0.0)


def test_error_codes_leave_output_untouched():
    od, idim, nt = 16, 512, 2
    W = _up(synth.weights(Q4, od, idim))
    x = _up(synth.activations(nt, idim))
    out = torch.full((nt, od), 7.0, device=DEV)
    ws = torch.empty(qmm.qmm_act_bytes(nt, idim) + 64, dtype=torch.uint8, device=DEV)
    L = qmm.lib()
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    assert L.qmm_matmul(99, P(W), P(x), nt, od, idim, P(out), P(ws), ws.numel(), st) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul(Q4, P(W), P(x), nt, od, 300, P(out), P(ws), ws.numel(), st) == qmm.QMM_ERR_SHAPE
    assert L.qmm_matmul(Q4, P(W), P(x), 0, od, idim, P(out), P(ws), ws.numel(), st) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul(Q4, P(W, 4), P(x), nt, od, idim, P(out), P(ws), ws.numel(), st) == qmm.QMM_ERR_ALIGN
    assert L.qmm_matmul(Q4, P(W), P(x), nt, od, idim, P(out), P(ws), 100, st) == qmm.QMM_ERR_WORKSPACE
    assert L.qmm_matmul(Q4, None, P(x), nt, od, idim, P(out), P(ws), ws.numel(), st) == qmm.QMM_ERR_ARG
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    with pytest.raises(qmm.QmmError):
        qmm.qmm_matmul(Q4, W, x[:, :300].contiguous(), od)


def test_single_hip_runtime_mapped():
    """torch and libqmm share one HIP runtime (one libamdhip64 mapped)."""
    qmm.lib()
    torch.zeros(1, device=DEV)
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths
