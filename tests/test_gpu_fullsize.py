"""GPU parity at the benchmark's full layer shapes, in the launch configuration the
benchmark times (qmm_quantize_act, then qmm_matmul_q8 on the quantized plane).

* The quantized activations (q, d, s) are compared bit-exact over the whole plane.
* Outputs: every element where the oracle takes a second or two, else a seeded
  sample of rows and tokens that always includes the first and last of each, the
  oracle computing those outputs one by one.
* Decode shapes: the nt rows of one MMVQ call equal nt separate nt = 1 calls bit for
  bit (the token loop keeps each token's reduction order).
* Edge cases: the longest rows and the most rows exercised here, activation blocks
  that are exactly zero, scales near the bottom and top of the f32 range.
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
Q4, Q6, Q5 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q5_K
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _say(*a):
    print(*a, flush=True)


def _run(qtype, W, x, od):
    """The benchmark's launch sequence; returns (q, d, s, out) on the host."""
    xt = _up(x)
    q, d, s = qmm.qmm_quantize_act(xt)
    out = qmm.qmm_matmul_q8(qtype, _up(W), q, d, s, od)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy(), s.cpu().numpy(), out.cpu().numpy()


def _check_q8(got, ref, what):
    for name, g, r in zip("qds", got, ref):
        assert g.dtype == r.dtype and np.array_equal(g.view(np.uint8), r.view(np.uint8)), f"{what}: {name} differs"


def _sample(n, k, rng):
    idx = rng.choice(n, size=min(n, k), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]]))


def _check_out(qtype, W, od, idim, rq, rd, rs, out, what, full, seed=0):
    nt = rq.shape[0]
    if full:
        ref, mag = oracle.matmul_q8(qtype, W, rq, rd, rs, od)
        return assert_close(out, ref, mag, qtype, idim, what)
    rng = np.random.default_rng(seed)
    ts = _sample(nt, 24, rng)
    rs_ = _sample(od, 160, rng)
    tt, rr = np.meshgrid(ts, rs_, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    ref, mag = oracle.matmul_q8_points(qtype, W, rq, rd, rs, od, tt, rr)
    return assert_close(out[tt, rr], ref, mag, qtype, idim, what)


# (label, type, od, id, nt, outlier fraction, seed, compare every output)
SHAPES = [
    ("Q4_K decode 1024x4096", Q4, 1024, 4096, 1, 0.0, 0, True),
    ("Q4_K decode 4096x4096 nt=1", Q4, 4096, 4096, 1, 0.0, 11, True),
    ("Q4_K decode 4096x4096 nt=4", Q4, 4096, 4096, 4, 0.0, 12, True),
    ("Q4_K decode 4096x4096 nt=8", Q4, 4096, 4096, 8, 0.0, 13, True),
    ("Q4_K decode 12288x4096 nt=1", Q4, 12288, 4096, 1, 0.0, 14, True),
    ("Q4_K decode 12288x4096 nt=4", Q4, 12288, 4096, 4, 0.0, 15, True),
    ("Q4_K decode 12288x4096 nt=8", Q4, 12288, 4096, 8, 0.0, 16, True),
    ("Q6_K head 32000x4096 nt=1", Q6, 32000, 4096, 1, 0.0, 17, True),
    ("Q4_K prefill 12288x4096 nt=512", Q4, 12288, 4096, 512, 0.01, 18, False),
    ("Q4_K prefill 4096x12288 nt=512", Q4, 4096, 12288, 512, 0.01, 19, False),
    ("dLLM q/k/v/o Q4_K 4096x4096 L=256", Q4, 4096, 4096, 256, 0.0, 20, False),
    ("dLLM gate/up Q4_K 12288x4096 L=256", Q4, 12288, 4096, 256, 0.0, 21, False),
    ("dLLM down Q6_K 4096x12288 L=256", Q6, 4096, 12288, 256, 0.0, 22, False),
]


@pytest.mark.parametrize("label,qtype,od,idim,nt,outl,seed,full", SHAPES, ids=[s[0] for s in SHAPES])
def test_full_size_parity(label, qtype, od, idim, nt, outl, seed, full):
    _say(f"full size: {label}")
    W = synth.weights(qtype, od, idim, seed=seed)
    x = synth.activations(nt, idim, seed=seed, outlier_frac=outl)
    ref_q8 = oracle.quantize(x)
    q, d, s, out = _run(qtype, W, x, od)
    _check_q8((q, d, s), ref_q8, label)
    worst, rel = _check_out(qtype, W, od, idim, *ref_q8, out, label, full, seed)
    _say(f"  worst err/tol {worst:.3f}, max rel err {rel:.2e}")


@pytest.mark.parametrize("qtype,od,idim", [(Q4, 12288, 4096), (Q4, 4096, 4096), (Q4, 4096, 12288),
                                           (Q6, 32000, 4096), (Q6, 12288, 4096), (Q6, 4096, 4096),
                                           (Q4, 100, 2304), (Q6, 257, 1024),
                                           (Q5, 12288, 4096), (Q5, 4096, 4096), (Q5, 8192, 4096)])
def test_mmvq_rows_equal_single_token_calls(qtype, od, idim):
    """Each token row of an nt = 2..16 MMVQ call is bit-identical to that token alone
    (also where the tokens' activations are loaded in batches: Q4_K, Q5_K and Q6_K
    with 4 rows per group, with and without the launch-size condition)."""
    _say(f"batch invariance type={qtype} od={od} id={idim}")
    W = _up(synth.weights(qtype, od, idim, seed=31))
    x = synth.activations(16, idim, seed=32)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    singles = [qmm.qmm_matmul_q8(qtype, W, q[t:t + 1].contiguous(), d[t:t + 1].contiguous(),
                                 s[t:t + 1].contiguous(), od) for t in range(16)]
    ref = torch.cat(singles).cpu().numpy()
    for nt in range(2, 17):
        args = (q[:nt].contiguous(), d[:nt].contiguous(), s[:nt].contiguous(), od)
        # MMVQ forced for nt > 8 too: one launch per slice of 8 tokens
        o = qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMVQ, qtype, W, *args)
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy().view(np.uint32), ref[:nt].view(np.uint32)), f"MMVQ nt={nt}"
        kind = qmm.qmm_dispatch_kind(qtype, nt, od, idim)
        if kind == qmm.QMM_KIND_MMVQ:
            o = qmm.qmm_matmul_q8(qtype, W, *args)
            torch.cuda.synchronize()
            assert np.array_equal(o.cpu().numpy().view(np.uint32), ref[:nt].view(np.uint32)), f"nt={nt}"
        elif kind == qmm.QMM_KIND_SKINNY:
            # the small-batch kernel is batch invariant too: against its own single-token calls
            o = qmm.qmm_matmul_q8(qtype, W, *args)
            ones = [qmm.qmm_matmul_q8_kind(kind, qtype, W, q[t:t + 1].contiguous(), d[t:t + 1].contiguous(),
                                           s[t:t + 1].contiguous(), od) for t in range(nt)]
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int32), torch.cat(ones).view(torch.int32)), f"small-batch nt={nt}"
        else:
            assert kind == qmm.QMM_KIND_MMQ and nt > 8 and od > 4096


EDGE = [
    ("longest rows Q4_K id=65536", Q4, 40, 65536, 3),
    ("longest rows Q4_K id=65536 MMQ", Q4, 40, 65536, 17),
    ("longest rows Q6_K id=65536", Q6, 40, 65536, 5),
    ("most rows Q4_K od=262144", Q4, 262144, 256, 1),
    ("most rows Q6_K od=131072 MMQ", Q6, 131072, 256, 33),
]


@pytest.mark.parametrize("label,qtype,od,idim,nt", EDGE, ids=[e[0] for e in EDGE])
def test_extreme_shapes(label, qtype, od, idim, nt):
    _say(f"edge: {label}")
    W = synth.weights(qtype, od, idim, seed=41)
    x = synth.activations(nt, idim, seed=42, outlier_frac=0.01)
    ref_q8 = oracle.quantize(x)
    q, d, s, out = _run(qtype, W, x, od)
    _check_q8((q, d, s), ref_q8, label)
    _check_out(qtype, W, od, idim, *ref_q8, out, label, full=True)


@pytest.mark.parametrize("qtype", [Q4, Q6])
@pytest.mark.parametrize("nt", [3, 12])
def test_zero_blocks_and_extreme_scales(qtype, nt):
    """Exactly-zero 32-blocks, blocks whose scale is subnormal, and blocks near the
    top of the f32 range, mixed in one activation matrix, through both kernels."""
    od, idim = 96, 2048
    x = synth.activations(nt, idim, seed=50 + nt).reshape(nt, idim // 32, 32)
    x[:, 0::5] = 0.0                      # whole blocks zero: d = q = s = 0
    x[:, 1::5] *= np.float32(1e-39)       # amax / 127 is subnormal
    x[:, 2::5] *= np.float32(1e-3)
    x[:, 3::5] *= np.float32(1e30)        # large but finite sums
    x = np.ascontiguousarray(x.reshape(nt, idim), dtype=np.float32)
    W = synth.weights(qtype, od, idim, seed=51)
    ref_q8 = oracle.quantize(x)
    q, d, s, out = _run(qtype, W, x, od)
    _check_q8((q, d, s), ref_q8, f"type {qtype} nt {nt}")
    assert np.all(d[:, 0::5] == 0.0) and np.all(q.reshape(nt, -1, 32)[:, 0::5] == 0)
    assert np.any((d[:, 1::5] > 0) & (d[:, 1::5] < np.finfo(np.float32).tiny))
    _check_out(qtype, W, od, idim, *ref_q8, out, f"type {qtype} nt {nt}", full=True)

LONG_K = [(qt, od, idim) for qt in (1, 2, 4, 6) for od, idim in ((1024, 12288), (2048, 12288), (300, 14336))]


@pytest.mark.parametrize("qtype,od,idim", LONG_K, ids=[f"t{q}-{a}x{b}" for q, a, b in LONG_K])
def test_mmvq_long_k_against_oracle(qtype, od, idim):
    """MMVQ on a K of six or seven windows and few rows, where the row-group size
    follows the wave count (2 or 4 rows per wave), at 1..8 tokens: every output
    against the oracle, which quantizes the activations itself."""
    _say(f"MMVQ long K type={qtype} od={od} id={idim}")
    W = synth.weights(qtype, od, idim, seed=51 + qtype)
    Wt = _up(W)
    for nt in (1, 2, 3, 5, 8):
        x = synth.activations(nt, idim, seed=52 + nt, outlier_frac=0.01)
        q, d, s = qmm.qmm_quantize_act(_up(x))
        out = qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMVQ, qtype, Wt, q, d, s, od)
        torch.cuda.synchronize()
        rq, rd, rs = oracle_activations(oracle.quantize, x, (q, d, s), f"nt={nt}")
        _check_out(qtype, W, od, idim, rq, rd, rs, out.cpu().numpy(), f"type {qtype} {od}x{idim} nt={nt}", full=True)
