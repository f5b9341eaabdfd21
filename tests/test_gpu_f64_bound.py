"""GPU outputs against the plain f64 definition, out[t][r] = sum_i W_deq[r][i] x[t][i].

The method quantizes the activations, so its result is not that sum; it is within
a bound fixed by the quantizer's rules ("The quantized GEMM", "Checks": both GEMMs
against an f64 reference over the same dequantized weights).  Per token t and
activation block k (32 values; 256 for Q8_K) with scale d_k, every x_i of the
block is represented by d_k * q_i with |x_i - d_k q_i| <= d_k (1/2 + 127 * 2^-24)
(a correctly rounded quotient, rounded to the nearest integer), so

  |out - W_deq . x| <= sum_k d_k (1/2 + 2^-17) sum_{i in k} |w_i|          (activations)
                     + 2^-24 sum_k |off_k| |s_k|                          (rounded s = d * sum q)
                     + (n + 4) 2^-24 sum_k sum_{i in k} (|w_i| + |off_k|) |d_k q_i|
                                                                         (f32 products and sums)
                     + 2^-24 |W_deq . x|                                  (final rounding)

with off_k the value block k subtracts from its scaled codes (dmin*m for Q4_K /
Q5_K, 8 d for Q4_0, 32 d sc for Q6_K's centring, 0 for Q8_0) and n the number of
scale-group terms per output.  The weights are dequantized in f64 by
tests/dequant_np.py (checked against the element-by-element decoder on the CPU);
d_k, q and s come from the oracle's quantizer (bit-equal to the GPU's, tested
elsewhere).  Each case logs the largest ratio of error to bound.

The RMS norm feeding the quantizer is checked the same way: the GPU's f32 y against
f64 x / sqrt(mean(x^2) + eps) * w within the first-order error bound of its f32
operations (n/256 fused adds per lane, 8 halving levels, the mean, + eps, the
square root, the reciprocal, two products).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import dequant_np as dq

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
DEV = "cuda:0"
U = 2.0 ** -24


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _offsets(qtype, W, od, idim, rows):
    """|off_k| per row and 32-block [len(rows)][idim/32]."""
    if qtype in (2, 3):
        B = np.asarray(W, np.uint8).reshape(od, idim // 256, dq.BLOCK[qtype])[np.asarray(rows)]
        d = dq._f16(B[..., 208], B[..., 209])[..., None]
        sc = np.abs(B[..., 192:208].view(np.int8).astype(np.float64))
        g = 32.0 * d * sc                                   # per 16-group
        return (g[..., 0::2] + g[..., 1::2]).reshape(len(rows), idim // 32)
    _, mins = dq.dequant_rows(qtype, W, od, idim, rows)
    return np.zeros((len(rows), idim // 32)) if mins is None else np.abs(mins)


def _bound_check(qtype, W, od, idim, x, got, ts, rs, blk, d, q, s, what):
    """got[i] for points (ts[i], rs[i]); d, q, s: the quantized activations (blk values
    per scale d; s per 32 values, or None)."""
    rows, rinv = np.unique(rs, return_inverse=True)
    Wd, _ = dq.dequant_rows(qtype, W, od, idim, rows)            # [R][idim]
    off = _offsets(qtype, W, od, idim, rows)                       # [R][idim/32]
    xd = np.repeat(d.astype(np.float64), blk, axis=1) * q.astype(np.float64)   # x_deq [nt][idim]
    n_terms = idim // 16 if qtype in (2, 3) else idim // 32
    bad = []
    ratio = 0.0
    for i, (t, ri) in enumerate(zip(ts, rinv)):
        w = Wd[ri]
        exact = float(np.dot(w, x[t].astype(np.float64)))
        absw_blk = np.abs(w).reshape(-1, blk).sum(axis=1)
        act = float(np.dot(d[t].astype(np.float64) * (0.5 + 2.0 ** -17), absw_blk))
        off_el = np.repeat(off[ri], 32)
        prod = float(np.dot(np.abs(w) + off_el, np.abs(xd[t])))
        sround = U * float(np.dot(off[ri], np.abs(s[t].astype(np.float64)))) if s is not None else 0.0
        bound = act + sround + (n_terms + 4) * U * prod * 1.01 + U * abs(exact)
        err = abs(float(got[i]) - exact)
        ratio = max(ratio, err / bound)
        if err > bound:
            bad.append((int(t), int(rs[i]), float(got[i]), exact, bound))
    print(f"{what}: {len(ts)} outputs, max error / bound = {ratio:.4f}", flush=True)
    assert not bad, f"{what}: {len(bad)} outputs outside the bound, first {bad[0]}"
    return ratio


def _points(nt, od, full, seed, nts=16, nrows=96):
    if full:
        tt, rr = np.meshgrid(np.arange(nt), np.arange(od), indexing="ij")
        return tt.reshape(-1), rr.reshape(-1)
    rng = np.random.default_rng(seed)
    ts = np.unique(np.concatenate([rng.choice(nt, size=min(nt, nts), replace=False), [0, nt - 1]]))
    rs = np.unique(np.concatenate([rng.choice(od, size=min(od, nrows), replace=False), [0, od - 1]]))
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    return tt.reshape(-1), rr.reshape(-1)


Q4, Q6, Q6P, Q40, Q80, Q5 = (qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q6_K_P224, qmm.QMM_TYPE_Q4_0,
                             qmm.QMM_TYPE_Q8_0, qmm.QMM_TYPE_Q5_K)

# (label, type, od, id, nt, outlier fraction, seed, every output)
CASES = [
    ("Q4_K 1024x4096 nt=1 (decode GEMV)", Q4, 1024, 4096, 1, 0.0, 0, True),
    ("Q4_K 100x512 nt=13", Q4, 100, 512, 13, 0.01, 1, True),
    ("Q4_K 7x2304 nt=64", Q4, 7, 2304, 64, 0.0, 2, True),
    ("Q6_K 257x768 nt=9", Q6, 257, 768, 9, 0.0, 3, True),
    ("Q6_K padded 64x1024 nt=20", Q6P, 64, 1024, 20, 0.01, 4, True),
    ("Q5_K 64x1024 nt=3", Q5, 64, 1024, 3, 0.0, 5, True),
    ("Q4_0 96x768 nt=17", Q40, 96, 768, 17, 0.0, 6, True),
    ("Q8_0 80x512 nt=2", Q80, 80, 512, 2, 0.0, 7, True),
    ("Q4_K 12288x4096 nt=8 (decode, sampled)", Q4, 12288, 4096, 8, 0.0, 8, False),
    ("Q6_K 32000x4096 nt=1 (output head, sampled)", Q6, 32000, 4096, 1, 0.0, 9, False),
    ("Q4_K 12288x4096 nt=512 (prefill, sampled)", Q4, 12288, 4096, 512, 0.01, 10, False),
    ("Q4_K 4096x12288 nt=512 (prefill, sampled)", Q4, 4096, 12288, 512, 0.01, 11, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_matmul_within_activation_quantization_bound(case):
    label, qtype, od, idim, nt, outl, seed, full = case
    print(f"case {label}", flush=True)
    base = qtype if qtype != Q6P else Q6
    W = synth.weights(base, od, idim, seed=seed)
    Wg = _up(W)
    if qtype == Q6P:
        Wg = qmm.qmm_pad_q6k(Wg)
        W = Wg.cpu().numpy()
    x = synth.activations(nt, idim, seed=seed + 100, outlier_frac=outl)
    out = qmm.qmm_matmul(qtype, Wg, _up(x), od).cpu().numpy()
    q, d, s = oracle.quantize(x)
    ts, rs = _points(nt, od, full, seed)
    _bound_check(qtype, W, od, idim, x, out[ts, rs], ts, rs, 32, d, q, s, label)


Q8K_CASES = [
    ("Q4_K 12288x4096 nt=512 Q8_K (sampled)", Q4, 12288, 4096, 512, 0.01, 12, False),
    ("Q6_K padded 4096x12288 nt=512 Q8_K (sampled)", Q6P, 4096, 12288, 512, 0.01, 13, False),
    ("Q5_K 96x1024 nt=40 Q8_K", Q5, 96, 1024, 40, 0.0, 14, True),
]


@pytest.mark.parametrize("case", Q8K_CASES, ids=[c[0] for c in Q8K_CASES])
def test_q8k_matmul_within_activation_quantization_bound(case):
    """The same bound with one activation scale per 256 values; the group sums are
    exact integers, so no rounded s enters."""
    label, qtype, od, idim, nt, outl, seed, full = case
    print(f"case {label}", flush=True)
    base = qtype if qtype != Q6P else Q6
    W = synth.weights(base, od, idim, seed=seed)
    Wg = _up(W)
    if qtype == Q6P:
        Wg = qmm.qmm_pad_q6k(Wg)
        W = Wg.cpu().numpy()
    x = synth.activations(nt, idim, seed=seed + 100, outlier_frac=outl)
    qg, dg, bg = qmm.qmm_quantize_act_q8k(_up(x))
    out = qmm.qmm_matmul_q8k(qtype, Wg, qg, dg, bg, od).cpu().numpy()
    q, d, _ = oracle.quantize_q8k(x)
    ts, rs = _points(nt, od, full, seed)
    _bound_check(qtype, W, od, idim, x, out[ts, rs], ts, rs, 256, d, q, None, label)


def _rms_f64(x, w, eps):
    x = x.astype(np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps) * w.astype(np.float64)


RMS_CASES = [(3, 4096, 1e-5), (2, 1056, 0.5), (4, 2048, 1e-6), (1, 32, 0.25), (512, 4096, 1e-5),
             (2, 16384, 1e-5), (2, 20480, 1e-5), (1, 12288, 1e-6)]


@pytest.mark.parametrize("nt,n,eps", RMS_CASES)
@pytest.mark.parametrize("add", [False, True])
def test_rmsnorm_against_f64_definition(nt, n, eps, add):
    """y (the f32 values the fused kernels quantize) against f64 x / sqrt(mean x^2 + eps) * w.
    With add, the input is the residual update h + o (one f32 add, compared bit for bit)."""
    print(f"case rmsnorm nt={nt} n={n} eps={eps} add={add}", flush=True)
    x = synth.activations(nt, n, seed=60 + n, outlier_frac=0.01)
    w = (1.0 + 0.1 * synth.activations(1, n, seed=70 + n)[0]).astype(np.float32)
    xg = _up(x)
    if add:
        o = synth.activations(nt, n, seed=80 + n)
        qmm.qmm_residual_add(xg, _up(o))
        h = xg.cpu().numpy()
        assert np.array_equal(h, (x + o).astype(np.float32)), "residual update is not one f32 add"
        x = h
    y = qmm.qmm_rmsnorm(xg, _up(w), eps).cpu().numpy().astype(np.float64)
    ref = _rms_f64(x, w, eps)
    c = 1.1 * ((n / 256 + 10) / 2 + 4)
    bound = c * U * np.abs(ref) + 1e-37
    ratio = float(np.max(np.abs(y - ref) / bound))
    print(f"rmsnorm nt={nt} n={n}: max error / bound = {ratio:.4f}", flush=True)
    assert ratio <= 1.0
