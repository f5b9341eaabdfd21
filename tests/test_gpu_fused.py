"""GPU parity of the producer-side steps fused with the quantizer, through the C ABI.

Page: "The quantized GEMM" (mojo-dllm kernels page), The GPU path, "Fused
elementwise kernels": the fused kernels (residual add + RMS norm + quantize, RMS
norm + quantize, silu(g) * u + quantize) must give exactly what the unfused chain
gives.  Checked here, every comparison bit for bit:

* fused q, d, s == the unfused chain on the GPU (qmm_residual_add, qmm_rmsnorm or
  qmm_silu_mul, then qmm_quantize_act);
* the chain's f32 values == the oracle's (fixed f32 sum order for the norm; f64
  silu * u rounded once);
* fused q, d, s == the oracle quantizer applied to the oracle's f32 values;
* the updated residual h == the oracle's h + o;
* the Q8_K variants (the same steps ending in the Q8_K quantizer): q, d and the
  16-value group sums == the chain ending in qmm_quantize_act_q8k and == the
  oracle's Q8_K quantizer on the oracle's f32 values.

Shapes cover every register-resident row length class (up to 16384 values), the
two-pass path for longer rows, ragged row lengths (not a multiple of 1024), one
row and many rows, and the benchmark's full shapes (512 x 4096 norms, 512 x 12288
silu).  Edge cases: zero rows, eps = 0, tiny and huge magnitudes, in-place y = x,
o aliasing h, large |g|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    return t.cpu().numpy()


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, f"{what}: {a.shape} {a.dtype} vs {b.shape} {b.dtype}"
    eq = a.view(np.uint8).reshape(a.shape + (-1,)) == b.view(np.uint8).reshape(b.shape + (-1,))
    if not np.all(eq):
        bad = np.argwhere(~np.all(eq, axis=-1))
        k = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ, first at {k}: {a[k]!r} vs {b[k]!r}")


def _same_q8(got, ref, what):
    for name, g, r in zip("qds", got, ref):
        _same(g, r, f"{what} {name}")


def _rows(nt, idim, seed, scale=1.0):
    return synth.activations(nt, idim, seed=seed, outlier_frac=0.01) * np.float32(scale)


def _weight(idim, seed):
    return (np.float32(1.0) + np.float32(0.25) * synth.activations(1, idim, seed=seed)[0]).astype(np.float32)


NORM_SHAPES = [(1, 32), (1, 4096), (3, 1056), (5, 2080), (7, 4096), (2, 12288), (1, 16384), (2, 20480),
               (1, 65536), (64, 4096), (33, 3104), (512, 4096)]


@pytest.mark.parametrize("nt,idim", NORM_SHAPES, ids=[f"{a}x{b}" for a, b in NORM_SHAPES])
def test_add_rmsnorm_quantize(nt, idim):
    _say(f"add_rmsnorm_quantize nt={nt} id={idim}")
    eps = 1e-5
    h = _rows(nt, idim, 100 + idim + nt)
    o = _rows(nt, idim, 200 + idim + nt, scale=0.5)
    w = _weight(idim, 300 + idim)
    ref_h, ref_y = oracle.add_rmsnorm(h, o, w, eps)
    ref_q8 = oracle.quantize(ref_y)

    hf, ot, wt = _up(h), _up(o), _up(w)
    got = qmm.qmm_add_rmsnorm_quantize(hf, ot, wt, eps)
    # unfused chain on the GPU
    hc = _up(h)
    qmm.qmm_residual_add(hc, ot)
    yc = qmm.qmm_rmsnorm(hc, wt, eps)
    chain = qmm.qmm_quantize_act(yc)
    torch.cuda.synchronize()

    _same(_host(hf), ref_h, "fused residual h + o")
    _same(_host(hc), ref_h, "chain residual h + o")
    _same(_host(yc), ref_y, "chain rmsnorm y")
    _same_q8([_host(t) for t in got], [_host(t) for t in chain], "fused vs chain")
    _same_q8([_host(t) for t in got], ref_q8, "fused vs oracle")


@pytest.mark.parametrize("nt,idim", NORM_SHAPES, ids=[f"{a}x{b}" for a, b in NORM_SHAPES])
def test_rmsnorm_quantize(nt, idim):
    _say(f"rmsnorm_quantize nt={nt} id={idim}")
    eps = 1e-6
    x = _rows(nt, idim, 400 + idim + nt, scale=3.0)
    w = _weight(idim, 500 + idim)
    ref_y = oracle.rmsnorm(x, w, eps)
    ref_q8 = oracle.quantize(ref_y)
    xt, wt = _up(x), _up(w)
    got = qmm.qmm_rmsnorm_quantize(xt, wt, eps)
    yc = qmm.qmm_rmsnorm(xt, wt, eps)
    chain = qmm.qmm_quantize_act(yc)
    torch.cuda.synchronize()
    _same(_host(xt), x, "input unchanged")
    _same(_host(yc), ref_y, "chain rmsnorm y")
    _same_q8([_host(t) for t in got], [_host(t) for t in chain], "fused vs chain")
    _same_q8([_host(t) for t in got], ref_q8, "fused vs oracle")


SILU_SHAPES = [(1, 32), (3, 96), (1, 12288), (8, 12288), (13, 4128), (512, 12288)]


@pytest.mark.parametrize("nt,idim", SILU_SHAPES, ids=[f"{a}x{b}" for a, b in SILU_SHAPES])
def test_silu_mul_quantize(nt, idim):
    _say(f"silu_mul_quantize nt={nt} id={idim}")
    g = _rows(nt, idim, 600 + idim + nt, scale=2.0)
    u = _rows(nt, idim, 700 + idim + nt)
    ref_y = oracle.silu_mul(g, u)
    ref_q8 = oracle.quantize(ref_y)
    gt, ut = _up(g), _up(u)
    got = qmm.qmm_silu_mul_quantize(gt, ut)
    yc = qmm.qmm_silu_mul(gt, ut)
    chain = qmm.qmm_quantize_act(yc)
    torch.cuda.synchronize()
    _same(_host(yc), ref_y, "chain silu * u")
    _same_q8([_host(t) for t in got], [_host(t) for t in chain], "fused vs chain")
    _same_q8([_host(t) for t in got], ref_q8, "fused vs oracle")


@pytest.mark.parametrize("idim", [1056, 4096, 20480])
def test_norm_edge_rows(idim):
    """Zero rows (eps > 0 gives zeros; d = q = s = 0), eps = 0 on non-zero rows,
    rows scaled by 1e-20 (squares in the subnormal range) and 1e15, in one call."""
    _say(f"norm edge rows id={idim}")
    nt = 6
    x = _rows(nt, idim, 800 + idim)
    x[0] = 0.0
    x[2] *= np.float32(1e-20)
    x[3] *= np.float32(1e15)
    x[4, : idim // 2] = 0.0
    w = _weight(idim, 801)
    for eps in (1e-5, 0.0):
        xx = x.copy()
        if eps == 0.0:
            xx[0] = 1.0  # eps = 0 needs non-zero rows
        ref_y = oracle.rmsnorm(xx, w, eps)
        assert np.all(np.isfinite(ref_y))
        ref_q8 = oracle.quantize(ref_y)
        xt, wt = _up(xx), _up(w)
        got = qmm.qmm_rmsnorm_quantize(xt, wt, eps)
        yc = qmm.qmm_rmsnorm(xt, wt, eps)
        torch.cuda.synchronize()
        _same(_host(yc), ref_y, f"eps={eps} chain y")
        _same_q8([_host(t) for t in got], ref_q8, f"eps={eps} fused vs oracle")
        if eps > 0:
            assert np.all(_host(got[1])[0] == 0) and np.all(_host(got[0])[0] == 0)


def test_aliasing_in_place():
    """qmm_rmsnorm with y = x, and the residual add with o = h (h becomes 2h)."""
    nt, idim, eps = 4, 2080, 1e-5
    x = _rows(nt, idim, 900)
    w = _weight(idim, 901)
    xt = _up(x)
    qmm.qmm_rmsnorm(xt, _up(w), eps, y=xt)
    h = _up(x)
    q, d, s = qmm.qmm_add_rmsnorm_quantize(h, h, _up(w), eps)
    torch.cuda.synchronize()
    _same(_host(xt), oracle.rmsnorm(x, w, eps), "in-place y = x")
    ref_h, ref_y = oracle.add_rmsnorm(x, x, w, eps)
    _same(_host(h), ref_h, "o = h")
    _same_q8([_host(q), _host(d), _host(s)], oracle.quantize(ref_y), "o = h quantized")


def test_silu_edge_values():
    """g = 0, |g| up to 100 (e^-g over- and underflow in f32 but not in f64), u = 0,
    and a block of tiny products."""
    nt, idim = 2, 256
    g = _rows(nt, idim, 910, scale=4.0)
    u = _rows(nt, idim, 911)
    g[0, :32] = 0.0
    g[0, 32:64] = np.linspace(-100, 100, 32, dtype=np.float32)
    g[0, 64:96] = np.linspace(-30, 30, 32, dtype=np.float32)
    u[1, :32] = 0.0
    u[1, 32:64] *= np.float32(1e-30)
    ref_y = oracle.silu_mul(g, u)
    ref_q8 = oracle.quantize(ref_y)
    gt, ut = _up(g), _up(u)
    got = qmm.qmm_silu_mul_quantize(gt, ut)
    yc = qmm.qmm_silu_mul(gt, ut)
    torch.cuda.synchronize()
    _same(_host(yc), ref_y, "silu * u edge values")
    _same_q8([_host(t) for t in got], ref_q8, "silu edge fused vs oracle")


def test_fused_feeds_matmul():
    """A fused quantized activation is consumed by qmm_matmul_q8 exactly like the
    plain quantizer's (one quantized input serving several weight matrices)."""
    nt, idim, od = 9, 4096, 96
    x = _rows(nt, idim, 920)
    w = _weight(idim, 921)
    xt, wt = _up(x), _up(w)
    q, d, s = qmm.qmm_rmsnorm_quantize(xt, wt, 1e-5)
    q2, d2, s2 = qmm.qmm_quantize_act(qmm.qmm_rmsnorm(xt, wt, 1e-5))
    for qtype in (qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K):
        W = _up(synth.weights(qtype, od, idim, seed=922))
        a = qmm.qmm_matmul_q8(qtype, W, q, d, s, od)
        b = qmm.qmm_matmul_q8(qtype, W, q2, d2, s2, od)
        torch.cuda.synchronize()
        _same(_host(a), _host(b), f"type {qtype} matmul on fused vs chain activations")


# ---- the same steps ending in the Q8_K quantizer (one scale per 256 values):
# fused q, d, bsum == the unfused chain (step, then qmm_quantize_act_q8k) on the
# GPU and == the oracle's Q8_K quantizer applied to the oracle's f32 values; rows
# of whole 256-value blocks (register-resident and two-pass lengths).
Q8K_NORM_SHAPES = [(1, 256), (3, 1024), (7, 4096), (2, 12288), (1, 16384), (2, 20480), (64, 4096), (512, 4096),
                   (5, 2304)]
Q8K_SILU_SHAPES = [(1, 256), (3, 768), (8, 12288), (13, 4352), (512, 12288)]


@pytest.mark.parametrize("nt,idim", Q8K_NORM_SHAPES, ids=[f"{a}x{b}" for a, b in Q8K_NORM_SHAPES])
def test_add_rmsnorm_quantize_q8k(nt, idim):
    _say(f"add_rmsnorm_quantize_q8k nt={nt} id={idim}")
    eps = 1e-5
    h = _rows(nt, idim, 1100 + idim + nt)
    o = _rows(nt, idim, 1200 + idim + nt, scale=0.5)
    w = _weight(idim, 1300 + idim)
    ref_h, ref_y = oracle.add_rmsnorm(h, o, w, eps)
    ref = oracle.quantize_q8k(ref_y)
    hf, ot, wt = _up(h), _up(o), _up(w)
    got = qmm.qmm_add_rmsnorm_quantize_q8k(hf, ot, wt, eps)
    hc = _up(h)
    qmm.qmm_residual_add(hc, ot)
    chain = qmm.qmm_quantize_act_q8k(qmm.qmm_rmsnorm(hc, wt, eps))
    torch.cuda.synchronize()
    _same(_host(hf), ref_h, "fused residual h + o")
    for name, g, c, r in zip(("q", "d", "bsum"), got, chain, ref):
        _same(_host(g), _host(c), f"fused vs chain {name}")
        _same(_host(g), r, f"fused vs oracle {name}")


@pytest.mark.parametrize("nt,idim", Q8K_NORM_SHAPES, ids=[f"{a}x{b}" for a, b in Q8K_NORM_SHAPES])
def test_rmsnorm_quantize_q8k(nt, idim):
    _say(f"rmsnorm_quantize_q8k nt={nt} id={idim}")
    eps = 1e-6
    x = _rows(nt, idim, 1400 + idim + nt, scale=3.0)
    w = _weight(idim, 1500 + idim)
    ref = oracle.quantize_q8k(oracle.rmsnorm(x, w, eps))
    xt, wt = _up(x), _up(w)
    got = qmm.qmm_rmsnorm_quantize_q8k(xt, wt, eps)
    chain = qmm.qmm_quantize_act_q8k(qmm.qmm_rmsnorm(xt, wt, eps))
    torch.cuda.synchronize()
    _same(_host(xt), x, "input unchanged")
    for name, g, c, r in zip(("q", "d", "bsum"), got, chain, ref):
        _same(_host(g), _host(c), f"fused vs chain {name}")
        _same(_host(g), r, f"fused vs oracle {name}")


@pytest.mark.parametrize("nt,idim", Q8K_SILU_SHAPES, ids=[f"{a}x{b}" for a, b in Q8K_SILU_SHAPES])
def test_silu_mul_quantize_q8k(nt, idim):
    _say(f"silu_mul_quantize_q8k nt={nt} id={idim}")
    g = _rows(nt, idim, 1600 + idim + nt, scale=2.0)
    u = _rows(nt, idim, 1700 + idim + nt)
    ref = oracle.quantize_q8k(oracle.silu_mul(g, u))
    gt, ut = _up(g), _up(u)
    got = qmm.qmm_silu_mul_quantize_q8k(gt, ut)
    chain = qmm.qmm_quantize_act_q8k(qmm.qmm_silu_mul(gt, ut))
    torch.cuda.synchronize()
    for name, gg, c, r in zip(("q", "d", "bsum"), got, chain, ref):
        _same(_host(gg), _host(c), f"fused vs chain {name}")
        _same(_host(gg), r, f"fused vs oracle {name}")


def test_q8k_fused_zero_rows_and_shape_errors():
    """A zero row gives d = q = bsum = 0; rows that are not whole 256-value blocks
    are refused."""
    x = _rows(2, 512, 1800)
    x[1] = 0.0
    q, d, bs = qmm.qmm_rmsnorm_quantize_q8k(_up(x), _up(_weight(512, 1801)), 1e-5)
    torch.cuda.synchronize()
    assert not _host(q)[1].any() and not _host(d)[1].any() and not _host(bs)[1].any()
    for fn, args in ((qmm.qmm_rmsnorm_quantize_q8k, (_up(_rows(1, 288, 1802)), _up(_weight(288, 1803)), 1e-5)),
                     (qmm.qmm_silu_mul_quantize_q8k, (_up(_rows(1, 288, 1804)), _up(_rows(1, 288, 1805))))):
        with pytest.raises(qmm.QmmError) as e:
            fn(*args)
        assert e.value.status == qmm.QMM_ERR_SHAPE
