"""GPU parity of the Q8_K path (activations with one scale per 256 values), through
the C ABI.

Page: "The quantized GEMM" (mojo-dllm kernels page), "Activations: int8 with a
scale per 256" and "The zero points do not touch the inner loop".

* qmm_quantize_act_q8k: q, d and the 16-value group sums bit-exact against the
  oracle (crafted blocks, ragged token counts, zero / subnormal / huge blocks, the
  full prefill plane);
* qmm_q8k_superblock_sums: the integer stage bit-exact against the oracle -- Q4_K
  and Q5_K: sum_j sc_j * sum(q*qx) and sum_j m_j * (bsum_2j + bsum_2j+1); Q6_K
  (both layouts): sum_g sc_g * sum((q6 - 32) * qx) and 0;
* qmm_matmul_q8k: f32 outputs within |g - o| <= 1e-5 * max(|o|, A / sqrt(n))
  of the oracle's f64 combine, for Q4_K, Q5_K and Q6_K in both layouts, over
  several tiles and ragged tails in every dimension, one token, one super-block,
  long rows, and the benchmark's prefill shapes on a sampled set of outputs;
* qmm_matmul_q8k_kind: every tile shape, the split over K included, against the
  oracle; the default call equals its chosen tile's call bit for bit.
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
Q4, Q6, P6, Q5 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q6_K_P224, qmm.QMM_TYPE_Q5_K
DEV = "cuda:0"


def _weights(qtype, od, idim, seed):
    """(device bytes, host bytes for the oracle, oracle type): the padded layout
    puts 14 zero bytes after each 210-byte Q6_K block; the oracle reads the
    unpadded blocks."""
    W = synth.weights(Q6 if qtype == P6 else qtype, od, idim, seed=seed)
    if qtype != P6:
        return _up(W), W, qtype
    b = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1, 210)
    pad = np.zeros((b.shape[0], 224), np.uint8)
    pad[:, :210] = b
    return _up(pad.reshape(-1)), W, Q6


def _say(*a):
    print(*a, flush=True)


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape and a.dtype == b.dtype, what
    if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
        bad = np.argwhere(a.view(np.uint8).reshape(a.shape + (-1,)) != b.view(np.uint8).reshape(b.shape + (-1,)))
        k = tuple(bad[0][:-1])
        raise AssertionError(f"{what}: differs at {k}: {a[k]!r} vs {b[k]!r}")


def _quant(x):
    q, d, bs = qmm.qmm_quantize_act_q8k(_up(x))
    torch.cuda.synchronize()
    return q, d, bs


QSHAPES = [(1, 256), (3, 1024), (7, 4096), (33, 2304), (512, 4096), (512, 12288)]


@pytest.mark.parametrize("nt,idim", QSHAPES, ids=[f"{a}x{b}" for a, b in QSHAPES])
def test_quantize_q8k_bit_exact(nt, idim):
    _say(f"quantize_q8k nt={nt} id={idim}")
    x = synth.activations(nt, idim, seed=1000 + nt + idim, outlier_frac=0.01)
    ref = oracle.quantize_q8k(x)
    got = [t.cpu().numpy() for t in _quant(x)]
    for name, g, r in zip(("q", "d", "bsum"), got, ref):
        _same(g, r, f"{nt}x{idim} {name}")


def test_quantize_q8k_edge_blocks():
    """Whole 256-blocks zero, with subnormal scale, near 1e30; and hand-made ties."""
    nt, idim = 4, 2048
    x = synth.activations(nt, idim, seed=1100).reshape(nt, idim // 256, 256)
    x[:, 0] = 0.0
    x[:, 1] *= np.float32(1e-39)
    x[:, 2] *= np.float32(1e-3)
    x[:, 3] *= np.float32(1e30)
    x[0, 4] = np.where(np.arange(256) % 2 == 0, 2.5, -2.5)
    x[0, 4, 0] = 127.0
    x = np.ascontiguousarray(x.reshape(nt, idim), dtype=np.float32)
    ref = oracle.quantize_q8k(x)
    got = [t.cpu().numpy() for t in _quant(x)]
    for name, g, r in zip(("q", "d", "bsum"), got, ref):
        _same(g, r, f"edge {name}")
    assert np.all(got[1][:, 0] == 0) and np.all(got[2][:, :16] == 0)
    assert got[2][0, 64] == 124.0


SHAPES = [(1, 1, 256), (5, 7, 512), (9, 100, 768), (64, 128, 1024), (70, 257, 2304), (130, 96, 4096),
          (3, 4096, 4096), (200, 300, 256)]
SHAPES6 = [(1, 1, 256), (9, 100, 768), (64, 128, 1024), (70, 257, 2304), (130, 96, 4096), (200, 300, 256)]
TYPED = [(Q4,) + c for c in SHAPES] + [(qt,) + c for qt in (Q6, P6, Q5) for c in SHAPES6]
TYPED_IDS = [f"t{q}-{a}x{b}x{c}" for q, a, b, c in TYPED]


@pytest.mark.parametrize("qtype,nt,od,idim", TYPED, ids=TYPED_IDS)
def test_q8k_superblock_sums_bit_exact(qtype, nt, od, idim):
    _say(f"q8k integer stage type={qtype} nt={nt} od={od} id={idim}")
    Wd, W, ot = _weights(qtype, od, idim, seed=1200 + od)
    x = synth.activations(nt, idim, seed=1300 + nt, outlier_frac=0.01)
    q, d, bs = _quant(x)
    S = qmm.qmm_q8k_superblock_sums(qtype, Wd, q, d, bs, od)
    torch.cuda.synchronize()
    # the oracle's reference runs on the oracle's own quantization of x, which the
    # GPU's must equal bit for bit
    oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
    ref = oracle.q8k_superblock_sums(ot, W, oq, obs, od)
    _same(S.cpu().numpy(), ref, "integer stage")


@pytest.mark.parametrize("qtype,nt,od,idim", TYPED, ids=TYPED_IDS)
def test_matmul_q8k_against_oracle(qtype, nt, od, idim):
    _say(f"matmul_q8k type={qtype} nt={nt} od={od} id={idim}")
    Wd, W, ot = _weights(qtype, od, idim, seed=1400 + od)
    x = synth.activations(nt, idim, seed=1500 + nt, outlier_frac=0.01)
    q, d, bs = _quant(x)
    out = qmm.qmm_matmul_q8k(qtype, Wd, q, d, bs, od)
    torch.cuda.synchronize()
    oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
    ref, mag = oracle.matmul_q8k(ot, W, oq, od_, obs, od)
    worst, rel = assert_close(out.cpu().numpy(), ref, mag, ot, idim, f"{nt}x{od}x{idim}")
    _say(f"  worst err/tol {worst:.3f}, max rel {rel:.2e}")


FULL = [(Q4, 12288, 4096, 512), (Q4, 4096, 12288, 512), (Q4, 12288, 4096, 256), (Q4, 40, 65536, 17),
        (Q6, 4096, 12288, 512), (P6, 4096, 12288, 256), (P6, 32000, 4096, 64), (Q6, 40, 65536, 17),
        (Q5, 12288, 4096, 512), (Q5, 4096, 12288, 256)]


@pytest.mark.parametrize("qtype,od,idim,nt", FULL, ids=[f"t{q}-{a}x{b}-{c}" for q, a, b, c in FULL])
def test_matmul_q8k_full_size_sampled(qtype, od, idim, nt):
    _say(f"matmul_q8k full size type={qtype} od={od} id={idim} nt={nt}")
    Wd, W, ot = _weights(qtype, od, idim, seed=1600 + od)
    x = synth.activations(nt, idim, seed=1700 + nt, outlier_frac=0.01)
    q, d, bs = _quant(x)
    qn, dn, bn = q.cpu().numpy(), d.cpu().numpy(), bs.cpu().numpy()
    ref_q = oracle.quantize_q8k(x)
    for name, g, r in zip(("q", "d", "bsum"), (qn, dn, bn), ref_q):
        _same(g, r, f"full-size quantize {name}")
    out = qmm.qmm_matmul_q8k(qtype, Wd, q, d, bs, od).cpu().numpy()
    rng = np.random.default_rng(od + nt)
    ts = np.unique(np.concatenate([rng.choice(nt, size=min(nt, 24), replace=False), [0, nt - 1]]))
    rs = np.unique(np.concatenate([rng.choice(od, size=min(od, 160), replace=False), [0, od - 1]]))
    tt, rr = np.meshgrid(ts, rs, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    ref, mag = oracle.matmul_q8k_points(ot, W, ref_q[0], ref_q[1], ref_q[2], od, tt, rr)
    worst, rel = assert_close(out[tt, rr], ref, mag, ot, idim, f"full size {od}x{idim} nt={nt}")
    _say(f"  worst err/tol {worst:.3f}, max rel {rel:.2e}")


KIND_SHAPES = [(1, 1, 256), (9, 100, 768), (64, 128, 1024), (70, 257, 2304), (130, 96, 4096), (65, 200, 1280)]
KINDS = [(qt, kind) + c for qt in (Q4, Q6, P6, Q5)
         for kind in (qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK)
         for c in KIND_SHAPES]


@pytest.mark.parametrize("qtype,kind,nt,od,idim", KINDS, ids=[f"t{q}-k{k}-{a}x{b}x{c}" for q, k, a, b, c in KINDS])
def test_matmul_q8k_every_tile(qtype, kind, nt, od, idim):
    """Each tile shape, the split over K included (odd super-block counts leave the
    second group a super-block past the end; one super-block leaves it nothing),
    against the oracle; the default call equals its own tile's call bit for bit."""
    _say(f"matmul_q8k kind={kind} type={qtype} nt={nt} od={od} id={idim}")
    Wd, W, ot = _weights(qtype, od, idim, seed=2000 + od + kind)
    x = synth.activations(nt, idim, seed=2100 + nt, outlier_frac=0.01)
    q, d, bs = _quant(x)
    out = qmm.qmm_matmul_q8k_kind(kind, qtype, Wd, q, d, bs, od)
    auto = qmm.qmm_matmul_q8k(qtype, Wd, q, d, bs, od)
    same = qmm.qmm_matmul_q8k_kind(qmm.qmm_q8k_tile(nt, od, idim), qtype, Wd, q, d, bs, od)
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int32), same.view(torch.int32))
    oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
    ref, mag = oracle.matmul_q8k(ot, W, oq, od_, obs, od)
    worst, rel = assert_close(out.cpu().numpy(), ref, mag, ot, idim, f"kind {kind} {nt}x{od}x{idim}")
    _say(f"  worst err/tol {worst:.3f}, max rel {rel:.2e}")


WKINDS = [(kind, base) + c
          for kind, base in ((qmm.QMM_KIND_MMQ_WAVE32X64, qmm.QMM_KIND_MMQ_128X64),
                             (qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK, qmm.QMM_KIND_MMQ_64X64_SPLITK))
          for c in KIND_SHAPES + [(64, 384, 3328), (130, 1000, 512)]]


@pytest.mark.parametrize("kind,base,nt,od,idim", WKINDS, ids=[f"k{k}-{a}x{b}x{c}" for k, _, a, b, c in WKINDS])
def test_matmul_q8k_wave_kernels(kind, base, nt, od, idim):
    """Q4_K on the wave kernels with the sub-block scales in the int8 operand (and
    their split over K): against the oracle, and bit for bit against the staged
    kernel of the same summation order (128 x 64, or the 64 x 64 split)."""
    _say(f"matmul_q8k wave kind={kind} nt={nt} od={od} id={idim}")
    Wd, W, ot = _weights(Q4, od, idim, seed=2400 + od + kind)
    x = synth.activations(nt, idim, seed=2500 + nt, outlier_frac=0.01)
    q, d, bs = _quant(x)
    out = qmm.qmm_matmul_q8k_kind(kind, Q4, Wd, q, d, bs, od)
    ref_same = qmm.qmm_matmul_q8k_kind(base, Q4, Wd, q, d, bs, od)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref_same.view(torch.int32))
    oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
    ref, mag = oracle.matmul_q8k(ot, W, oq, od_, obs, od)
    worst, rel = assert_close(out.cpu().numpy(), ref, mag, ot, idim, f"wave kind {kind} {nt}x{od}x{idim}")
    _say(f"  worst err/tol {worst:.3f}, max rel {rel:.2e}")


def test_q8k_wave_integer_stage_bit_exact():
    """The integer stage of the wave kernel (S1 = 8 Ca + Cb from the two chained
    accumulators, and S2): qmm_q8k_superblock_sums takes it where qmm_matmul_q8k
    does (Q4_K, more than 256 tiles of 128 x 64, whichever tile the cost model
    names); ragged rows and tokens, three
    super-blocks (the two-per-trip loop with an odd count)."""
    nt, od, idim = 50, 33243, 768
    _say(f"q8k wave integer stage nt={nt} od={od} id={idim}")
    Wd, W, ot = _weights(Q4, od, idim, seed=2600)
    x = synth.activations(nt, idim, seed=2700, outlier_frac=0.01)
    q, d, bs = _quant(x)
    S = qmm.qmm_q8k_superblock_sums(Q4, Wd, q, d, bs, od)
    torch.cuda.synchronize()
    oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
    ref = oracle.q8k_superblock_sums(ot, W, oq, obs, od)
    _same(S.cpu().numpy(), ref, "wave integer stage")


def test_matmul_q8k_split_full_size_sampled():
    """The split tile on the long-K shape it is chosen for (padded Q6_K 4096 x 12288
    at 256 tokens; Q4_K 4096 x 4096 at 256), sampled against the oracle."""
    for qtype, od, idim, nt in ((P6, 4096, 12288, 256), (Q4, 4096, 4096, 256)):
        assert qmm.qmm_q8k_tile(nt, od, idim) == qmm.QMM_KIND_MMQ_64X64_SPLITK
        _say(f"matmul_q8k split full size type={qtype} od={od} id={idim} nt={nt}")
        Wd, W, ot = _weights(qtype, od, idim, seed=2200 + od)
        x = synth.activations(nt, idim, seed=2300 + nt, outlier_frac=0.01)
        q, d, bs = _quant(x)
        out = qmm.qmm_matmul_q8k(qtype, Wd, q, d, bs, od).cpu().numpy()
        rng = np.random.default_rng(od + nt + 7)
        ts = np.unique(np.concatenate([rng.choice(nt, size=24, replace=False), [0, nt - 1]]))
        rs = np.unique(np.concatenate([rng.choice(od, size=160, replace=False), [0, od - 1]]))
        tt, rr = np.meshgrid(ts, rs, indexing="ij")
        tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
        oq, od_, obs = oracle_activations(oracle.quantize_q8k, x, (q, d, bs), "quantize_q8k")
        ref, mag = oracle.matmul_q8k_points(ot, W, oq, od_, obs, od, tt, rr)
        assert_close(out[tt, rr], ref, mag, ot, idim, f"split full size {od}x{idim} nt={nt}")


def test_q8k_padded_equals_unpadded():
    """The padded Q6_K layout gives the unpadded one's outputs bit for bit (same
    arithmetic in the same order), on both tile shapes."""
    for nt, od, idim in ((64, 4096, 4096), (512, 4096, 4096), (17, 300, 2304)):
        _say(f"matmul_q8k padded vs unpadded nt={nt} od={od} id={idim}")
        W = synth.weights(Q6, od, idim, seed=1900 + nt)
        q, d, bs = _quant(synth.activations(nt, idim, seed=1910 + nt))
        a = qmm.qmm_matmul_q8k(Q6, _up(W), q, d, bs, od)
        b = qmm.qmm_matmul_q8k(P6, qmm.qmm_pad_q6k(_up(W)), q, d, bs, od)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_q8k_rejects_other_types():
    q, d, bs = _quant(synth.activations(1, 256, seed=1800))
    for qt, nbytes in ((qmm.QMM_TYPE_Q4_0, 144), (qmm.QMM_TYPE_Q8_0, 272)):
        W = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        with pytest.raises(qmm.QmmError) as e:
            qmm.qmm_matmul_q8k(qt, W, q, d, bs, 1)
        assert e.value.status == qmm.QMM_ERR_TYPE
