"""GPU parity of the stream-K matrix kernel (Q4_K, Q6_K in both layouts), through the C ABI.

The (tile, super-block) units of a launch are cut into equal ranges, one per
workgroup; tiles split between workgroups are added by a fixup kernel in a fixed
order ("llama.cpp MMQ" page, section 12.3, on tile counts that leave CUs idle; the
pages warn that split reductions must not make results depend on timing).

* outputs within |g - o| <= 1e-5 * max(|o|, A / sqrt(n)) of the oracle, for shapes
  with fewer units than workgroups, tiles split over several workgroups, ranges
  spanning several tiles, ragged edges, and the benchmark's shapes;
* determinism: repeated launches are bit-identical;
* the workspace is filled with NaN bytes before each launch: every partial read
  was written in that launch;
* a launch after one of another shape on the same workspace gives the same bits as
  one on a fresh workspace.
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
Q4, Q6, P6 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q6_K_P224
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _weights(qtype, od, idim, seed):
    """Host weight bytes of the type (the padded layout: each 210-byte Q6_K block
    followed by 14 zero bytes), as the oracle and the kernels take them."""
    W = synth.weights(Q6 if qtype == P6 else qtype, od, idim, seed=seed)
    if qtype != P6:
        return W
    b = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1, 210)
    out = np.zeros((b.shape[0], 224), np.uint8)
    out[:, :210] = b
    return out.reshape(-1)


CASES = [(1, 1, 256), (9, 100, 768), (64, 128, 1024), (17, 40, 65536), (300, 1000, 2304), (130, 96, 4096),
         (256, 4096, 4096), (256, 12288, 4096), (512, 12288, 4096), (512, 4096, 12288)]


CASES6 = [(1, 1, 256), (9, 100, 768), (17, 40, 65536), (300, 1000, 2304), (130, 96, 4096), (64, 4096, 4096),
          (192, 12288, 4096), (17, 4096, 12288)]
TYPED = [(Q4,) + c for c in CASES] + [(qt,) + c for qt in (Q6, P6) for c in CASES6]


@pytest.mark.parametrize("qtype,nt,od,idim", TYPED, ids=[f"t{q}-{a}x{b}x{c}" for q, a, b, c in TYPED])
def test_streamk(qtype, nt, od, idim):
    print(f"stream-K type={qtype} nt={nt} od={od} id={idim}", flush=True)
    W = _weights(qtype, od, idim, seed=4000 + od)
    x = synth.activations(nt, idim, seed=4100 + nt, outlier_frac=0.01)
    Wt = _up(W)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    ws = torch.full((qmm.qmm_streamk_ws_bytes(),), 0xFF, dtype=torch.uint8, device=DEV)
    a = qmm.qmm_matmul_q8_streamk(qtype, Wt, q, d, s, od, ws)
    ws.fill_(0xFF)  # a partial read before it is written in this launch shows as NaN
    b = qmm.qmm_matmul_q8_streamk(qtype, Wt, q, d, s, od, ws)
    torch.cuda.synchronize()
    an = a.cpu().numpy()
    assert np.array_equal(an.view(np.uint32), b.cpu().numpy().view(np.uint32)), "not deterministic"
    assert np.all(np.isfinite(an))
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    if nt * od <= 300 * 1000:
        ref, mag = oracle.matmul_q8(qtype, W, qn, dn, sn, od)
        assert_close(an, ref, mag, qtype, idim, "stream-K vs oracle")
    else:
        rng = np.random.default_rng(od + nt)
        ts = np.unique(np.concatenate([rng.choice(nt, 24, replace=False), [0, nt - 1]]))
        rs = np.unique(np.concatenate([rng.choice(od, 160, replace=False), [0, od - 1]]))
        tt, rr = np.meshgrid(ts, rs, indexing="ij")
        tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
        ref, mag = oracle.matmul_q8_points(qtype, W, qn, dn, sn, od, tt, rr)
        assert_close(an[tt, rr], ref, mag, qtype, idim, "stream-K vs oracle (sampled)")


PATH_CASES = [(Q4, 20, 96, 8192), (Q4, 9, 40, 65536), (Q4, 300, 1000, 2304), (Q4, 384, 4096, 12288),
              (Q4, 512, 4096, 12288), (Q4, 384, 12288, 4096), (Q4, 512, 12288, 4096), (Q4, 128, 12288, 4096),
              (Q6, 64, 4096, 4096), (Q6, 192, 4096, 4096), (Q6, 20, 96, 8192), (P6, 192, 12288, 4096),
              (P6, 128, 12288, 4096), (P6, 256, 4096, 12288), (P6, 128, 4096, 12288),
              # Q4_K within one round of the 4-wave kernel (per tile there), and beside it
              (Q4, 256, 12288, 4096), (Q4, 448, 8192, 4096), (Q4, 320, 8192, 4096), (P6, 256, 12288, 4096),
              # Q4_K on 192..256 tiles of 128 x 64: the 4-wave kernel split over K per tile
              (Q4, 512, 4096, 8192), (Q4, 448, 4096, 12288)]


@pytest.mark.parametrize("qtype,nt,od,idim", PATH_CASES, ids=[f"t{q}-{a}x{b}x{c}" for q, a, b, c in PATH_CASES])
def test_qmm_matmul_takes_streamk_where_preferred(qtype, nt, od, idim):
    """qmm_matmul with a workspace of qmm_matmul_ws_bytes runs the stream-K kernel
    exactly where qmm_streamk_preferred says so (same bits as the stream-K entry
    point on the same quantized input), the per-tile kernel elsewhere and with a
    workspace of only the q8 plane (same bits as qmm_matmul_q8); outputs within the
    tolerance of the oracle."""
    pref = qmm.qmm_streamk_preferred(qtype, nt, od, idim)
    print(f"qmm_matmul path type={qtype} nt={nt} od={od} id={idim} stream-K preferred={pref}", flush=True)
    mmq = qmm.qmm_dispatch_kind(qtype, nt, od, idim) == qmm.QMM_KIND_MMQ
    tiles = -(-nt // 64) * -(-od // 128)
    slots = 256 * -(-tiles // 256)
    rule = ((slots - tiles) * 10 >= slots if tiles > 256 else
            ((idim // 256 >= 32 and tiles != 128) or (qtype != Q4 and tiles <= 64)))
    # Q4_K runs the 4-wave kernel (two workgroups per CU, 512 tiles a round) on more
    # than 256 tiles where the cost model names 128 x 64, or names the split with
    # 384..512 tiles; within one such round it stays per tile
    wave = (qtype == Q4 and mmq and tiles > 256 and
            (qmm.qmm_mmq_tile(nt, od, idim) == qmm.QMM_KIND_MMQ_128X64 or 384 <= tiles <= 512))
    assert pref == (mmq and tiles % 256 != 0 and rule and not (wave and tiles <= 512))
    split = (qtype == Q4 and mmq and not wave and 192 <= tiles <= 256 and
             qmm.qmm_mmq_tile(nt, od, idim) == qmm.QMM_KIND_MMQ_128X64)
    W = _weights(qtype, od, idim, seed=4200 + od)
    x = synth.activations(nt, idim, seed=4300 + nt, outlier_frac=0.01)
    Wt, xt = _up(W), _up(x)
    full = qmm.qmm_matmul(qtype, Wt, xt, od)   # workspace of qmm_matmul_ws_bytes
    small = qmm.qmm_matmul(qtype, Wt, xt, od,
                           workspace=torch.empty(qmm.qmm_act_bytes(nt, idim), dtype=torch.uint8, device=DEV))
    q, d, s = qmm.qmm_quantize_act(xt)
    ws = torch.empty(qmm.qmm_streamk_ws_bytes(), dtype=torch.uint8, device=DEV)
    sk = qmm.qmm_matmul_q8_streamk(qtype, Wt, q, d, s, od, ws)
    pt = qmm.qmm_matmul_q8(qtype, Wt, q, d, s, od)
    wv = (qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_WAVE32X64, qtype, Wt, q, d, s, od) if wave else
          qmm.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK, qtype, Wt, q, d, s, od) if split else None)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32)
    assert torch.equal(bits(full), bits(sk if pref else pt))
    assert torch.equal(bits(small), bits(pt))
    if wave or split:
        assert torch.equal(bits(pt), bits(wv))
    qn, dn, sn = oracle_activations(oracle.quantize, x, (q, d, s), "quantize")
    if nt * od <= 300 * 1000:
        ref, mag = oracle.matmul_q8(qtype, W, qn, dn, sn, od)
        assert_close(full.cpu().numpy(), ref, mag, qtype, idim, "qmm_matmul vs oracle")
    else:
        rng = np.random.default_rng(od + nt + 1)
        ts = np.unique(np.concatenate([rng.choice(nt, 16, replace=False), [0, nt - 1]]))
        rs = np.unique(np.concatenate([rng.choice(od, 128, replace=False), [0, od - 1]]))
        tt, rr = np.meshgrid(ts, rs, indexing="ij")
        tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
        ref, mag = oracle.matmul_q8_points(qtype, W, qn, dn, sn, od, tt, rr)
        assert_close(full.cpu().numpy()[tt, rr], ref, mag, qtype, idim, "qmm_matmul vs oracle (sampled)")


def test_streamk_workspace_reuse_across_shapes():
    """Partials left by launches of other shapes (and other types) on the same
    workspace change nothing: each launch equals, bit for bit, a launch on a
    workspace of NaN bytes."""
    print("stream-K workspace reuse across shapes", flush=True)
    shapes = [(Q4, 64, 4096, 4096), (Q6, 130, 96, 4096), (Q4, 256, 12288, 4096), (P6, 17, 4096, 12288),
              (Q4, 64, 4096, 4096)]
    ws = torch.full((qmm.qmm_streamk_ws_bytes(),), 0xFF, dtype=torch.uint8, device=DEV)
    for i, (qtype, nt, od, idim) in enumerate(shapes):
        Wt = _up(_weights(qtype, od, idim, seed=4400 + i))
        q, d, s = qmm.qmm_quantize_act(_up(synth.activations(nt, idim, seed=4500 + i)))
        shared = qmm.qmm_matmul_q8_streamk(qtype, Wt, q, d, s, od, ws)
        fresh = qmm.qmm_matmul_q8_streamk(qtype, Wt, q, d, s, od,
                                          torch.full_like(ws, 0xFF))
        torch.cuda.synchronize()
        assert torch.equal(shared.view(torch.int32), fresh.view(torch.int32)), (qtype, nt, od, idim)
        assert bool(torch.isfinite(shared).all())
