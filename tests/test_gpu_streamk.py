"""GPU parity of the stream-K matrix kernel (Q4_K), through the C ABI.

The (tile, super-block) units of a launch are cut into equal ranges, one per
workgroup; tiles split between workgroups are added by a fixup kernel in a fixed
order ("llama.cpp MMQ" page, section 12.3, on tile counts that leave CUs idle; the
pages warn that split reductions must not make results depend on timing).

* outputs within |g - o| <= 1e-5 * max(|o|, A / sqrt(n)) of the oracle, for shapes
  with fewer units than workgroups, tiles split over several workgroups, ranges
  spanning several tiles, ragged edges, and the benchmark's shapes;
* determinism: repeated launches are bit-identical;
* the workspace is filled with NaN bytes first: every partial read was written.
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
Q4 = qmm.QMM_TYPE_Q4_K
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = [(1, 1, 256), (9, 100, 768), (64, 128, 1024), (17, 40, 65536), (300, 1000, 2304), (130, 96, 4096),
         (256, 4096, 4096), (256, 12288, 4096), (512, 12288, 4096), (512, 4096, 12288)]


@pytest.mark.parametrize("nt,od,idim", CASES, ids=[f"{a}x{b}x{c}" for a, b, c in CASES])
def test_streamk(nt, od, idim):
    print(f"stream-K nt={nt} od={od} id={idim}", flush=True)
    W = synth.weights(Q4, od, idim, seed=4000 + od)
    x = synth.activations(nt, idim, seed=4100 + nt, outlier_frac=0.01)
    Wt = _up(W)
    q, d, s = qmm.qmm_quantize_act(_up(x))
    ws = torch.full((qmm.qmm_streamk_ws_bytes(),), 0xFF, dtype=torch.uint8, device=DEV)
    a = qmm.qmm_matmul_q8_streamk(Q4, Wt, q, d, s, od, ws)
    b = qmm.qmm_matmul_q8_streamk(Q4, Wt, q, d, s, od, ws)
    torch.cuda.synchronize()
    an = a.cpu().numpy()
    assert np.array_equal(an.view(np.uint32), b.cpu().numpy().view(np.uint32)), "not deterministic"
    assert np.all(np.isfinite(an))
    qn, dn, sn = q.cpu().numpy(), d.cpu().numpy(), s.cpu().numpy()
    if nt * od <= 300 * 1000:
        ref, mag = oracle.matmul_q8(Q4, W, qn, dn, sn, od)
        assert_close(an, ref, mag, Q4, idim, "stream-K vs oracle")
    else:
        rng = np.random.default_rng(od + nt)
        ts = np.unique(np.concatenate([rng.choice(nt, 24, replace=False), [0, nt - 1]]))
        rs = np.unique(np.concatenate([rng.choice(od, 160, replace=False), [0, od - 1]]))
        tt, rr = np.meshgrid(ts, rs, indexing="ij")
        tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
        ref, mag = oracle.matmul_q8_points(Q4, W, qn, dn, sn, od, tt, rr)
        assert_close(an[tt, rr], ref, mag, Q4, idim, "stream-K vs oracle (sampled)")


PATH_CASES = [(20, 96, 8192), (9, 40, 65536), (300, 1000, 2304), (384, 4096, 12288), (512, 4096, 12288),
              (384, 12288, 4096), (512, 12288, 4096), (128, 12288, 4096)]


@pytest.mark.parametrize("nt,od,idim", PATH_CASES, ids=[f"{a}x{b}x{c}" for a, b, c in PATH_CASES])
def test_qmm_matmul_takes_streamk_where_preferred(nt, od, idim):
    """qmm_matmul with a workspace of qmm_matmul_ws_bytes runs the stream-K kernel
    exactly where qmm_streamk_preferred says so (same bits as the stream-K entry
    point on the same quantized input), the per-tile kernel elsewhere and with a
    workspace of only the q8 plane (same bits as qmm_matmul_q8); outputs within the
    tolerance of the oracle."""
    pref = qmm.qmm_streamk_preferred(Q4, nt, od, idim)
    print(f"qmm_matmul path nt={nt} od={od} id={idim} stream-K preferred={pref}", flush=True)
    mmq = qmm.qmm_dispatch_kind(Q4, nt, od, idim) == qmm.QMM_KIND_MMQ
    tiles = -(-nt // 64) * -(-od // 128)
    assert pref == (mmq and tiles % 256 != 0 and (idim // 256 >= 32 or tiles > 256))
    W = synth.weights(Q4, od, idim, seed=4200 + od)
    x = synth.activations(nt, idim, seed=4300 + nt, outlier_frac=0.01)
    Wt, xt = _up(W), _up(x)
    full = qmm.qmm_matmul(Q4, Wt, xt, od)   # workspace of qmm_matmul_ws_bytes
    small = qmm.qmm_matmul(Q4, Wt, xt, od,
                           workspace=torch.empty(qmm.qmm_act_bytes(nt, idim), dtype=torch.uint8, device=DEV))
    q, d, s = qmm.qmm_quantize_act(xt)
    ws = torch.empty(qmm.qmm_streamk_ws_bytes(), dtype=torch.uint8, device=DEV)
    sk = qmm.qmm_matmul_q8_streamk(Q4, Wt, q, d, s, od, ws)
    pt = qmm.qmm_matmul_q8(Q4, Wt, q, d, s, od)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int32)
    assert torch.equal(bits(full), bits(sk if pref else pt))
    assert torch.equal(bits(small), bits(pt))
    qn, dn, sn = q.cpu().numpy(), d.cpu().numpy(), s.cpu().numpy()
    if nt * od <= 300 * 1000:
        ref, mag = oracle.matmul_q8(Q4, W, qn, dn, sn, od)
        assert_close(full.cpu().numpy(), ref, mag, Q4, idim, "qmm_matmul vs oracle")
    else:
        rng = np.random.default_rng(od + nt + 1)
        ts = np.unique(np.concatenate([rng.choice(nt, 16, replace=False), [0, nt - 1]]))
        rs = np.unique(np.concatenate([rng.choice(od, 128, replace=False), [0, od - 1]]))
        tt, rr = np.meshgrid(ts, rs, indexing="ij")
        tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
        ref, mag = oracle.matmul_q8_points(Q4, W, qn, dn, sn, od, tt, rr)
        assert_close(full.cpu().numpy()[tt, rr], ref, mag, Q4, idim, "qmm_matmul vs oracle (sampled)")
