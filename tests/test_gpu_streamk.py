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
