"""GPU parity of the small-batch Q4_K kernel (QMM_KIND_SKINNY: 16 x 16 x 32 int8
MFMA tiles, 1..16 tokens per launch) against the CPU oracle through the C ABI.

Outputs within the f32 tolerance of tests/_parity.py, elementwise: every output on
shapes with ragged row tiles (od not a multiple of 16 or 32), odd super-block
counts (1, 3, 9, 18: the waves splitting K then get unequal shares or none) and
every token count 1..16 (padding lanes of the 16-token tile); matrices of more than
256 row tiles with K split over 1 to 8 waves (straight-line and loop forms, 4, 8
and 16 token slots, a last row tile of 8 rows); sampled outputs at the decode layer
shapes; more than 16 tokens as token slices of 16; and the refusal of other weight
types.
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
K7 = qmm.QMM_KIND_SKINNY


def _up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _say(*a):
    print(*a, flush=True)


CASES = [(nt, od, idim) for nt in (1, 2, 3, 4, 5, 7, 8, 9, 12, 13, 16)
         for od, idim in ((1, 256), (7, 768), (33, 4608), (100, 2304), (257, 1024))]
# larger matrices (with the waves splitting K that the launch rule gives): 5480 x 256
# (1, the last row tile holds 8 rows), 5480 x 512 (2), 6000 x 1024 (4), 9000 x 768
# (2, 3 super-blocks: the loop form, unequal shares), 8200 x 2304 (8, 9
# super-blocks: the loop form), 7000 x 12288 (8, 6 super-blocks per wave: the loop
# form)
CASES += [(1, 5480, 256), (4, 5480, 512), (8, 6000, 1024), (16, 9000, 768), (5, 8200, 2304),
          (3, 7000, 12288), (12, 5480, 512), (7, 9000, 768)]
# more than 16 tokens: launches on token slices of 16 (ragged last slice)
CASES += [(17, 33, 4608), (24, 257, 1024), (33, 100, 2304), (48, 7, 768), (40, 5480, 512)]


@pytest.mark.parametrize("nt,od,idim", CASES)
def test_skinny_parity(nt, od, idim):
    _say(f"skinny nt={nt} od={od} id={idim}")
    W = synth.weights(Q4, od, idim, seed=5000 + nt)
    x = synth.activations(nt, idim, seed=6000 + od, outlier_frac=0.01)
    rq, rd, rs = oracle.quantize(x)
    ref, mag = oracle.matmul_q8(Q4, W, rq, rd, rs, od)
    out = qmm.qmm_matmul_q8_kind(K7, Q4, _up(W), _up(rq), _up(rd), _up(rs), od)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, mag, Q4, idim, f"skinny nt={nt} od={od} id={idim}")


def _sample(n, k, rng):
    idx = rng.choice(n, size=min(n, k), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]]))


@pytest.mark.parametrize("od,idim,nt", [(12288, 4096, 8), (12288, 4096, 1), (4096, 4096, 16), (4096, 12288, 4),
                                        (1024, 4096, 3)])
def test_skinny_full_size_sampled(od, idim, nt):
    _say(f"skinny full size {od}x{idim} nt={nt}")
    W = synth.weights(Q4, od, idim, seed=7000 + nt)
    x = synth.activations(nt, idim, seed=7100 + od, outlier_frac=0.01)
    rq, rd, rs = oracle.quantize(x)
    out = qmm.qmm_matmul_q8_kind(K7, Q4, _up(W), _up(rq), _up(rd), _up(rs), od).cpu().numpy()
    rng = np.random.default_rng(nt)
    ts, rs_ = _sample(nt, 16, rng), _sample(od, 160, rng)
    tt, rr = np.meshgrid(ts, rs_, indexing="ij")
    tt, rr = tt.reshape(-1).astype(np.int32), rr.reshape(-1).astype(np.int32)
    ref, mag = oracle.matmul_q8_points(Q4, W, rq, rd, rs, od, tt, rr)
    assert_close(out[tt, rr], ref, mag, Q4, idim, f"skinny {od}x{idim} nt={nt}")


def test_skinny_deterministic():
    """The waves splitting K add their partial sums in a fixed order."""
    W = _up(synth.weights(Q4, 4096, 4096, seed=1))
    q, d, s = qmm.qmm_quantize_act(_up(synth.activations(8, 4096, seed=2)))
    o1 = qmm.qmm_matmul_q8_kind(K7, Q4, W, q, d, s, 4096)
    o2 = qmm.qmm_matmul_q8_kind(K7, Q4, W, q, d, s, 4096)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


@pytest.mark.parametrize("od,idim,nt", [(12288, 4096, 4), (12288, 4096, 8), (12288, 4096, 16), (1000, 2304, 5),
                                        (500, 768, 3), (4096, 12288, 8), (257, 1024, 12), (4096, 8192, 4)])
def test_skinny_split_independent(od, idim, nt):
    """The K split (1, 2, 4, 8 or 16 waves per workgroup, forced through
    qmm_set_skinny_split; capped by the super-blocks of a row) does not change the
    bits: 16 super-blocks (straight-line at 16, 8 and 4 waves, the loop at 2 and 1),
    9 and 3 super-blocks (loop forms, unequal shares), 48 and 32 super-blocks (16
    waves by default; loops with 2 to 16 accumulators per wave), 4 super-blocks; and
    every token row equals that token alone."""
    _say(f"skinny split independence {od}x{idim} nt={nt}")
    W = _up(synth.weights(Q4, od, idim, seed=41 + nt))
    q, d, s = qmm.qmm_quantize_act(_up(synth.activations(nt, idim, seed=42 + od)))
    outs = {}
    try:
        for ks in (8, 16, 4, 2, 1):
            qmm.qmm_set_skinny_split(ks)
            outs[ks] = qmm.qmm_matmul_q8_kind(K7, Q4, W, q, d, s, od)
            torch.cuda.synchronize()
        qmm.qmm_set_skinny_split(0)
        ones = [qmm.qmm_matmul_q8_kind(K7, Q4, W, q[t:t + 1].contiguous(), d[t:t + 1].contiguous(),
                                       s[t:t + 1].contiguous(), od) for t in range(nt)]
        torch.cuda.synchronize()
    finally:
        qmm.qmm_set_skinny_split(0)
    ref = outs[8].view(torch.int32)
    for ks in (16, 4, 2, 1):
        assert torch.equal(outs[ks].view(torch.int32), ref), f"{od}x{idim} nt={nt}: split {ks} against 8"
    assert torch.equal(torch.cat(ones).view(torch.int32), ref), f"{od}x{idim} nt={nt}: single tokens"


@pytest.mark.parametrize("od,idim,nt", [(4096, 4096, 40), (12288, 4096, 32), (4096, 12288, 24)])
def test_skinny_slices_match_single_tokens(od, idim, nt):
    """qmm_matmul_q8 on 17..48 tokens takes the small-batch kernel on token slices of
    16 (the dispatcher's choice here); every token row equals that token alone."""
    _say(f"skinny slices {od}x{idim} nt={nt}")
    assert qmm.qmm_dispatch_kind(Q4, nt, od, idim) == K7
    W = _up(synth.weights(Q4, od, idim, seed=51))
    q, d, s = qmm.qmm_quantize_act(_up(synth.activations(nt, idim, seed=52)))
    whole = qmm.qmm_matmul_q8(Q4, W, q, d, s, od)
    ones = [qmm.qmm_matmul_q8_kind(K7, Q4, W, q[t:t + 1].contiguous(), d[t:t + 1].contiguous(),
                                   s[t:t + 1].contiguous(), od) for t in range(nt)]
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int32), torch.cat(ones).view(torch.int32))


def test_skinny_refusals():
    W6 = _up(synth.weights(Q6, 16, 256, seed=5))
    q, d, s = qmm.qmm_quantize_act(_up(synth.activations(17, 256, seed=4)))
    with pytest.raises(qmm.QmmError):
        qmm.qmm_matmul_q8_kind(K7, Q6, W6, q[:4], d[:32], s[:32], 16)
