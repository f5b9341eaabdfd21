"""HIP graph replays of the hot path give the eager results, bit for bit.

The library's calls only enqueue kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a caller can capture a whole step -- quantize, the
producer-fused quantize, the vector kernel, its 8-token slices and the matrix
kernel with and without the split over K -- into one HIP graph and replay it.
The stream-K kernel and its fixup (three launches sharing one workspace) are in
the step too, and the Q8_K path (a fused RMS-norm Q8_K quantize, a Q4_K matmul
split over K, a padded Q6_K matmul).  Checked here: the graph is replayed several
times, with other GPU work and host synchronisation between replays and the
outputs cleared before each, and every output of every replay equals the eagerly
computed one (the kernels are deterministic: no atomics, fixed reduction orders).
"""
from __future__ import annotations

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

qmm = pytest.importorskip("quantized_matmul_amd")
DEV = "cuda:0"


def _up(a):
    return torch.from_numpy(a).to(DEV)


class Step:
    """Fixed buffers and the calls of one small step, issued on the current stream."""

    # (type, od, id, nt): vector kernel, 8-token slices, matrix kernel split over K
    # (4096 x 4096 at 64 tokens) and per tile (12288 x 4096 at 128 tokens)
    SHAPES = [(qmm.QMM_TYPE_Q4_K, 4096, 4096, 4), (qmm.QMM_TYPE_Q6_K, 4096, 4096, 12),
              (qmm.QMM_TYPE_Q4_K, 4096, 4096, 64), (qmm.QMM_TYPE_Q4_K, 12288, 4096, 128)]

    def __init__(self):
        self.items = []
        for i, (qt, od, idim, nt) in enumerate(self.SHAPES):
            W = _up(synth.weights(qt, od, idim, seed=60 + i))
            x = _up(synth.activations(nt, idim, seed=70 + i, outlier_frac=0.01))
            q = torch.empty(nt, idim, dtype=torch.int8, device=DEV)
            d = torch.empty(nt, idim // 32, dtype=torch.float32, device=DEV)
            s = torch.empty_like(d)
            out = torch.empty(nt, od, dtype=torch.float32, device=DEV)
            self.items.append((qt, od, W, x, q, d, s, out))
        # producer-fused quantize feeding a matmul
        self.h = _up(synth.activations(16, 4096, seed=80))
        self.w = _up(1.0 + 0.25 * synth.activations(1, 4096, seed=81)[0])
        self.fq = torch.empty(16, 4096, dtype=torch.int8, device=DEV)
        self.fd = torch.empty(16, 128, dtype=torch.float32, device=DEV)
        self.fs = torch.empty_like(self.fd)
        self.fW = _up(synth.weights(qmm.QMM_TYPE_Q4_K, 4096, 4096, seed=82))
        self.fout = torch.empty(16, 4096, dtype=torch.float32, device=DEV)
        # stream-K launches (tiles split over up to 8 workgroups; a padded Q6_K one)
        # sharing one workspace, on the first and the third item's quantized input
        self.ws = torch.full((qmm.qmm_streamk_ws_bytes(),), 0xFF, dtype=torch.uint8, device=DEV)
        self.skW6 = qmm.qmm_pad_q6k(_up(synth.weights(qmm.QMM_TYPE_Q6_K, 1000, 4096, seed=83)))
        self.skout = [torch.empty(4, 4096, dtype=torch.float32, device=DEV),
                      torch.empty(64, 4096, dtype=torch.float32, device=DEV),
                      torch.empty(64, 1000, dtype=torch.float32, device=DEV)]
        # the Q8_K path: a fused RMS-norm Q8_K quantize feeding a Q4_K matmul split
        # over K (4096 x 4096 at 16 tokens) and a padded Q6_K matmul
        self.kq = torch.empty(16, 4096, dtype=torch.int8, device=DEV)
        self.kd = torch.empty(16, 16, dtype=torch.float32, device=DEV)
        self.kb = torch.empty(16, 256, dtype=torch.float32, device=DEV)
        self.kout = [torch.empty(16, 4096, dtype=torch.float32, device=DEV),
                     torch.empty(16, 1000, dtype=torch.float32, device=DEV)]

    def issue(self):
        for qt, od, W, x, q, d, s, out in self.items:
            qmm.qmm_quantize_act(x, q, d, s)
            qmm.qmm_matmul_q8(qt, W, q, d, s, od, out=out)
        qmm.qmm_rmsnorm_quantize(self.h, self.w, 1e-5, self.fq, self.fd, self.fs)
        qmm.qmm_matmul_q8(qmm.QMM_TYPE_Q4_K, self.fW, self.fq, self.fd, self.fs, 4096, out=self.fout)
        for (qt, W, q, d, s), out in zip((self.items[0][:1] + self.items[0][2:3] + self.items[0][4:7],
                                          self.items[2][:1] + self.items[2][2:3] + self.items[2][4:7],
                                          (qmm.QMM_TYPE_Q6_K_P224, self.skW6) + self.items[2][4:7]),
                                         self.skout):
            qmm.qmm_matmul_q8_streamk(qt, W, q, d, s, out.shape[1], self.ws, out=out)
        qmm.qmm_rmsnorm_quantize_q8k(self.h, self.w, 1e-5, self.kq, self.kd, self.kb)
        qmm.qmm_matmul_q8k(qmm.QMM_TYPE_Q4_K, self.fW, self.kq, self.kd, self.kb, 4096, out=self.kout[0])
        qmm.qmm_matmul_q8k(qmm.QMM_TYPE_Q6_K_P224, self.skW6, self.kq, self.kd, self.kb, 1000, out=self.kout[1])

    def outputs(self):
        res = []
        for item in self.items:
            res += [t.clone() for t in item[4:]]
        return res + [self.fq.clone(), self.fd.clone(), self.fs.clone(), self.fout.clone()] + \
            [t.clone() for t in self.skout] + [t.clone() for t in (self.kq, self.kd, self.kb, *self.kout)]

    def clear(self):
        # eager fill kernels (not recorded in the graph)
        for item in self.items:
            for t in item[4:]:
                t.zero_()
        for t in (self.fq, self.fd, self.fs, self.fout, *self.skout, self.kq, self.kd, self.kb, *self.kout):
            t.zero_()


def test_graph_replays_match_eager():
    print("graph replay: capture a step of 5 quantize, 5 matmul, 3 stream-K and 3 Q8_K calls", flush=True)
    assert qmm.qmm_q8k_tile(16, 4096, 4096) == qmm.QMM_KIND_MMQ_64X64_SPLITK
    assert qmm.qmm_dispatch_kind(qmm.QMM_TYPE_Q6_K, 12, 4096, 4096) == qmm.QMM_KIND_MMVQ
    assert qmm.qmm_dispatch_kind(qmm.QMM_TYPE_Q4_K, 64, 4096, 4096) == qmm.QMM_KIND_MMQ
    step = Step()
    step.issue()
    torch.cuda.synchronize()
    eager = step.outputs()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.issue()  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        step.issue()
    torch.cuda.synchronize()

    other = Step.SHAPES[0]
    W2 = _up(synth.weights(other[0], other[1], other[2], seed=90))
    x2 = _up(synth.activations(other[3], other[2], seed=91))
    for rep in range(3):
        step.clear()
        # unrelated eager work between replays
        q2, d2, s2 = qmm.qmm_quantize_act(x2)
        qmm.qmm_matmul_q8(other[0], W2, q2, d2, s2, other[1])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for k, (a, b) in enumerate(zip(got, eager)):
            assert a.dtype == b.dtype and a.shape == b.shape
            same = torch.equal(a.view(torch.uint8), b.view(torch.uint8))
            assert same, f"replay {rep}: output {k} differs from the eager result"
    print("  3 replays equal the eager outputs", flush=True)
