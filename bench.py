"""Benchmark of the quantized-weight matmul on one MI355X.

Default workload ("q4k_decode_prefill"): one step is the whole hot path --
activation quantize, nt dispatch, and the selected kernel -- over
  * Q4_K decode: W 1024x4096 at nt = 1, and W 4096x4096 and 12288x4096 at nt = 1, 4
    and 8 (the vector kernel at nt = 1, the small-batch MFMA kernel at 4 and 8),
  * the Q6_K output projection W 32000x4096 at nt = 1, as stored (210-byte blocks)
    and padded to 224 bytes,
  * Q4_K prefill: W 12288x4096 and 4096x12288 at nt = 512, activations N(0,1) with
    1 % of elements x20, on per-32 activations (the path) and, on the same weights
    and inputs, on Q8_K activations (one scale per 256 values; its own numerics).
Inputs are seeded synthetic data (see synth/), resident in HBM before timing.
Weight copies rotate so every weight read of the timed region comes from HBM
(more than 1 GB of copies per shape, above the 256 MB last-level cache); calls on
the same matrix start at evenly spaced points of its rotation, so no call reads
copies another call has just read.

Reported (one JSON line): value = HBM GB/s of the vector kernel at nt = 1
(algorithmic bytes: weights + q8 activations + f32 output, over the kernel's
average launch time, the 4096x4096 and 12288x4096 calls together), its roofline on
the 12288x4096 call against 8 TB/s and against the streaming read of the same bytes
measured in the same process (bench_peaks: frac_of_measured); small_batch (nt = 4
and 8), q6k_head, mmq (int8 TOP/s at nt = 512 against 5.0 POP/s and the measured
int8 MFMA rate), mmq_q8k, the diffusion-LM step as one HIP graph (dllm_step; skip
with --no-dllm), and the CPU oracle timed on a bounded sample (cpu_baseline).

Kernel times come from HIP events on the launch stream inside the timed region.
The K steps are issued call by call: for each call, a chunk of 20 quantize
launches and then 20 matmul launches (rotating weight copies) run back to back
between events, and the per-launch time is the chunk time over 20 (a HIP event
itself costs about 4 us of GPU time).  A bounded busy-wait kernel
(torch.cuda._sleep) at the head of each chunk group lets the host queue ahead of
the GPU.  ms_per_step is wall time per step (gate included); gpu_ms_per_step sums
the per-launch quantize and matmul times of one step.

roofline.traffic is the HBM bytes per launch of the roofline kernel as measured by
the rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised in profiles/ (scaled by a
plain copy of known size), or null when that summary is missing or was taken from
kernel sources other than the ones built here.

Workload "fused_quantize": the producer-side steps fused with the quantizer
(residual add + RMS norm, RMS norm, silu(g) * u), each against its unfused chain
(the f32 step, then the plain quantizer), at a decode row (nt = 1) and a prefill
block (nt = 512) of an 8B model (hidden 4096; FFN 12288 for silu).  One step runs
every fused call once and every chain once; inputs rotate over copies of more than
1 GiB per shape.  value = HBM GB/s of the fused kernels at nt = 512 (algorithmic
bytes over their summed launch times); roofline on silu_mul_quantize 512 x 12288.

Workload "q8k_prefill": the two prefill shapes above on Q8_K activations (one scale
per 256 values, 16-value code sums; its own numerics) and, on the same weights and
inputs, on the per-32 activations.  value = int8 TOP/s of the Q4_K Q8_K matmul
kernel; per32_same_shapes gives the per-32 kernel's rate from the same process;
q6k_padded_4096x12288 the same comparison for the down projection's shape in the
padded Q6_K layout.

Workload "dllm_step": the 224 matmuls of one diffusion-LM step at L = 256 (32 layers x
q, k, v, o, gate, up Q4_K and down Q6_K in the padded layout; distinct weights per
layer).  value = int8 ops over the summed kernel times; graph = the whole step
(quantize + matmul per call) captured into one HIP graph and replayed;
graph_layers = the same matmuls fed as a model's layers feed them (fused RMS-norm,
residual-add and silu * up producers; one quantized input shared by q, k, v and one
by gate, up: 4 producer launches per layer), also one graph; graph_q8k = "graph"
on Q8_K activations (quantize_q8k + the Q8_K matrix kernels; other numerics);
graph_layers_q8k = graph_layers with the producers' Q8_K variants and the Q8_K
matrix kernels.

Workload "formats": Q4_0, Q8_0 and Q5_K (and Q4_K for comparison) at 12288 x 4096, nt = 1
and nt = 512.  value = HBM GB/s of the Q4_0 vector kernel at nt = 1.

Workload "streamk": the Q4_K matrix shapes of the diffusion-LM step (4096x4096 and
12288x4096 at nt = 256) and of prefill (nt = 512), on the per-tile dispatch and on
the stream-K kernel (two launches: the kernel and its fixup), same inputs.

Workload "peaks": the measured limits of this GPU (bench_peaks.hip): a plain
streaming read at the decode weight sizes, int8 and f32 MFMA issue rates, VALU issue
rates, LDS read rate, MFMA/VALU overlap and the per-32 step on its own.

Options: --gpus N (1 only), --steps K, --warmup W, --workload
{q4k_decode_prefill, q6k_head, dllm_step, fused_quantize, q8k_prefill, formats, streamk, peaks},
--no-cpu-baseline, --no-dllm, --chunk, --spread-chunks, --copy-calibration
MIB (before warm-up, run five plain device copies of MIB MiB between two spin-kernel
markers, for scaling the HBM counters of a profiled run).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
COPY_BYTES = 1 << 30           # weight copies per shape: at least 1 GiB
CHUNK = 20                     # launches per event-timed chunk
COUNTERS = os.path.join(ROOT, "profiles", "q4k_decode_prefill_hbm_counters.md")
FUSED_COUNTERS = os.path.join(ROOT, "profiles", "fused_quantize_hbm_counters.md")
Q8K_COUNTERS = os.path.join(ROOT, "profiles", "q8k_prefill_hbm_counters.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="multiple of 20")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="q4k_decode_prefill",
                    choices=["q4k_decode_prefill", "q6k_head", "dllm_step", "fused_quantize", "q8k_prefill",
                             "formats", "streamk", "peaks"])
    ap.add_argument("--chunk", type=int, default=CHUNK, help="launches per event-timed chunk")
    ap.add_argument("--spread-chunks", type=int, default=8,
                    help="event-timed chunks per call after the timed region, for the median and p10/p90")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dllm", action="store_true", help="default workload: skip the diffusion-LM step graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB")
    return ap.parse_args()


def copy_calibration(torch, mib):
    """Five plain device-to-device copies of `mib` MiB between two spin-kernel markers."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.cuda._sleep(1)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda._sleep(1)
    torch.cuda.synchronize()
    del src, dst
    return {"bytes": n, "reps": 5}


MMQ_TILES = {3: (4, 2, 1), 4: (2, 2, 1), 5: (2, 2, 2)}   # tile kind -> (row waves, token waves, K groups)


def mmq_kernel(qmm, nt, od, idim):
    """(kernel name, launch threads) of the Q4_K matrix kernel qmm_matmul runs for this
    shape with a full workspace: stream-K (256 workgroups of 8 waves) where
    qmm_streamk_preferred, else the per-tile kernel: 32*WR rows x 32*WC tokens per
    workgroup, KS groups splitting K, the workgroup count padded to a multiple of the
    8 XCDs."""
    if qmm.qmm_streamk_preferred(qmm.QMM_TYPE_Q4_K, nt, od, idim):
        return "qmm::mmq_q4k_streamk_kernel<4, 2>", 256 * 512
    tile = qmm.qmm_mmq_tile(nt, od, idim)
    tiles = -(-nt // 64) * -(-od // 128)
    # the 4-wave kernel of 32 x 64 per wave (the library's mmq_q4k_wave_form), and its
    # split over K in 8 waves
    if tiles > 256 and (tile == qmm.QMM_KIND_MMQ_128X64 or 384 <= tiles <= 512):
        return "qmm::{anonymous}::mmq_q4k_v2_kernel<1, false>", 8 * -(-tiles // 8) * 256
    if tile == qmm.QMM_KIND_MMQ_128X64 and tiles >= 192:
        return "qmm::{anonymous}::mmq_q4k_v2_kernel<2, false>", 8 * -(-tiles // 8) * 512
    wr, wc, ks = MMQ_TILES[tile]
    tiles = -(-nt // (32 * wc)) * -(-od // (32 * wr))
    return f"qmm::mmq_q4k_kernel<{wr}, {wc}, {ks}, false>", 8 * -(-tiles // 8) * 64 * wr * wc * ks


class Call:
    """One matmul of the step: weights (rotating copies), activations, buffers."""

    def __init__(self, torch, qmm, qtype, od, idim, nt, seed, outliers, copies=None, label="", x=None, q8k=False,
                 streamk=None):
        self.qtype, self.od, self.idim, self.nt, self.q8k = qtype, od, idim, nt, q8k
        self.label = label or f"{'Q4_K' if qtype == 1 else 'Q6_K'} {od}x{idim} nt={nt}" + (" Q8_K" if q8k else "")
        dev = torch.device("cuda:0")
        self.w_host = None   # host bytes of the weights when generated here (for the CPU baseline)
        if copies is None:
            self.w_host = synth.weights(qtype, od, idim, seed=seed)
            w = torch.from_numpy(self.w_host).to(dev)
            n = max(1, -(-COPY_BYTES // w.numel()))
            copies = [w] + [w.clone() for _ in range(n - 1)]
        self.W = copies
        if x is None:
            x = torch.from_numpy(synth.activations(nt, idim, seed=seed + 1,
                                                   outlier_frac=0.01 if outliers else 0.0)).to(dev)
        self.x = x
        self.q = torch.empty((nt, idim), dtype=torch.int8, device=dev)
        self.d = torch.empty((nt, idim // 32), dtype=torch.float32, device=dev)
        self.s = torch.empty((nt, idim // 32), dtype=torch.float32, device=dev)
        self.out = torch.empty((nt, od), dtype=torch.float32, device=dev)
        self.kind = qmm.QMM_KIND_MMQ if q8k else qmm.qmm_dispatch_kind(qtype, nt, od, idim)
        self.wbytes = qmm.qmm_weight_bytes(qtype, od, idim)
        # algorithmic bytes of the matmul kernel: weights + quantized activations + output
        act = nt * idim * ((1 + 4 / 256 + 4 / 16) if q8k else (1 + 8 / 32))
        self.kbytes = self.wbytes + act + nt * od * 4
        self.ops = 2.0 * nt * od * idim
        self.k_ms = []   # matmul kernel time per launch, one entry per timed chunk
        self.q_ms = []   # quantize kernel time per launch, one entry per timed chunk
        self.i0 = 0      # first copy of the rotation (calls sharing copies start apart)
        self.i = 0
        # raw C-ABI arguments, built once so the timed loop only makes the calls
        P, I = ctypes.c_void_p, ctypes.c_int
        st = P(torch.cuda.current_stream().cuda_stream)
        self.L = qmm.lib()
        if q8k:  # Q8_K activations: d per 256 values, group sums per 16 (in self.s)
            self.d = torch.empty((nt, idim // 256), dtype=torch.float32, device=dev)
            self.s = torch.empty((nt, idim // 16), dtype=torch.float32, device=dev)
        self.qfn = self.L.qmm_quantize_act_q8k if q8k else self.L.qmm_quantize_act
        self.mfn = self.L.qmm_matmul_q8k if q8k else self.L.qmm_matmul_q8
        self.qargs = (P(self.x.data_ptr()), I(nt), I(idim), P(self.q.data_ptr()), P(self.d.data_ptr()),
                      P(self.s.data_ptr()), st)
        self.margs = [(I(qtype), P(w.data_ptr()), P(self.q.data_ptr()), P(self.d.data_ptr()),
                       P(self.s.data_ptr()), I(nt), I(od), I(idim), P(self.out.data_ptr()), st) for w in self.W]
        if streamk is not None:  # the stream-K kernel, with its workspace
            self.mfn = self.L.qmm_matmul_q8_streamk
            self.margs = [a[:9] + (P(streamk.data_ptr()), ctypes.c_size_t(streamk.numel()), st) for a in self.margs]
            self.label += " stream-K"

    def quantize(self):
        rc = self.qfn(*self.qargs)
        if rc:
            raise RuntimeError(f"quantize failed: {rc}")

    def matmul(self):
        rc = self.mfn(*self.margs[self.i % len(self.margs)])
        self.i += 1
        if rc:
            raise RuntimeError(f"matmul failed: {rc}")

    def run(self):
        self.quantize()
        self.matmul()


def graph_replay_ms(torch, calls, replays=5):
    """One step (every call's quantize and matmul, its first weight copy) captured
    into a HIP graph on a side stream; mean replay time in ms (HIP events on that
    stream), replays back to back after one untimed replay."""
    P = ctypes.c_void_p
    side = torch.cuda.Stream()
    sp = P(side.cuda_stream)
    qa = [c.qargs[:-1] + (sp,) for c in calls]
    ma = [c.margs[0][:-1] + (sp,) for c in calls]

    def issue():
        for c, a, b in zip(calls, qa, ma):
            if c.qfn(*a) or c.mfn(*b):
                raise RuntimeError(f"{c.label}: launch failed while capturing")

    side.wait_stream(torch.cuda.current_stream())
    issue()  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        issue()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(replays):
            g.replay()
        e1.record(side)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / replays


def layer_graph_ms(torch, qmm, calls, replays=5, q8k=False):
    """The step's 224 matmuls with the data flow of a model's layers, captured as one
    HIP graph like graph_replay_ms.  Per layer: q, k and v read one fused RMS-norm
    quantize of the residual stream; o reads the quantized v output (standing in
    for the attention output); gate and up read one fused residual-add + RMS-norm
    quantize; down reads the fused silu(gate) * up quantize of their outputs; the
    next layer's first producer adds the down output into the residual stream.  So
    4 producer launches and 7 matmuls per layer (the plain step: 7 quantize
    launches, one per matmul), the same matmul kernels and weights.  q8k: the
    producers' Q8_K variants and calls on the Q8_K matrix path."""
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L = qmm.lib()
    dev = torch.device("cuda:0")
    nt, hid, ffn = calls[0].nt, 4096, 12288
    h = torch.from_numpy(synth.activations(nt, hid, seed=300)).to(dev)
    w_attn = torch.from_numpy(1.0 + 0.25 * synth.activations(1, hid, seed=301)[0]).to(dev)
    w_ffn = torch.from_numpy(1.0 + 0.25 * synth.activations(1, hid, seed=302)[0]).to(dev)

    def q8(n):
        if q8k:  # codes, d per 256 values, 16-value group sums
            return (torch.empty((nt, n), dtype=torch.int8, device=dev), torch.empty((nt, n // 256), device=dev),
                    torch.empty((nt, n // 16), device=dev))
        return (torch.empty((nt, n), dtype=torch.int8, device=dev), torch.empty((nt, n // 32), device=dev),
                torch.empty((nt, n // 32), device=dev))

    sfx = "_q8k" if q8k else ""
    rms_q, add_rms_q, silu_q = (getattr(L, f"qmm_rmsnorm_quantize{sfx}"), getattr(L, f"qmm_add_rmsnorm_quantize{sfx}"),
                                getattr(L, f"qmm_silu_mul_quantize{sfx}"))
    quant = L.qmm_quantize_act_q8k if q8k else L.qmm_quantize_act

    qa, qo, qf, qd = q8(hid), q8(hid), q8(hid), q8(ffn)
    ptr = lambda t: P(t.data_ptr())  # noqa: E731
    side = torch.cuda.Stream()
    sp = P(side.cuda_stream)
    eps = F(1e-5)

    def mm(c, src):
        a = c.margs[0]
        return c.mfn(*(a[:2] + (ptr(src[0]), ptr(src[1]), ptr(src[2])) + a[5:-1] + (sp,)))

    def issue():
        rc = []
        for layer in range(len(calls) // 7):
            cq, ck, cv, co, cg, cu, cd = calls[7 * layer:7 * layer + 7]
            if layer == 0:
                rc.append(rms_q(ptr(h), ptr(w_attn), eps, I(nt), I(hid), *map(ptr, qa), sp))
            else:
                prev = calls[7 * layer - 1].out
                rc.append(add_rms_q(ptr(h), ptr(prev), ptr(w_attn), eps, I(nt), I(hid), *map(ptr, qa), sp))
            rc += [mm(cq, qa), mm(ck, qa), mm(cv, qa)]
            rc.append(quant(ptr(cv.out), I(nt), I(hid), *map(ptr, qo), sp))
            rc.append(mm(co, qo))
            rc.append(add_rms_q(ptr(h), ptr(co.out), ptr(w_ffn), eps, I(nt), I(hid), *map(ptr, qf), sp))
            rc += [mm(cg, qf), mm(cu, qf)]
            rc.append(silu_q(ptr(cg.out), ptr(cu.out), I(nt), I(ffn), *map(ptr, qd), sp))
            rc.append(mm(cd, qd))
        if any(rc):
            raise RuntimeError(f"layer data flow: a launch failed ({[r for r in rc if r]})")

    side.wait_stream(torch.cuda.current_stream())
    issue()  # warm-up on the capture stream
    torch.cuda.synchronize()
    if not bool(torch.isfinite(h).all()):
        raise RuntimeError("layer data flow: the residual stream is not finite")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        issue()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(side)
        for _ in range(replays):
            g.replay()
        e1.record(side)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / replays


def build_calls(torch, qmm, workload):
    Q4, Q6 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K
    calls = []
    sk_ws = []

    def path_ws(qt, nt, od, idim):
        """The stream-K workspace where qmm_matmul (with a full workspace) runs the
        stream-K kernel, else None: matrix calls run what qmm_matmul runs."""
        if not qmm.qmm_streamk_preferred(qt, nt, od, idim):
            return None
        if not sk_ws:  # one workspace: the calls run one after another on one stream
            sk_ws.append(torch.empty(qmm.qmm_streamk_ws_bytes(), dtype=torch.uint8, device="cuda:0"))
        return sk_ws[0]

    if workload == "q4k_decode_prefill":
        # the decode GEMV of one 1024 x 4096 matrix
        calls.append(Call(torch, qmm, Q4, 1024, 4096, 1, seed=0, outliers=False))
        shared = {}
        for od, idim in ((4096, 4096), (12288, 4096)):
            for nt in (1, 4, 8):
                c = Call(torch, qmm, Q4, od, idim, nt, seed=10 * nt + od, outliers=False,
                         copies=shared.get((od, idim)))
                if (od, idim) not in shared:
                    shared[(od, idim)] = c.W
                    shared[("host", od, idim)] = c.w_host
                c.w_host = shared[("host", od, idim)]
                calls.append(c)
        # the Q6_K output projection, as stored (210-byte blocks) and padded to 224 bytes
        c6 = Call(torch, qmm, Q6, 32000, 4096, 1, seed=3, outliers=False)
        calls.append(c6)
        calls.append(Call(torch, qmm, qmm.QMM_TYPE_Q6_K_P224, 32000, 4096, 1, seed=3, outliers=False,
                          copies=[qmm.qmm_pad_q6k(w) for w in c6.W], x=c6.x, label="Q6_K padded 32000x4096 nt=1"))
        # prefill: per-32 activations (the path), then the same weights and inputs on Q8_K activations
        pa = Call(torch, qmm, Q4, 12288, 4096, 512, seed=7, outliers=True, copies=shared[(12288, 4096)],
                  streamk=path_ws(Q4, 512, 12288, 4096))
        pa.w_host = shared[("host", 12288, 4096)]
        pb = Call(torch, qmm, Q4, 4096, 12288, 512, seed=8, outliers=True, streamk=path_ws(Q4, 512, 4096, 12288))
        calls += [pa, pb]
        for c in (pa, pb):
            calls.append(Call(torch, qmm, Q4, c.od, c.idim, 512, seed=0, outliers=True, copies=c.W, x=c.x, q8k=True))
    elif workload == "q8k_prefill":
        # the prefill shapes on both activation schemes, same weights and inputs
        for od, idim, seed in ((12288, 4096, 7), (4096, 12288, 8)):
            per32 = Call(torch, qmm, Q4, od, idim, 512, seed=seed, outliers=True)
            calls.append(per32)
            calls.append(Call(torch, qmm, Q4, od, idim, 512, seed=seed, outliers=True, copies=per32.W, x=per32.x,
                              q8k=True))
        # and the down projection's shape in the padded Q6_K layout
        P6 = qmm.QMM_TYPE_Q6_K_P224
        w = qmm.qmm_pad_q6k(torch.from_numpy(synth.weights(Q6, 4096, 12288, seed=9)).to("cuda:0"))
        copies = [w] + [w.clone() for _ in range(max(1, -(-COPY_BYTES // w.numel())) - 1)]
        per32 = Call(torch, qmm, P6, 4096, 12288, 512, seed=9, outliers=True, copies=copies,
                     label="Q6_K padded 4096x12288 nt=512")
        calls.append(per32)
        calls.append(Call(torch, qmm, P6, 4096, 12288, 512, seed=9, outliers=True, copies=copies, x=per32.x,
                          q8k=True, label="Q6_K padded 4096x12288 nt=512 Q8_K"))
    elif workload == "streamk":
        # the Q4_K matrix shapes of the diffusion-LM step (L = 256) and of prefill
        # (nt = 512), per-tile dispatch and stream-K on the same weights and inputs
        ws = torch.empty(qmm.qmm_streamk_ws_bytes(), dtype=torch.uint8, device="cuda:0")
        for od, idim, nt, seed in ((4096, 4096, 256, 50), (12288, 4096, 256, 51), (12288, 4096, 512, 52),
                                   (4096, 12288, 512, 53)):
            base = Call(torch, qmm, Q4, od, idim, nt, seed=seed, outliers=nt == 512)
            calls.append(base)
            calls.append(Call(torch, qmm, Q4, od, idim, nt, seed=seed, outliers=nt == 512, copies=base.W,
                              x=base.x, streamk=ws))
    elif workload == "formats":
        # Q4_0 and Q8_0 at the 12288 x 4096 shape, decode and prefill, beside Q4_K
        for qt in (qmm.QMM_TYPE_Q4_0, qmm.QMM_TYPE_Q8_0, qmm.QMM_TYPE_Q5_K, Q4):
            shared = None
            for nt in (1, 512):
                c = Call(torch, qmm, qt, 12288, 4096, nt, seed=40 + qt, outliers=nt > 8, copies=shared,
                         label=f"{ {1: 'Q4_K', 4: 'Q4_0', 5: 'Q8_0', 6: 'Q5_K'}[qt] } 12288x4096 nt={nt}")
                shared = c.W
                calls.append(c)
    elif workload == "q6k_head":
        c6 = Call(torch, qmm, Q6, 32000, 4096, 1, seed=3, outliers=False)
        calls.append(c6)
        # the same matrix in the padded layout (224-byte blocks), same activations
        padded = [qmm.qmm_pad_q6k(w) for w in c6.W]
        calls.append(Call(torch, qmm, qmm.QMM_TYPE_Q6_K_P224, 32000, 4096, 1, seed=3, outliers=False,
                          copies=padded, x=c6.x, label="Q6_K padded 32000x4096 nt=1"))
    else:  # dllm_step: 32 layers x (q, k, v, o, gate, up Q4_K; down Q6_K) at L = 256
        # the down projections in the padded Q6_K layout, as the upload pads Q6_K
        P6 = qmm.QMM_TYPE_Q6_K_P224
        shapes = [(Q4, 4096, 4096)] * 4 + [(Q4, 12288, 4096)] * 2 + [(P6, 4096, 12288)]
        # distinct weights per layer (4.34 GB per step, 4.46 GB with the padding): one
        # seeded matrix per projection, copied to 32 distinct HBM places; one input
        # per projection
        per_proj = []
        for p, (qt, od, idim) in enumerate(shapes):
            host = synth.weights(Q6 if qt == P6 else qt, od, idim, seed=100 + p)
            w = torch.from_numpy(host).to("cuda:0")
            if qt == P6:
                w = qmm.qmm_pad_q6k(w)
            x = torch.from_numpy(synth.activations(256, idim, seed=200 + p)).to("cuda:0")
            per_proj.append(([w] + [w.clone() for _ in range(31)], x, host if qt == Q4 else None))
        for layer in range(32):
            for p, (qt, od, idim) in enumerate(shapes):
                copies, x, host = per_proj[p]
                c = Call(torch, qmm, qt, od, idim, 256, seed=0, outliers=False, copies=[copies[layer]],
                         label=f"layer{layer} proj{p} {od}x{idim}", x=x, streamk=path_ws(qt, 256, od, idim))
                c.w_host = host if layer == 0 else None   # the CPU baseline times layer 0's Q4_K projections
                calls.append(c)
    # calls that share a matrix's weight copies start at evenly spaced points of the
    # rotation: one call's chunk of launches then never reads copies another call
    # has just read (20 copies of a 4096 x 4096 matrix, 188 MB, would still sit in
    # the 256 MB last-level cache)
    groups = {}
    for c in calls:
        groups.setdefault(id(c.W), []).append(c)
    for g in groups.values():
        for k, c in enumerate(g):
            c.i0 = c.i = k * (len(c.W) // len(g))
    return calls


class FusedCall:
    """One producer-side step at one shape: the fused kernel and its unfused chain,
    each with inputs rotating over copies of more than COPY_BYTES in total."""

    EPS = 1e-5

    def __init__(self, torch, qmm, op, nt, idim, seed):
        self.op, self.nt, self.idim = op, nt, idim
        self.label = f"{op} {nt}x{idim}"
        dev = torch.device("cuda:0")
        n = nt * idim
        a = torch.from_numpy(synth.activations(nt, idim, seed=seed)).to(dev)
        b = torch.from_numpy(synth.activations(nt, idim, seed=seed + 1)).to(dev) * 0.5
        self.w = torch.from_numpy(1.0 + 0.25 * synth.activations(1, idim, seed=seed + 2)[0]).to(dev)
        per_copy = 4 * n * (2 if op != "rmsnorm_quantize" else 1)
        ncopy = min(256, max(2, -(-COPY_BYTES // per_copy)))  # decode rows: 256 small copies
        self.a = [a] + [a.clone() for _ in range(ncopy - 1)]
        self.b = [b] + [b.clone() for _ in range(ncopy - 1)] if op != "rmsnorm_quantize" else [None] * ncopy
        self.y = torch.empty((nt, idim), dtype=torch.float32, device=dev)
        self.q = torch.empty((nt, idim), dtype=torch.int8, device=dev)
        self.d = torch.empty((nt, idim // 32), dtype=torch.float32, device=dev)
        self.s = torch.empty((nt, idim // 32), dtype=torch.float32, device=dev)
        # algorithmic HBM bytes per launch: inputs read, outputs written once
        q8 = n * (1 + 8 / 32)
        self.fbytes = {"add_rmsnorm_quantize": 12 * n + 4 * idim + q8,
                       "rmsnorm_quantize": 4 * n + 4 * idim + q8,
                       "silu_mul_quantize": 8 * n + q8}[op]
        self.cbytes = {"add_rmsnorm_quantize": 12 * n + (8 * n + 4 * idim) + (4 * n + q8),
                       "rmsnorm_quantize": (8 * n + 4 * idim) + (4 * n + q8),
                       "silu_mul_quantize": 12 * n + (4 * n + q8)}[op]
        self.f_ms, self.c_ms = [], []
        self.i = 0
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        st = P(torch.cuda.current_stream().cuda_stream)
        L = self.L = qmm.lib()
        ptr = lambda t: P(t.data_ptr())  # noqa: E731
        q8a = (ptr(self.q), ptr(self.d), ptr(self.s), st)
        W, y = ptr(self.w), ptr(self.y)
        self.fused_calls, self.chain_calls = [], []
        for k in range(ncopy):
            A = ptr(self.a[k])
            if op == "add_rmsnorm_quantize":
                B = ptr(self.b[k])
                self.fused_calls.append([(L.qmm_add_rmsnorm_quantize, (A, B, W, F(self.EPS), I(nt), I(idim)) + q8a)])
                self.chain_calls.append([(L.qmm_residual_add, (A, B, I(nt), I(idim), st)),
                                         (L.qmm_rmsnorm, (A, W, F(self.EPS), I(nt), I(idim), y, st)),
                                         (L.qmm_quantize_act, (y, I(nt), I(idim)) + q8a)])
            elif op == "rmsnorm_quantize":
                self.fused_calls.append([(L.qmm_rmsnorm_quantize, (A, W, F(self.EPS), I(nt), I(idim)) + q8a)])
                self.chain_calls.append([(L.qmm_rmsnorm, (A, W, F(self.EPS), I(nt), I(idim), y, st)),
                                         (L.qmm_quantize_act, (y, I(nt), I(idim)) + q8a)])
            else:
                B = ptr(self.b[k])
                self.fused_calls.append([(L.qmm_silu_mul_quantize, (A, B, I(nt), I(idim)) + q8a)])
                self.chain_calls.append([(L.qmm_silu_mul, (A, B, I(nt), I(idim), y, st)),
                                         (L.qmm_quantize_act, (y, I(nt), I(idim)) + q8a)])

    @staticmethod
    def _issue(seq):
        for f, args in seq:
            rc = f(*args)
            if rc:
                raise RuntimeError(f"{f.__name__} failed: {rc}")

    def fused(self):
        self._issue(self.fused_calls[self.i % len(self.fused_calls)])
        self.i += 1

    def chain(self):
        self._issue(self.chain_calls[self.i % len(self.chain_calls)])
        self.i += 1


def fused_kernel_name(op, idim):
    """(trace name, launch threads per row or per element group) of a fused kernel."""
    if op == "silu_mul_quantize":
        return "qmm::{anonymous}::silu_mul_kernel<1>"
    nch = (idim // 4 + 255) // 256
    ch = next((c for c in (1, 2, 4, 8, 16) if nch <= c), 0)
    add = "true" if op == "add_rmsnorm_quantize" else "false"
    return f"qmm::{{anonymous}}::rmsnorm_kernel<{ch}, {add}, 1>"


def fused_cpu_baseline(calls):
    """The oracle's fused steps (f32 step, then the quantizer) on a bounded sample."""
    import oracle
    oracle.build(force=False)
    nbytes, t_total, reps = 0.0, 0.0, 0
    rows = 64
    data = []
    for c in calls:
        if c.nt < 512:
            continue
        a = c.a[0][:rows].cpu().numpy()
        b = c.b[0][:rows].cpu().numpy() if c.b[0] is not None else None
        data.append((c, a, b, c.w.cpu().numpy(), c.fbytes * rows / c.nt))
    while t_total < 10.0:
        for c, a, b, w, nb in data:
            t0 = time.perf_counter()
            if c.op == "add_rmsnorm_quantize":
                oracle.quantize(oracle.add_rmsnorm(a, b, w, FusedCall.EPS)[1])
            elif c.op == "rmsnorm_quantize":
                oracle.quantize(oracle.rmsnorm(a, w, FusedCall.EPS))
            else:
                oracle.quantize(oracle.silu_mul(a, b))
            t_total += time.perf_counter() - t0
            nbytes += nb
        reps += 1
    return {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the three fused steps on the first {rows} rows of each nt=512 call "
                      f"({', '.join(c.label for c, *_ in data)}), repeated {reps}x, {t_total:.1f} s"}


def run_fused(args, torch, qmm):
    from profile_summary import read_traffic

    calls = []
    for op, idim in (("add_rmsnorm_quantize", 4096), ("rmsnorm_quantize", 4096), ("silu_mul_quantize", 12288)):
        for nt in (1, 512):
            calls.append(FusedCall(torch, qmm, op, nt, idim, seed=31 + nt + idim))
    cal = copy_calibration(torch, args.copy_calibration) if args.copy_calibration > 0 else None
    st = torch.cuda.current_stream()
    chunk = min(CHUNK, args.steps)
    nchunks = max(1, args.steps // chunk)
    steps = chunk * nchunks
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in calls] for _ in range(nchunks)]
    for _ in range(args.warmup):
        for c in calls:
            c.fused()
            c.chain()
    torch.cuda.synchronize()
    gate_cycles = 2_000_000
    t0 = time.perf_counter()
    for ch in range(nchunks):
        torch.cuda._sleep(gate_cycles)
        for c, (e0, e1, e2) in zip(calls, evs[ch]):
            e0.record(st)
            for _ in range(chunk):
                c.fused()
            e1.record(st)
            for _ in range(chunk):
                c.chain()
            e2.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ch in range(nchunks):
        for c, (e0, e1, e2) in zip(calls, evs[ch]):
            c.f_ms.append(e0.elapsed_time(e1) / chunk)
            c.c_ms.append(e1.elapsed_time(e2) / chunk)

    detail = []
    for c in calls:
        f, cm = float(np.mean(c.f_ms)), float(np.mean(c.c_ms))
        gbs = c.fbytes / (f * 1e-3) / 1e9
        detail.append({"call": c.label, "fused_us": round(f * 1e3, 2), "chain_us": round(cm * 1e3, 2),
                       "chain_over_fused": round(cm / f, 2), "fused_bytes": int(c.fbytes),
                       "chain_bytes": int(c.cbytes), "fused_GB_s": round(gbs, 1),
                       "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    big = [c for c in calls if c.nt == 512]
    tb = sum(c.fbytes for c in big)
    tt = sum(float(np.mean(c.f_ms)) * 1e-3 for c in big)
    head = max(big, key=lambda c: c.fbytes)
    kh = float(np.mean(head.f_ms)) * 1e-3
    kname = fused_kernel_name(head.op, head.idim)
    grid = -(-head.nt * head.idim // 4 // 256) * 256
    line = {"metric": "producer-fused quantize: HBM GB/s of the fused kernels at nt=512",
            "value": round(tb / tt / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
            "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / steps, 4),
            "gpu_ms_per_step": round(sum(float(np.mean(c.f_ms)) + float(np.mean(c.c_ms)) for c in calls), 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded; no model weights)",
            "roofline": {"bound": "hbm", "achieved": round(head.fbytes / kh / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(head.fbytes / kh / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": read_traffic(FUSED_COUNTERS, kname, grid),
                         "kernel": kname.replace("qmm::{anonymous}::", "").replace(" ", ""),
                         "call": head.label, "bytes_per_launch": int(head.fbytes)},
            "config": {"workload": "fused_quantize", "hidden": 4096, "ffn": 12288, "nt": [1, 512],
                       "input_copies_bytes_per_shape": COPY_BYTES},
            "detail": detail}
    if cal:
        line["copy_calibration"] = cal
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = fused_cpu_baseline(calls)
    print(json.dumps(line), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _median_rate(fn, units, min_s):
    """Median over 3 timing loops (each at least min_s seconds of calls to fn) of units per
    second, and the three rates."""
    rates = []
    for _ in range(3):
        t, u = 0.0, 0.0
        while t < min_s:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            u += units
        rates.append(u / t)
    return float(np.median(rates)), rates


def cpu_baseline(calls):
    """The CPU oracle as it stands (plain C, -O2, OpenMP over output rows) on a bounded
    sample of the same workload, on one thread and on every thread OpenMP starts;
    each figure the median of 3 timing loops.  Decode: quantize + matmul of every nt = 1
    call (GB/s of the same algorithmic bytes as the GPU line).  Prefill: quantize +
    matmul of the first rows of the largest nt >= 9 per-32 call (int8 TOP/s)."""
    import oracle
    oracle.build(force=False)
    allc = oracle.num_threads()
    dec = [c for c in calls if c.nt == 1 and c.w_host is not None]
    big = [c for c in calls if c.nt >= 9 and not c.q8k and c.w_host is not None]
    res = {"kind": "oracle", "cores": allc, "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
           "timing": "median of 3 loops per figure, compute only (inputs on the host)"}
    data = [(c, c.x.cpu().numpy()) for c in dec]
    if not dec and not big:
        return {"kind": "oracle", "cores": allc, "cpu_model": _cpu_model(), "value": None, "unit": None,
                "sample": "none: no call of this workload keeps host weights"}
    pre = None
    if big:
        c = max(big, key=lambda b: b.ops)
        pre = (c, c.x.cpu().numpy(), c.wbytes // c.od)
    try:
        for threads, key in ((1, "single_thread"), (allc, "all_cores")):
            oracle.set_num_threads(threads)
            row = {"threads": threads}
            if data:
                nbytes = sum(c.kbytes for c, _ in data)
                v, runs = _median_rate(lambda: [oracle.matmul(c.qtype, c.w_host, x, c.od) for c, x in data],
                                       nbytes, 1.5)
                row.update(GB_s=round(v / 1e9, 3), GB_s_runs=[round(r / 1e9, 3) for r in runs])
            if pre is not None:
                c, x, bpr = pre
                rows = 64 if threads == 1 else 64 * threads
                W = c.w_host[: rows * bpr]
                v, runs = _median_rate(lambda: oracle.matmul(c.qtype, W, x, rows), 2.0 * c.nt * rows * c.idim, 1.0)
                row.update(TOP_s=round(v / 1e12, 5), TOP_s_runs=[round(r / 1e12, 5) for r in runs],
                           prefill_rows=rows)
            res[key] = row
    finally:
        oracle.set_num_threads(allc)
    a = res["all_cores"]
    if "GB_s" in a:
        res.update(value=a["GB_s"], unit="GB/s")
    else:
        res.update(value=a["TOP_s"], unit="TOP/s")
    parts = []
    if data:
        parts.append(f"decode: quantize + matmul of every nt=1 call ({', '.join(c.label for c, _ in data)})")
    if pre is not None:
        parts.append(f"prefill: quantize + matmul of {pre[0].label} on its first 64 rows per thread")
    res["sample"] = "; ".join(parts)
    if pre is not None:
        res["mmq_value"], res["mmq_unit"] = a["TOP_s"], "TOP/s"
    return res


KIND_LABEL = {1: "mmvq", 7: "small_batch"}   # QMM_KIND_MMVQ, QMM_KIND_SKINNY; the rest are MMQ kernels


def kms(c):
    """Mean per-launch matmul kernel time of a call over the timed region, in seconds."""
    return float(np.mean(c.k_ms)) * 1e-3


def q8k_kernel(qmm, c):
    """Name and launch size (threads) of the Q4_K Q8_K matrix kernel qmm_matmul_q8k runs
    for call c: the wave kernel with the scales in the int8 operand above 256 tiles of
    128 x 64, else the staged kernel of the cost model's tile."""
    t128 = -(-c.nt // 64) * -(-c.od // 128)
    if c.qtype == qmm.QMM_TYPE_Q4_K and t128 > 256:
        return "qmm::{anonymous}::mmq_k4_q8k_v2_kernel<1, false>", 8 * -(-t128 // 8) * 256
    wr, wc, ks = MMQ_TILES[qmm.qmm_q8k_tile(c.nt, c.od, c.idim)]
    tiles = -(-c.nt // (32 * wc)) * -(-c.od // (32 * wr))
    return f"qmm::mmq_k4_q8k_kernel<{wr}, {wc}, {ks}, false, false>", 8 * -(-tiles // 8) * 64 * wr * wc * ks


def report_default(line, calls, qmm, torch, read_traffic):
    """The default workload's line: value = Q4_K MMVQ GB/s at nt = 1 over the 4096 x 4096
    and 12288 x 4096 calls; roofline = the 12288 x 4096 one; mmq = the per-32 matrix
    kernel at nt = 512 (int8 TOP/s); mmq_q8k = the Q8_K matrix kernel on the same
    weights and inputs; q6k_head and gemv_1024x4096 the Q6_K output projection and
    the small decode GEMV; measured = the GPU's measured limits (bench_peaks), each
    roofline also given as a fraction of them."""
    import bench_peaks

    Q4 = qmm.QMM_TYPE_Q4_K
    dec = [c for c in calls if c.nt == 1 and c.qtype == Q4 and c.od in (4096, 12288)]
    tb = sum(c.kbytes for c in dec)
    tt = sum(kms(c) for c in dec)
    line.update(value=round(tb / tt / 1e9, 1), unit="GB/s")
    # the same bytes over quantize + MMVQ time: the whole decode call
    tq = sum(float(np.mean(c.q_ms)) * 1e-3 for c in dec)
    line["decode_with_quantize_GB_s"] = round(tb / (tt + tq) / 1e9, 1)

    # measured limits: streaming reads of the weight byte counts, int8 MFMA issue rate
    rd = {r["bytes"]: r for r in bench_peaks.stream_read(torch, [9437184, 28311552, 107520000])}
    mf = bench_peaks.mfma_rate(torch, reps=3, waves=(4,))["int8"][0]
    line["measured"] = {"stream_read": list(rd.values()), "int8_mfma_TOP_s": mf["T_s"],
                        "int8_mfma_clock_GHz": mf["clock_GHz"],
                        "note": "plain kernels of bench_peaks.hip run in this process"}

    head = max(dec, key=lambda c: c.od)
    kh = kms(head)
    ach = head.kbytes / kh / 1e9
    line["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                        "frac_of_measured": round(ach / rd[28311552]["GB_s"], 4),
                        "measured_peak": rd[28311552]["GB_s"],
                        "traffic": read_traffic(COUNTERS, "qmm::mmvq_q4k_kernel<1, 4, false>", None),
                        "kernel": "mmvq_q4k_kernel<1,4,false>", "call": head.label,
                        "bytes_per_launch": int(head.kbytes)}

    # decode with a few tokens (the weights streamed once for all of them)
    few = [c for c in calls if c.qtype == Q4 and 2 <= c.nt <= 16 and not c.q8k]
    if few:
        line["small_batch"] = {
            c.label: {"kernel": KIND_LABEL.get(c.kind, "mmq"), "us": round(kms(c) * 1e6, 2),
                      "GB_s": round(c.kbytes / kms(c) / 1e9, 1),
                      "frac_of_measured": round(c.kbytes / kms(c) / 1e9 / rd[min(rd, key=lambda b: abs(b - c.kbytes))]
                                                ["GB_s"], 4)}
            for c in few}

    big = [c for c in calls if c.nt >= 9 and not c.q8k]
    ops = sum(c.ops for c in big)
    m = max(big, key=kms)
    ta = m.ops / kms(m) / 1e12
    mk, mg = mmq_kernel(qmm, m.nt, m.od, m.idim)
    line["mmq"] = {"value": round(ops / sum(kms(c) for c in big) / 1e12, 2), "unit": "TOP/s",
                   "roofline": {"bound": "mfma", "achieved": round(ta, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                                "frac": round(ta / INT8_PEAK_TOPS, 4),
                                "frac_of_measured": round(ta / mf["T_s"], 4), "measured_peak": mf["T_s"],
                                "traffic": read_traffic(COUNTERS, mk, mg),
                                "kernel": mk.replace("qmm::", "").replace(" ", ""), "call": m.label,
                                "ops_per_launch": int(m.ops)},
                   "per_call": {c.label: {"us": round(kms(c) * 1e6, 2), "TOP_s": round(c.ops / kms(c) / 1e12, 2),
                                          "int8_frac": round(c.ops / kms(c) / 1e12 / INT8_PEAK_TOPS, 4)}
                                for c in big}}
    if "streamk" in mk:
        # one kernel and one grid for both prefill shapes: the counters give their mean
        line["mmq"]["roofline"]["traffic_note"] = "HBM bytes per launch, mean over both nt=512 shapes"

    k8 = [c for c in calls if c.q8k]
    if k8:
        m8 = max(k8, key=kms)
        t8 = m8.ops / kms(m8) / 1e12
        k8name, k8threads = q8k_kernel(qmm, m8)
        line["mmq_q8k"] = {"value": round(sum(c.ops for c in k8) / sum(kms(c) for c in k8) / 1e12, 2),
                           "unit": "TOP/s", "activations": "Q8_K: one scale per 256 values (its own numerics)",
                           "roofline": {"bound": "mfma", "achieved": round(t8, 2), "peak": INT8_PEAK_TOPS,
                                        "unit": "TOP/s", "frac": round(t8 / INT8_PEAK_TOPS, 4),
                                        "frac_of_measured": round(t8 / mf["T_s"], 4),
                                        "traffic": read_traffic(COUNTERS, k8name, k8threads),
                                        "kernel": k8name.replace("qmm::", "").replace(" ", ""), "call": m8.label},
                           "per_call": {c.label: {"us": round(kms(c) * 1e6, 2),
                                                  "TOP_s": round(c.ops / kms(c) / 1e12, 2)} for c in k8}}

    q6 = [c for c in calls if c.nt == 1 and c.od == 32000]
    if q6:
        alg = q6[0].kbytes   # 210-byte blocks: the algorithmic bytes of either layout
        line["q6k_head"] = {c.label: {"us": round(kms(c) * 1e6, 2), "GB_s": round(alg / kms(c) / 1e9, 1),
                                      "hbm_frac": round(alg / kms(c) / 1e9 / HBM_PEAK_GBS, 4),
                                      "frac_of_measured": round(alg / kms(c) / 1e9 / rd[107520000]["GB_s"], 4)}
                            for c in q6}
        line["q6k_head"]["bytes"] = "algorithmic: 210-byte blocks + q8 activations + f32 output, both layouts"
    c1 = [c for c in calls if c.nt == 1 and c.od == 1024]
    if c1:
        c = c1[0]
        line["gemv_1024x4096"] = {"us": round(kms(c) * 1e6, 2), "GB_s": round(c.kbytes / kms(c) / 1e9, 1),
                                  "note": "2.4 MB of weights: launch-latency bound, no roofline claim"}
    line["config"] = {"workload": "q4k_decode_prefill",
                      "mmvq": "Q4_K 4096x4096 and 12288x4096, nt=1,4,8; Q4_K 1024x4096 nt=1; "
                              "Q6_K 32000x4096 nt=1 (210- and 224-byte blocks)",
                      "mmq": "Q4_K 12288x4096 and 4096x12288, nt=512, 1% outliers x20 (per-32 and Q8_K activations)",
                      "weight_copies_bytes_per_shape": COPY_BYTES}


def dllm_graph(torch, qmm):
    """One diffusion-LM step (32 layers x q, k, v, o, gate, up Q4_K and down Q6_K padded
    at L = 256, distinct weights per layer) as one HIP graph of 224 quantize and 224
    matmul launches: ms per replay and int8 TOP/s including the quantize launches."""
    calls = build_calls(torch, qmm, "dllm_step")
    ops = sum(c.ops for c in calls)
    gms = graph_replay_ms(torch, calls)
    del calls
    torch.cuda.empty_cache()
    return {"ms_per_step": round(gms, 4), "replays": 5, "TOP_s_incl_quantize": round(ops / (gms * 1e-3) / 1e12, 2),
            "int8_frac": round(ops / (gms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "shape": "32 layers x 7 projections at L=256; 4.46 GB of distinct weights per step"}


def spread_pass(torch, calls, chunk, nchunks, gate_cycles):
    """Per call, `nchunks` more event-timed chunks of `chunk` matmul launches after the
    timed region (the same launches and weight rotation): the per-launch time of each
    chunk, for the median and p10 / p90.  The timed region itself holds one chunk per
    call at the default 20 steps, and chunks shorter than 20 launches would let the
    fixed cost of an event (a few microseconds) into the per-launch time."""
    st = torch.cuda.current_stream()
    out = {c: [] for c in calls}
    if nchunks < 1:
        return {c: c.k_ms for c in calls}
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
           for _ in range(nchunks)]
    torch.cuda.synchronize()
    for ch in range(nchunks):
        torch.cuda._sleep(gate_cycles)
        for c, (e0, e1) in zip(calls, evs[ch]):
            c.quantize()
            e0.record(st)
            for _ in range(chunk):
                c.matmul()
            e1.record(st)
    torch.cuda.synchronize()
    for ch in range(nchunks):
        for c, (e0, e1) in zip(calls, evs[ch]):
            out[c].append(e0.elapsed_time(e1) / chunk)
    return out


def run_peaks(args, torch):
    """The measured limits of the GPU (bench_peaks): streaming read at the weight
    byte counts of the decode shapes, MFMA and VALU issue rates, MFMA/VALU overlap."""
    import bench_peaks

    sizes = [9437184, 28311552, 107520000, 112896000]   # Q4_K 4096^2, 12288x4096; Q6_K 32000x4096 (210 / 224 B)
    t0 = time.perf_counter()
    res = bench_peaks.run_all(torch, sizes)
    wall = time.perf_counter() - t0
    i8 = max(res["mfma"]["int8"], key=lambda r: r["T_s"])
    rd = {r["bytes"]: r for r in res["stream_read"]}
    line = {"metric": "measured limits: HBM streaming read (GB/s) and int8 MFMA rate (TOP/s)",
            "value": rd[28311552]["GB_s"], "unit": "GB/s", "n_gpus": 1, "steps": 1, "warmup": 1,
            "ms_per_step": round(wall * 1e3, 1), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8", "data": "synthetic (register-only loops; a plain read of device buffers)",
            "roofline": {"bound": "hbm", "achieved": rd[28311552]["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(rd[28311552]["GB_s"] / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "stream_read_kernel", "bytes_per_launch": 28311552},
            "int8_mfma": {"T_s": i8["T_s"], "unit": "TOP/s", "frac": round(i8["T_s"] / INT8_PEAK_TOPS, 4),
                          "waves_per_simd": i8["waves_per_simd"]},
            "config": {"workload": "peaks", "stream_read_bytes": sizes}, "detail": res}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; across "
              "GPUs each one would hold a slice of the weight rows and run these same kernels "
              "on it, with the outputs gathered afterwards", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_matmul_amd as qmm

    from profile_summary import read_traffic

    torch.cuda.set_device(0)
    if args.workload == "fused_quantize":
        return run_fused(args, torch, qmm)
    if args.workload == "peaks":
        return run_peaks(args, torch)
    calls = build_calls(torch, qmm, args.workload)
    cal = copy_calibration(torch, args.copy_calibration) if args.copy_calibration > 0 else None
    st = torch.cuda.current_stream()
    chunk = min(args.chunk, args.steps)
    nchunks = max(1, args.steps // chunk)
    steps = chunk * nchunks
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in calls] for _ in range(nchunks)]

    for _ in range(args.warmup):
        for c in calls:
            c.run()
    torch.cuda.synchronize()

    # gate: a bounded busy-wait kernel covering the host time to queue the first
    # chunk, so the GPU then runs the queued launches back to back
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(st)
    torch.cuda._sleep(1_000_000)
    g1.record(st)
    torch.cuda.synchronize()
    ns_per_cycle = g0.elapsed_time(g1) * 1e6 / 1_000_000
    h0 = time.perf_counter()
    for c in calls:
        for _ in range(chunk):
            c.run()
    host_s = time.perf_counter() - h0
    torch.cuda.synchronize()
    gate_cycles = int(max(1.5 * host_s, 100e-6) * 1e9 / ns_per_cycle)
    for c in calls:
        c.i = c.i0

    # timed region: K steps, i.e. K launches of every call of the step; launches of
    # one call are issued back to back in chunks bracketed by HIP events on the
    # launch stream (an event costs about 4 us of GPU time, so a chunk of CHUNK
    # launches amortises it)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ch in range(nchunks):
        torch.cuda._sleep(gate_cycles)
        for c, (e0, e1, e2) in zip(calls, evs[ch]):
            e0.record(st)
            for _ in range(chunk):
                c.quantize()
            e1.record(st)
            for _ in range(chunk):
                c.matmul()
            e2.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ch in range(nchunks):
        for c, (e0, e1, e2) in zip(calls, evs[ch]):
            c.q_ms.append(e0.elapsed_time(e1) / chunk)
            c.k_ms.append(e1.elapsed_time(e2) / chunk)
    spread = spread_pass(torch, calls, chunk, args.spread_chunks, gate_cycles)

    detail = []
    for c in calls:
        k = float(np.mean(c.k_ms))
        qm = float(np.mean(c.q_ms))
        sp = spread[c]
        row = {"call": c.label, "kernel": KIND_LABEL.get(c.kind, "mmq"),
               "kernel_us": round(k * 1e3, 2), "quantize_us": round(qm * 1e3, 2),
               "kernel_us_median": round(float(np.median(sp)) * 1e3, 2),
               "kernel_us_p10_p90": [round(float(np.percentile(sp, 10)) * 1e3, 2),
                                     round(float(np.percentile(sp, 90)) * 1e3, 2)],
               "GB_s": round(c.kbytes / (k * 1e-3) / 1e9, 1),
               "TOP_s": round(c.ops / (k * 1e-3) / 1e12, 2)}
        row["hbm_frac"] = round(row["GB_s"] / HBM_PEAK_GBS, 4)
        row["int8_frac"] = round(row["TOP_s"] / INT8_PEAK_TOPS, 4)
        detail.append(row)

    ms_per_step = wall * 1e3 / steps
    gpu_ms = sum(float(np.mean(c.k_ms)) + float(np.mean(c.q_ms)) for c in calls)
    line = {"metric": "Q4_K×q8 matmul: HBM GB/s at nt=1 and int8 TOPS at nt=512 (% of roofline)",
            "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
            "gpu_ms_per_step": round(gpu_ms, 4), "gate_us": round(gate_cycles * ns_per_cycle / 1e3, 1),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic (seeded; no model weights)"}

    dec = [c for c in calls if c.nt == 1]
    big = [c for c in calls if c.nt >= 9]
    if args.workload == "q4k_decode_prefill":
        report_default(line, calls, qmm, torch, read_traffic)
    elif args.workload == "q8k_prefill":
        q8 = [c for c in calls if c.q8k and c.qtype == qmm.QMM_TYPE_Q4_K]
        p32 = [c for c in calls if not c.q8k and c.qtype == qmm.QMM_TYPE_Q4_K]
        k6 = {c.q8k: float(np.mean(c.k_ms)) * 1e3 for c in calls if c.qtype != qmm.QMM_TYPE_Q4_K}
        ops = sum(c.ops for c in q8)
        t8 = sum(float(np.mean(c.k_ms)) * 1e-3 for c in q8)
        t32 = sum(float(np.mean(c.k_ms)) * 1e-3 for c in p32)
        line.update(metric="Q4_K x Q8_K activations matmul: int8 TOP/s at nt=512 (% of roofline)",
                    value=round(ops / t8 / 1e12, 2), unit="TOP/s")
        m = max(q8, key=lambda c: float(np.mean(c.k_ms)))
        km = float(np.mean(m.k_ms)) * 1e-3
        kname, threads = q8k_kernel(qmm, m)
        line["roofline"] = {"bound": "mfma", "achieved": round(m.ops / km / 1e12, 2), "peak": INT8_PEAK_TOPS,
                            "unit": "TOP/s", "frac": round(m.ops / km / 1e12 / INT8_PEAK_TOPS, 4),
                            "traffic": read_traffic(Q8K_COUNTERS, kname, threads),
                            "kernel": kname.replace("qmm::", "").replace(" ", ""), "call": m.label,
                            "ops_per_launch": int(m.ops)}
        line["per32_same_shapes"] = {"value": round(sum(c.ops for c in p32) / t32 / 1e12, 2), "unit": "TOP/s",
                                     "speedup_q8k": round(t32 / t8, 3)}
        ops6 = 2.0 * 512 * 4096 * 12288
        line["q6k_padded_4096x12288"] = {"per32_us": round(k6[False], 2), "q8k_us": round(k6[True], 2),
                                         "q8k_TOP_s": round(ops6 / k6[True] / 1e6, 2),
                                         "speedup_q8k": round(k6[False] / k6[True], 3)}
        line["config"] = {"workload": "q8k_prefill", "shapes": "Q4_K 12288x4096 and 4096x12288, nt=512, "
                          "1% outliers x20", "activations": "Q8_K (one scale per 256) vs per-32"}
    elif args.workload == "streamk":
        sk = [c for c in calls if c.label.endswith("stream-K")]
        tiles = [c for c in calls if not c.label.endswith("stream-K")]
        ksum = lambda cs: sum(float(np.mean(c.k_ms)) * 1e-3 for c in cs)  # noqa: E731
        line.update(metric="Q4_K matmul, stream-K: int8 TOP/s over the diffusion-LM and prefill shapes",
                    value=round(sum(c.ops for c in sk) / ksum(sk) / 1e12, 2), unit="TOP/s")
        m = max(sk, key=lambda c: c.ops / float(np.mean(c.k_ms)))
        km = float(np.mean(m.k_ms)) * 1e-3
        line["roofline"] = {"bound": "mfma", "achieved": round(m.ops / km / 1e12, 2), "peak": INT8_PEAK_TOPS,
                            "unit": "TOP/s", "frac": round(m.ops / km / 1e12 / INT8_PEAK_TOPS, 4), "traffic": None,
                            "kernel": "mmq_q4k_streamk_kernel<4,2> + fixup", "call": m.label,
                            "ops_per_launch": int(m.ops)}
        line["per_tile_dispatch"] = {"value": round(sum(c.ops for c in tiles) / ksum(tiles) / 1e12, 2),
                                     "unit": "TOP/s", "speedup_streamk": round(ksum(tiles) / ksum(sk), 3)}
        line["config"] = {"workload": "streamk", "shapes": "Q4_K 4096x4096 and 12288x4096 at nt=256; "
                          "12288x4096 and 4096x12288 at nt=512"}
    elif args.workload == "formats":
        by = {c.label: c for c in calls}
        k = lambda lab: float(np.mean(by[lab].k_ms)) * 1e-3  # noqa: E731
        head = by["Q4_0 12288x4096 nt=1"]
        line.update(metric="Q4_0 / Q8_0 matmul: HBM GB/s at nt=1 and int8 TOP/s at nt=512",
                    value=round(head.kbytes / k(head.label) / 1e9, 1), unit="GB/s")
        line["roofline"] = {"bound": "hbm", "achieved": line["value"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(line["value"] / HBM_PEAK_GBS, 4), "traffic": None,
                            "kernel": "mmvq_b32_kernel<1,4,false,false>", "call": head.label,
                            "bytes_per_launch": int(head.kbytes)}
        line["per_format"] = {lab: ({"GB_s": round(c.kbytes / k(lab) / 1e9, 1),
                                     "hbm_frac": round(c.kbytes / k(lab) / 1e9 / HBM_PEAK_GBS, 4)} if c.nt == 1 else
                                    {"TOP_s": round(c.ops / k(lab) / 1e12, 2),
                                     "int8_frac": round(c.ops / k(lab) / 1e12 / INT8_PEAK_TOPS, 4)})
                              for lab, c in by.items()}
        line["config"] = {"workload": "formats", "shape": "12288x4096", "nt": [1, 512],
                          "types": ["Q4_0", "Q8_0", "Q5_K", "Q4_K"]}
    elif args.workload == "q6k_head":
        c, cp = dec[0], dec[1]
        k = float(np.mean(c.k_ms)) * 1e-3
        kp = float(np.mean(cp.k_ms)) * 1e-3
        line.update(value=round(c.kbytes / k / 1e9, 1), unit="GB/s")
        line["padded_224"] = {"kernel_us": round(kp * 1e6, 2), "GB_s_bytes_read": round(cp.kbytes / kp / 1e9, 1),
                              "GB_s_unpadded_bytes": round(c.kbytes / kp / 1e9, 1),
                              "speedup_vs_unpadded": round(k / kp, 3)}
        line["roofline"] = {"bound": "hbm", "achieved": line["value"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(line["value"] / HBM_PEAK_GBS, 4), "traffic": None,
                            "kernel": "mmvq_q6k_kernel<1,4,false,false>", "bytes_per_launch": int(c.kbytes)}
        line["config"] = {"workload": "q6k_head", "shape": "Q6_K 32000x4096 nt=1"}
    else:
        ops = sum(c.ops for c in calls)
        t = sum(float(np.mean(c.k_ms)) * 1e-3 for c in calls)
        line.update(value=round(ops / t / 1e12, 2), unit="TOP/s")
        line["note"] = "value = int8 ops of the 224 matmuls over the sum of their kernel times"
        # the whole step (224 quantize + 224 matmul launches) as one HIP graph
        gms = graph_replay_ms(torch, calls)
        line["graph"] = {"ms_per_step": round(gms, 4), "replays": 5,
                         "TOP_s_incl_quantize": round(ops / (gms * 1e-3) / 1e12, 2)}
        # the same matmuls fed as a model's layers feed them (fused producers, one
        # quantized input for q, k, v and one for gate, up)
        lms = layer_graph_ms(torch, qmm, calls)
        line["graph_layers"] = {"ms_per_step": round(lms, 4), "replays": 5, "producer_launches_per_layer": 4,
                                "TOP_s_incl_producers": round(ops / (lms * 1e-3) / 1e12, 2)}
        # the same step on Q8_K activations (one scale per 256 values: other numerics),
        # one Q8_K quantize per matmul as in "graph"
        q8k_calls = [Call(torch, qmm, c.qtype, c.od, c.idim, c.nt, seed=0, outliers=False, copies=c.W[:1], x=c.x,
                          q8k=True, label=c.label + " Q8_K") for c in calls]
        kms = graph_replay_ms(torch, q8k_calls)
        line["graph_q8k"] = {"ms_per_step": round(kms, 4), "replays": 5,
                             "TOP_s_incl_quantize": round(ops / (kms * 1e-3) / 1e12, 2),
                             "activations": "Q8_K (one scale per 256 values, its own numerics)"}
        lkms = layer_graph_ms(torch, qmm, q8k_calls, q8k=True)
        line["graph_layers_q8k"] = {"ms_per_step": round(lkms, 4), "replays": 5, "producer_launches_per_layer": 4,
                                    "TOP_s_incl_producers": round(ops / (lkms * 1e-3) / 1e12, 2)}
        del q8k_calls
        line["config"] = {"workload": "dllm_step", "layers": 32, "canvas": 256, "hidden": 4096, "ffn": 12288,
                          "matmuls_per_step": len(calls), "down_projection": "Q6_K padded to 224-byte blocks"}
        detail = detail[:7]
    line["detail"] = detail
    if cal:
        line["copy_calibration"] = cal
    if args.workload == "q4k_decode_prefill" and not args.no_dllm:
        line["dllm_step"] = dllm_graph(torch, qmm)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(calls)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
