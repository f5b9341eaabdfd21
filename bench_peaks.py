"""Measured limits of the GPU, for the roofline figures of bench.py.

The kernels are in bench_peaks.hip (built into libbench_peaks.so by
__graft_entry__.build()).  [CH04, section 4.2] puts a measured streaming rate
beside the documented peak; these functions give the measured side:

  stream_read   HBM streaming-read rate at given byte counts (16-byte loads, every
                byte read once, launches rotating over more than 1 GiB of buffer so
                every read comes from HBM);
  mfma_rate     issue rate of v_mfma_i32_32x32x32_i8 (int8 TOP/s) and of the f32
                outer-product pair, at 1, 2 and 4 waves per SIMD, with the shader
                clock the chip ran at;
  valu_rate     issue rate of v_fma_f32 and of the epilogue pair cvt + fma;
  overlap       time of MFMA work and VALU work together against each alone, in
                one wave (interleaved) and split over the two waves of a SIMD;
  load_shape    loads without arithmetic of a Q4_K 12288 x 4096 matrix in the vector
                kernel's shape (a 16-byte header and a 16-byte code chunk per lane and
                row) and as each row's consecutive 16-byte pieces, same rotation.

All times come from HIP events on the launch stream.
"""
from __future__ import annotations

import ctypes
import os
import statistics
import subprocess

ROOT = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ROOT, "bench_peaks.hip")
LIB = os.path.join(ROOT, "libbench_peaks.so")
CUS, SIMDS = 256, 4

_lib = None


def build(out: str = LIB) -> str:
    from quantized_matmul_amd import _build

    tmp = out + ".tmp"
    # MFMA results in VGPRs, where the library's matrix kernels get them (the compiler
    # otherwise moves the results of these small kernels to AGPRs and reads them back)
    subprocess.run([_build.HIPCC, *_build.FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form=1", SRC, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB)
        P, I = ctypes.c_void_p, ctypes.c_int
        L.peaks_stream_read.argtypes = [P, ctypes.c_size_t, I, P, P]
        L.peaks_load_shape.argtypes = [P, I, I, P, P]
        L.peaks_rate.argtypes = [I, I, I, P, P, P]
        L.peaks_overlap.argtypes = [I, I, I, I, I, P, P]
        L.peaks_valu_instr.argtypes = [I, I, I, P, P]
        L.peaks_lds_read.argtypes = [I, I, P, P]
        L.peaks_mfma_mix.argtypes = [I, I, I, P, P]
        L.peaks_shadow.argtypes = [I, I, I, I, P, P]
        L.peaks_pingpong.argtypes = [I, I, I, P, P]
        L.peaks_burst.argtypes = [I, I, I, P, P]
        for f in ("peaks_stream_read", "peaks_rate", "peaks_overlap", "peaks_valu_instr", "peaks_lds_read",
                  "peaks_mfma_mix", "peaks_shadow", "peaks_pingpong", "peaks_burst", "peaks_load_shape"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _check(rc, what):
    if rc:
        raise RuntimeError(f"{what}: launch failed (hipError {rc})")


def _timed(torch, launch, per_chunk, chunks):
    """Per-launch ms of each of `chunks` chunks of `per_chunk` back-to-back launches
    (events around each chunk, a busy-wait gate first so the host queues ahead)."""
    st = torch.cuda.current_stream()
    launch(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(chunks)]
    torch.cuda._sleep(200_000)
    i = 0
    for e0, e1 in evs:
        e0.record(st)
        for _ in range(per_chunk):
            launch(i)
            i += 1
        e1.record(st)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) / per_chunk for e0, e1 in evs]


def stream_read(torch, sizes, copy_bytes=1 << 30, per_chunk=20, chunks=5):
    """For each byte count: the fastest (over 1, 2, 4, 8 loads per lane) median
    per-launch time of a plain streaming read, and its rate."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = []
    for size in sizes:
        best = None
        for u in (1, 2, 4, 8):
            per_wg = 4096 * u
            n = -(-size // per_wg) * per_wg          # whole workgroups: may read a few KiB more
            stride = -(-n // 65536) * 65536
            copies = max(2, -(-copy_bytes // stride))
            buf = torch.empty(stride * copies, dtype=torch.uint8, device="cuda:0")
            sink = torch.empty(n // per_wg, dtype=torch.int32, device="cuda:0")
            base = buf.data_ptr()
            sp = ctypes.c_void_p(sink.data_ptr())

            def launch(i, base=base, n=n, u=u, stride=stride, copies=copies, sp=sp):
                _check(L.peaks_stream_read(ctypes.c_void_p(base + (i % copies) * stride), n, u, sp, st), "stream_read")

            ms = statistics.median(_timed(torch, launch, per_chunk, chunks))
            if best is None or ms < best[0]:
                best = (ms, u, n)
            del buf, sink
        ms, u, n = best
        res.append({"bytes": size, "bytes_read": n, "us": round(ms * 1e3, 3),
                    "GB_s": round(n / (ms * 1e-3) / 1e9, 1), "loads_per_lane": u})
    return res


def load_shape(torch, rows=12288, copy_bytes=1 << 30, per_chunk=20, chunks=5):
    """Median per-launch time of both load shapes over a Q4_K rows x 4096 matrix
    (144-byte blocks, 16 per row), launches rotating over > copy_bytes of copies."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = rows * 16 * 144
    stride = -(-n // 65536) * 65536
    copies = max(2, -(-copy_bytes // stride))
    buf = torch.empty(stride * copies, dtype=torch.uint8, device="cuda:0")
    sink = torch.empty(rows // 4, dtype=torch.int32, device="cuda:0")
    base, sp = buf.data_ptr(), ctypes.c_void_p(sink.data_ptr())
    res = []
    for shape, name in ((0, "header + code chunk per lane and row"), (1, "consecutive 16-byte pieces per row")):
        def launch(i, shape=shape):
            _check(L.peaks_load_shape(ctypes.c_void_p(base + (i % copies) * stride), rows, shape, sp, st),
                   "load_shape")

        ms = statistics.median(_timed(torch, launch, per_chunk, chunks))
        res.append({"shape": name, "rows": rows, "bytes": n, "us": round(ms * 1e3, 3),
                    "GB_s": round(n / (ms * 1e-3) / 1e9, 1)})
    del buf, sink
    return res


def _clock_ghz(clk):
    c = clk.cpu().tolist()
    return round(c[0] / c[1] * 0.1, 3) if c[1] > 0 else None


def mfma_rate(torch, reps=3, waves=(1, 2, 4)):
    """int8 MFMA (32x32x32) and f32 outer-product MFMA rates at 1, 2, 4 waves per SIMD."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {"int8": [], "f32_outer": []}
    for w in waves:
        blocks = CUS * w                       # 4 waves per workgroup: w per SIMD
        iters = 8192 // w
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")
        clk = torch.zeros(2, dtype=torch.int64, device="cuda:0")
        for kind, key, ops_per in ((0, "int8", 8 * 32 * 32 * 32 * 2), (1, "f32_outer", 4 * 2 * 32 * 32 * 2)):
            def launch(i, kind=kind):
                _check(L.peaks_rate(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.c_void_p(clk.data_ptr()) if kind == 0 else None, st), "peaks_rate")

            ms = statistics.median(_timed(torch, launch, 1, reps))
            ops = ops_per * iters * blocks * 4
            row = {"waves_per_simd": w, "ms": round(ms, 4), "T_s": round(ops / (ms * 1e-3) / 1e12, 1)}
            if kind == 0:
                row["clock_GHz"] = _clock_ghz(clk)
                # SIMD clocks per instruction at the measured clock
                if row["clock_GHz"]:
                    row["clocks_per_instr"] = round(ms * 1e-3 * row["clock_GHz"] * 1e9 / (iters * 8 * w), 2)
            out[key].append(row)
    return out


def valu_rate(torch, reps=3):
    """v_fma_f32 and cvt + fma pair rates at 1, 2, 4 waves per SIMD, as SIMD clocks
    per wave64 instruction at the measured clock."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = {"fma": [], "cvt_fma": []}
    for w in (1, 2, 4):
        blocks = CUS * w
        iters = 4096 // w
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")
        clk = torch.zeros(2, dtype=torch.int64, device="cuda:0")
        for kind, key, instr in ((2, "fma", 128), (3, "cvt_fma", 256 + 16)):
            def launch(i, kind=kind):
                _check(L.peaks_rate(kind, blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.c_void_p(clk.data_ptr()), st), "peaks_rate")

            ms = statistics.median(_timed(torch, launch, 1, reps))
            ghz = _clock_ghz(clk)
            n_instr = instr * iters * w      # wave instructions per SIMD
            row = {"waves_per_simd": w, "ms": round(ms, 4), "clock_GHz": ghz,
                   "lane_ops_T_s": round(instr * iters * blocks * 4 * 64 / (ms * 1e-3) / 1e12, 2)}
            if ghz:
                row["clocks_per_instr"] = round(ms * 1e-3 * ghz * 1e9 / n_instr, 3)
            out[key].append(row)
    return out


VALU_OPS = ["v_fmac_f32 (VOP2)", "v_fma_f32 (VOP3)", "v_fma_f32 (VOP3, SGPR operand)", "v_cvt_f32_i32",
            "v_mul_f32", "v_and_b32", "v_lshrrev_b32", "v_add_u32", "v_cvt_f32_i32 + v_fmac_f32 (pair)",
            "v_mad_u32_u24"]


def valu_instr(torch, clock_ghz, reps=3):
    """SIMD clocks per wave64 instruction of each VALU form (at the clock measured by
    valu_rate), 1, 2 and 4 waves per SIMD."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for op, name in enumerate(VALU_OPS):
        row = {"instr": name}
        for w in (1, 2, 4):
            blocks, iters = CUS * w, 2048 // w
            sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

            def launch(i, op=op):
                _check(L.peaks_valu_instr(op, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "valu_instr")

            ms = statistics.median(_timed(torch, launch, 1, reps))
            n_instr = 128 * iters * w * (2 if op == 8 else 1)
            row[f"clocks_w{w}"] = round(ms * 1e-3 * clock_ghz * 1e9 / n_instr, 3)
        out.append(row)
    return out


def lds_read(torch, clock_ghz, reps=3):
    """LDS read bandwidth with ds_read_b128, 8 waves per CU: bytes per CU per clock."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = CUS, 4096
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

    def launch(i):
        _check(L.peaks_lds_read(blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "lds_read")

    ms = statistics.median(_timed(torch, launch, 1, reps))
    nbytes = blocks * 512 * 16 * 16 * iters
    return {"ms": round(ms, 4), "TB_s": round(nbytes / (ms * 1e-3) / 1e12, 2),
            "bytes_per_cu_per_clock": round(nbytes / CUS / (ms * 1e-3 * clock_ghz * 1e9), 1)}


def overlap(torch, reps=3):
    """MFMA + VALU together against each alone (2 waves per SIMD: 256 workgroups of
    8 waves).  overlap = (t_mfma + t_valu - t_both) / min(t_mfma, t_valu): 1 when the
    shorter part hides completely under the longer, 0 when the times add."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = CUS, 2048
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")
    res = []
    for split in (0, 1):
        for nv in (4, 8, 16):
            t = {}
            for parts in (1, 2, 3):
                def launch(i, parts=parts):
                    _check(L.peaks_overlap(nv, split, parts, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st),
                           "peaks_overlap")

                t[parts] = statistics.median(_timed(torch, launch, 1, reps))
            tm, tv, tb = t[1], t[2], t[3]
            res.append({"mode": "one wave, interleaved" if split == 0 else "two waves per SIMD, one MFMA, one VALU",
                        "valu_per_mfma": nv, "mfma_ms": round(tm, 4), "valu_ms": round(tv, 4),
                        "both_ms": round(tb, 4), "overlap": round((tm + tv - tb) / min(tm, tv), 3)})
    return res


MIX_MODES = ["2 int8 (fixed accumulator input) + 1 f32 outer pair", "2 int8 (fixed accumulator input)",
             "1 f32 outer pair", "2 int8 (accumulating)"]


def mfma_mix(torch, clock_ghz, reps=3):
    """SIMD clocks per step of each MFMA mix (mfma_mix_kernel), 1 and 2 waves per SIMD."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for mode, name in enumerate(MIX_MODES):
        row = {"mix": name}
        for w in (1, 2):
            blocks, iters = CUS * w, 1024 // w
            sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

            def launch(i, mode=mode):
                _check(L.peaks_mfma_mix(mode, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "mfma_mix")

            ms = statistics.median(_timed(torch, launch, 1, reps))
            row[f"clocks_per_step_w{w}"] = round(ms * 1e-3 * clock_ghz * 1e9 / (8 * iters * w), 1)
        out.append(row)
    return out


def shadow(torch, clock_ghz, reps=3):
    """SIMD clocks per step (one int8 MFMA + nv VOP2 fmacs in one wave) at 1 and 2
    waves per SIMD, with the MFMA-only and VALU-only times: hidden = the share of
    the shorter part that does not add to the time."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for nv in (4, 8, 12, 16, 24, 32):
        row = {"valu_per_mfma": nv}
        for w in (1, 2):
            blocks, iters = CUS * w, 1024 // w
            sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")
            t = {}
            for parts in (1, 2, 3):
                def launch(i, parts=parts):
                    _check(L.peaks_shadow(nv, parts, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "shadow")

                t[parts] = statistics.median(_timed(torch, launch, 1, reps)) * 1e-3 * clock_ghz * 1e9 / (8 * iters * w)
            row[f"w{w}"] = {"mfma": round(t[1], 1), "valu": round(t[2], 1), "both": round(t[3], 1),
                            "hidden": round((t[1] + t[2] - t[3]) / min(t[1], t[2]), 3)}
        out.append(row)
    return out


def pingpong(torch, clock_ghz, reps=3):
    """SIMD clocks per round (per wave: the MFMAs of two per-32 sub-blocks over two
    token blocks and their epilogue) with the phases alternating between the two
    waves of a SIMD (barrier between phases) and with each wave doing both in turn."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = CUS, 512
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")
    out = {}
    for pp, key in ((0, "serial"), (1, "pingpong")):
        def launch(i, pp=pp):
            _check(L.peaks_pingpong(pp, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "pingpong")

        ms = statistics.median(_timed(torch, launch, 1, reps))
        out[key] = round(ms * 1e-3 * clock_ghz * 1e9 / iters, 1)   # SIMD clocks per round (2 waves)
    return out


BURST_MODES = [(1, 2), (2, 2), (2, 1), (4, 1), (8, 1), (4, 2)]   # (sub-blocks per burst, token blocks)


def burst(torch, clock_ghz, reps=3):
    """SIMD clocks per 32 x 32 x 32 block (one int8 MFMA, its share of the outer
    products and its 32-instruction epilogue) by burst length, 2 waves per SIMD."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for mode, (nb, nn) in enumerate(BURST_MODES):
        blocks = CUS * 2
        iters = 2048 // (nb * nn)
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

        def launch(i, mode=mode):
            _check(L.peaks_burst(mode, blocks, iters, ctypes.c_void_p(sink.data_ptr()), st), "burst")

        ms = statistics.median(_timed(torch, launch, 1, reps))
        per_block = ms * 1e-3 * clock_ghz * 1e9 / (iters * nb * nn * 2)   # 2 waves per SIMD
        out.append({"subblocks_per_burst": nb, "token_blocks": nn, "clocks_per_block": round(per_block, 1),
                    "int8_frac_of_mfma": round(32.8 / per_block, 3)})
    return out


def run_all(torch, sizes):
    res = {"stream_read": stream_read(torch, sizes), "mfma": mfma_rate(torch), "valu": valu_rate(torch)}
    ghz = res["valu"]["fma"][-1]["clock_GHz"] or 2.4
    res["valu_instr"] = valu_instr(torch, ghz)
    res["lds_read"] = lds_read(torch, ghz)
    res["mfma_mix"] = mfma_mix(torch, res["mfma"]["int8"][-1]["clock_GHz"] or ghz)
    res["shadow"] = shadow(torch, res["mfma"]["int8"][-1]["clock_GHz"] or ghz)
    res["pingpong"] = pingpong(torch, res["mfma"]["int8"][-1]["clock_GHz"] or ghz)
    res["burst"] = burst(torch, res["mfma"]["int8"][-1]["clock_GHz"] or ghz)
    res["overlap"] = overlap(torch)
    res["load_shape"] = load_shape(torch)
    return res
