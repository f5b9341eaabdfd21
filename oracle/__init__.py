"""Python access to the CPU oracle (oracle/qmm_oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg may import this package.  The product path (quantized_matmul_amd)
never imports it.  Arrays are numpy; the oracle computes on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

TYPE_Q4_K = 1
TYPE_Q6_K = 2
TYPE_Q6_K_P224 = 3   # Q6_K blocks padded to 224 bytes
TYPE_Q4_0 = 4        # 18-byte blocks of 32 weights
TYPE_Q8_0 = 5        # 34-byte blocks of 32 weights
TYPE_Q5_K = 6        # 176-byte super-blocks (5-bit codes)

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True, out: str = LIB, mutate: int = 0) -> str:
    """Compile the oracle with gcc (into oracle/liboracle.so unless `out` says otherwise).

    mutate > 0 builds a copy with one planted mistake (see OQ_MUTATE in the C file);
    only the tests that check the pins catch those mistakes use it.
    """
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        defs = [f"-DOQ_MUTATE={int(mutate)}"] if mutate else []
        subprocess.run(["gcc", *CFLAGS, *defs, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


def _bind(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L.oracle_quantize.argtypes = [P, I, I, P, P, P]
    L.oracle_subblock_dots.argtypes = [I, P, P, I, I, I, P]
    L.oracle_matmul_q8.argtypes = [I, P, P, P, P, I, I, I, P, P]
    L.oracle_matmul_q8_points.argtypes = [I, P, P, P, P, I, I, I, I, P, P, P, P]
    L.oracle_matmul.argtypes = [I, P, P, I, I, I, P, P, P, P, P]
    L.oracle_decode_block.argtypes = [I, P, P, P, P, P, P]
    F = ctypes.c_float
    L.oracle_rmsnorm.argtypes = [P, P, F, I, I, P]
    L.oracle_add_rmsnorm.argtypes = [P, P, P, F, I, I, P, P]
    L.oracle_silu_mul.argtypes = [P, P, ctypes.c_size_t, P]
    L.oracle_quantize_q8k.argtypes = [P, I, I, P, P, P]
    L.oracle_matmul_q8k.argtypes = [I, P, P, P, P, I, I, I, P, P]
    L.oracle_matmul_q8k_points.argtypes = [I, P, P, P, P, I, I, I, I, P, P, P, P]
    L.oracle_q8k_superblock_sums.argtypes = [I, P, P, P, I, I, I, P]
    L.oracle_decode_group32.argtypes = [I, P, P, P]
    L.oracle_num_threads.restype = I
    L.oracle_set_num_threads.argtypes = [I]
    for f in ("oracle_quantize", "oracle_subblock_dots", "oracle_matmul_q8",
              "oracle_matmul_q8_points", "oracle_matmul", "oracle_decode_block",
              "oracle_rmsnorm", "oracle_add_rmsnorm", "oracle_silu_mul", "oracle_quantize_q8k",
              "oracle_matmul_q8k", "oracle_matmul_q8k_points", "oracle_q8k_superblock_sums",
              "oracle_decode_group32"):
        getattr(L, f).restype = I
    return L


_lib = None
_override = None


def lib():
    """The loaded oracle library (a planted-mistake copy while `use()` is active)."""
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = _bind(LIB)
    return _lib


class use:
    """Context manager: route this module's functions to another oracle build."""

    def __init__(self, path: str):
        self.L = _bind(path)

    def __enter__(self):
        global _override
        self.prev = _override
        _override = self.L
        return self

    def __exit__(self, *exc):
        global _override
        _override = self.prev
        return False


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def quantize(x: np.ndarray):
    """x [nt][id] f32 -> (q [nt][id] int8, d [nt][id/32] f32, s [nt][id/32] f32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nt, idim = x.shape
    q = np.empty((nt, idim), np.int8)
    d = np.empty((nt, idim // 32), np.float32)
    s = np.empty((nt, idim // 32), np.float32)
    _check(lib().oracle_quantize(_p(x), nt, idim, _p(q), _p(d), _p(s)), "oracle_quantize")
    return q, d, s


def subblock_dots(qtype: int, W: np.ndarray, q: np.ndarray, od: int):
    """Integer dot per scale group: [nt][od][id/256][8 (Q4_K) or 16 (Q6_K)] int32."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    nt, idim = q.shape
    ng = 16 if qtype in (TYPE_Q6_K, TYPE_Q6_K_P224) else 8
    S = np.empty((nt, od, idim // 256, ng), np.int32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    _check(lib().oracle_subblock_dots(qtype, _p(W), _p(q), nt, od, idim, _p(S)), "oracle_subblock_dots")
    return S


def matmul_q8(qtype: int, W: np.ndarray, q, d, s, od: int):
    """out [nt][od] f32 and mag [nt][od] f64 (sum of |term|) from quantized activations."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nt, idim = q.shape
    out = np.empty((nt, od), np.float32)
    mag = np.empty((nt, od), np.float64)
    _check(lib().oracle_matmul_q8(qtype, _p(W), _p(q), _p(d), _p(s), nt, od, idim, _p(out), _p(mag)),
           "oracle_matmul_q8")
    return out, mag


def matmul_q8_points(qtype: int, W: np.ndarray, q, d, s, od: int, t_idx, r_idx):
    """Selected outputs (t_idx[k], r_idx[k]) only: returns (out [k] f32, mag [k] f64)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int32)
    r_idx = np.ascontiguousarray(r_idx, dtype=np.int32)
    nt, idim = q.shape
    n = int(t_idx.size)
    out = np.empty(n, np.float32)
    mag = np.empty(n, np.float64)
    _check(lib().oracle_matmul_q8_points(qtype, _p(W), _p(q), _p(d), _p(s), nt, od, idim, n,
                                         _p(t_idx), _p(r_idx), _p(out), _p(mag)), "oracle_matmul_q8_points")
    return out, mag


def matmul(qtype: int, W: np.ndarray, x: np.ndarray, od: int):
    """The whole path on the CPU: returns (out, mag, (q, d, s))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nt, idim = x.shape
    q = np.empty((nt, idim), np.int8)
    d = np.empty((nt, idim // 32), np.float32)
    s = np.empty((nt, idim // 32), np.float32)
    out = np.empty((nt, od), np.float32)
    mag = np.empty((nt, od), np.float64)
    _check(lib().oracle_matmul(qtype, _p(W), _p(x), nt, od, idim, _p(q), _p(d), _p(s), _p(out), _p(mag)),
           "oracle_matmul")
    return out, mag, (q, d, s)


def decode_block(qtype: int, block: np.ndarray):
    """Decoded fields of one super-block: dict(d, dmin, sc, m, codes)."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    d = np.zeros(1, np.float64)
    dmin = np.zeros(1, np.float64)
    sc = np.zeros(16, np.int32)
    m = np.zeros(16, np.int32)
    codes = np.zeros(256, np.int32)
    _check(lib().oracle_decode_block(qtype, _p(b), _p(d), _p(dmin), _p(sc), _p(m), _p(codes)),
           "oracle_decode_block")
    if qtype in (TYPE_Q4_K, TYPE_Q5_K):
        return dict(d=float(d[0]), dmin=float(dmin[0]), sc=sc[:8].copy(), m=m[:8].copy(), codes=codes)
    return dict(d=float(d[0]), sc=sc.copy(), codes=codes)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float):
    """y = (x * r) * w per row, r = 1 / sqrt(mean(x^2) + eps) in the fixed f32 order."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    nt, idim = x.shape
    assert w.shape == (idim,)
    y = np.empty_like(x)
    _check(lib().oracle_rmsnorm(_p(x), _p(w), float(eps), nt, idim, _p(y)), "oracle_rmsnorm")
    return y


def add_rmsnorm(h: np.ndarray, o: np.ndarray, w: np.ndarray, eps: float):
    """Returns (h + o, rmsnorm(h + o))."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    o = np.ascontiguousarray(o, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    nt, idim = h.shape
    assert o.shape == h.shape and w.shape == (idim,)
    hn = np.empty_like(h)
    y = np.empty_like(h)
    _check(lib().oracle_add_rmsnorm(_p(h), _p(o), _p(w), float(eps), nt, idim, _p(hn), _p(y)),
           "oracle_add_rmsnorm")
    return hn, y


def silu_mul(g: np.ndarray, u: np.ndarray):
    """silu(g) * u elementwise (f64 evaluation, one rounding to f32)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    assert g.shape == u.shape
    y = np.empty_like(g)
    _check(lib().oracle_silu_mul(_p(g), _p(u), g.size, _p(y)), "oracle_silu_mul")
    return y


def quantize_q8k(x: np.ndarray):
    """Q8_K activations: (q [nt][id] int8, d [nt][id/256] f32, bsum [nt][id/16] f32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nt, idim = x.shape
    q = np.empty((nt, idim), np.int8)
    d = np.empty((nt, idim // 256), np.float32)
    bs = np.empty((nt, idim // 16), np.float32)
    _check(lib().oracle_quantize_q8k(_p(x), nt, idim, _p(q), _p(d), _p(bs)), "oracle_quantize_q8k")
    return q, d, bs


def matmul_q8k(qtype: int, W: np.ndarray, q, d, bsum, od: int):
    """out [nt][od] f32 and mag [nt][od] f64 from Q8_K activations."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    bsum = np.ascontiguousarray(bsum, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nt, idim = q.shape
    out = np.empty((nt, od), np.float32)
    mag = np.empty((nt, od), np.float64)
    _check(lib().oracle_matmul_q8k(qtype, _p(W), _p(q), _p(d), _p(bsum), nt, od, idim, _p(out), _p(mag)),
           "oracle_matmul_q8k")
    return out, mag


def matmul_q8k_points(qtype: int, W: np.ndarray, q, d, bsum, od: int, t_idx, r_idx):
    """Selected outputs (t_idx[k], r_idx[k]) from Q8_K activations: (out [k] f32, mag [k] f64)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    d = np.ascontiguousarray(d, dtype=np.float32)
    bsum = np.ascontiguousarray(bsum, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    t_idx = np.ascontiguousarray(t_idx, dtype=np.int32)
    r_idx = np.ascontiguousarray(r_idx, dtype=np.int32)
    nt, idim = q.shape
    n = int(t_idx.size)
    out = np.empty(n, np.float32)
    mag = np.empty(n, np.float64)
    _check(lib().oracle_matmul_q8k_points(qtype, _p(W), _p(q), _p(d), _p(bsum), nt, od, idim, n, _p(t_idx),
                                          _p(r_idx), _p(out), _p(mag)), "oracle_matmul_q8k_points")
    return out, mag


def q8k_superblock_sums(qtype: int, W: np.ndarray, q, bsum, od: int):
    """Integer stage of the Q8_K matmul: [nt][od][id/256][2] int32 (scaled dot sum, min sum)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    bsum = np.ascontiguousarray(bsum, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    nt, idim = q.shape
    S = np.empty((nt, od, idim // 256, 2), np.int32)
    _check(lib().oracle_q8k_superblock_sums(qtype, _p(W), _p(q), _p(bsum), nt, od, idim, _p(S)),
           "oracle_q8k_superblock_sums")
    return S


def decode_group32(qtype: int, group: np.ndarray):
    """Eight 32-weight blocks (Q4_0 or Q8_0): (d [8] f64, centred codes [256] int32)."""
    g = np.ascontiguousarray(group, dtype=np.uint8)
    d = np.zeros(8, np.float64)
    codes = np.zeros(256, np.int32)
    _check(lib().oracle_decode_group32(qtype, _p(g), _p(d), _p(codes)), "oracle_decode_group32")
    return d, codes


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))
