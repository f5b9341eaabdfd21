"""Element-indexed f64 dequantizer and brute-force matmul (test helper).

Written independently of the oracle's block loops: every weight is produced on
its own from its element index, straight from the byte layouts the pages give,
and the matmul is a plain f64 dot of dequantized weights with activations.
Small sizes only (pure Python over elements).

Pages: "The quantized GEMM" (mojo-dllm), The GPU path (Q4_K header / code split
and the nibble-pair rule; Q6_K field order); "llama.cpp MMQ ..." section 6
(get_scale_min_k4 semantics, value d*sc*v - dmin*m) and section 4 (Q6_K value
d*sc*(code-32), one int8 scale per 16).  The Q6_K element-to-bit map is this
build's reading (public GGUF arrangement), not fixed by the pages.
"""
from __future__ import annotations

import numpy as np


def f16(lo: int, hi: int) -> float:
    return float(np.array([lo | (hi << 8)], dtype=np.uint16).view(np.float16)[0])


def q4k_field(block: np.ndarray, j: int):
    """(sc, m) of sub-block j read as bit fields of the 12 header bytes 4..15."""
    s = [int(v) for v in block[4:16]]
    if j < 4:
        sc = s[j] % 64
        m = s[4 + j] % 64
    else:
        sc = (s[4 + j] % 16) + 16 * (s[j - 4] // 64)
        m = (s[4 + j] // 16) + 16 * (s[j] // 64)
    return sc, m


def q4k_code(block: np.ndarray, e: int) -> int:
    j, l = divmod(e, 32)
    byte = int(block[16 + 32 * (j // 2) + l])
    return byte % 16 if j % 2 == 0 else byte // 16


def q4k_weight(block: np.ndarray, e: int) -> float:
    d = f16(int(block[0]), int(block[1]))
    dmin = f16(int(block[2]), int(block[3]))
    code = q4k_code(block, e)
    sc, m = q4k_field(block, e // 32)
    return d * sc * code - dmin * m


def q6k_code(block: np.ndarray, e: int) -> int:
    h, r = divmod(e, 128)
    quad, l = divmod(r, 32)
    low_byte = int(block[64 * h + 32 * (quad % 2) + l])
    low = low_byte % 16 if quad < 2 else low_byte // 16
    high = (int(block[128 + 32 * h + l]) >> (2 * quad)) & 3
    return low + 16 * high


def q6k_weight(block: np.ndarray, e: int) -> float:
    d = f16(int(block[208]), int(block[209]))
    sc = int(np.int8(np.uint8(block[192 + e // 16])))
    return d * sc * (q6k_code(block, e) - 32)


def dequant(qtype: int, W: np.ndarray, od: int, idim: int) -> np.ndarray:
    """[od][idim] f64 dequantized weights."""
    bb = {1: 144, 2: 210, 6: 176}[qtype]
    nsb = idim // 256
    blocks = W.reshape(od, nsb, bb)
    f = {1: q4k_weight, 2: q6k_weight, 6: q5k_weight}[qtype]
    out = np.empty((od, idim), np.float64)
    for r in range(od):
        for b in range(nsb):
            for e in range(256):
                out[r, 256 * b + e] = f(blocks[r, b], e)
    return out


def min_term_mag(W: np.ndarray, s: np.ndarray, od: int, idim: int) -> np.ndarray:
    """[nt][od] sum over sub-blocks of |dmin*m| * |s| (Q4_K only)."""
    nsb = idim // 256
    blocks = W.reshape(od, nsb, 144)
    nt = s.shape[0]
    out = np.zeros((nt, od), np.float64)
    for r in range(od):
        for b in range(nsb):
            dmin = f16(int(blocks[r, b, 2]), int(blocks[r, b, 3]))
            for j in range(8):
                _, m = q4k_field(blocks[r, b], j)
                out[:, r] += abs(dmin * m) * np.abs(s[:, 8 * b + j].astype(np.float64))
    return out


def group_dots(qtype: int, W: np.ndarray, q: np.ndarray, od: int, idim: int) -> np.ndarray:
    """[nt][od][nsb][groups] integer dots, one element at a time."""
    nsb = idim // 256
    bb = 144 if qtype == 1 else 210
    gs = 32 if qtype == 1 else 16
    blocks = W.reshape(od, nsb, bb)
    nt = q.shape[0]
    out = np.zeros((nt, od, nsb, 256 // gs), np.int64)
    for r in range(od):
        for b in range(nsb):
            if qtype == 1:
                codes = np.array([q4k_code(blocks[r, b], e) for e in range(256)], np.int64)
            else:
                codes = np.array([q6k_code(blocks[r, b], e) - 32 for e in range(256)], np.int64)
            for t in range(nt):
                prod = codes * q[t, 256 * b:256 * (b + 1)].astype(np.int64)
                out[t, r, b] = prod.reshape(-1, gs).sum(axis=1)
    return out


def b32_code(qtype: int, group: np.ndarray, e: int) -> int:
    """Centred code of weight e of a group of eight Q4_0 / Q8_0 blocks (nibble - 8, or the int8)."""
    j, l = divmod(e, 32)
    if qtype == 4:
        byte = int(group[18 * j + 2 + (l % 16)])
        return (byte % 16 if l < 16 else byte // 16) - 8
    return int(np.int8(np.uint8(group[34 * j + 2 + l])))


def b32_weight(qtype: int, group: np.ndarray, e: int) -> float:
    """Weight e (0..255) of a group of eight Q4_0 / Q8_0 blocks, from the byte rules:
    Q4_0 block = f16 d, 16 bytes; byte l low nibble = element l, high = element l+16;
    w = d (nibble - 8).  Q8_0 block = f16 d, 32 int8; w = d q."""
    j, l = divmod(e, 32)
    if qtype == 4:
        b = group[18 * j: 18 * j + 18]
        d = f16(int(b[0]), int(b[1]))
        byte = int(b[2 + (l % 16)])
        nib = byte % 16 if l < 16 else byte // 16
        return d * (nib - 8)
    b = group[34 * j: 34 * j + 34]
    d = f16(int(b[0]), int(b[1]))
    return d * int(np.int8(np.uint8(b[2 + l])))


def b32_dequant(qtype: int, W: np.ndarray, od: int, idim: int) -> np.ndarray:
    gb = 144 if qtype == 4 else 272
    G = np.ascontiguousarray(W, dtype=np.uint8).reshape(od, idim // 256, gb)
    out = np.empty((od, idim), np.float64)
    for r in range(od):
        for g in range(idim // 256):
            for e in range(256):
                out[r, 256 * g + e] = b32_weight(qtype, G[r, g], e)
    return out


def q5k_code(block: np.ndarray, e: int) -> int:
    """Q5_K code of element e: the Q4_K-arranged low nibble of bytes 48.. plus 16 *
    bit j of high-bit byte 16 + l (e = 32 j + l)."""
    j, l = divmod(e, 32)
    byte = int(block[48 + 32 * (j // 2) + l])
    lo = byte % 16 if j % 2 == 0 else byte // 16
    return lo + 16 * ((int(block[16 + l]) >> j) & 1)


def q5k_weight(block: np.ndarray, e: int) -> float:
    d = f16(int(block[0]), int(block[1]))
    dmin = f16(int(block[2]), int(block[3]))
    sc, m = q4k_field(block, e // 32)
    return d * sc * q5k_code(block, e) - dmin * m
