"""Vectorised f64 dequantizer of every weight layout (test helper).

The same byte rules as tests/bruteforce.py, applied to whole arrays of blocks at
once so that rows of full-size matrices can be dequantized in seconds; a CPU test
checks it against the element-by-element decoder on random blocks.  Written from
the byte layouts, independently of the oracle and of the kernels:

* Q4_K ("The quantized GEMM", "The GPU path"; "llama.cpp MMQ ...", section 6):
  f16 d, f16 dmin, 12 bytes of packed 6-bit (scale, min) pairs, 128 code bytes;
  32-byte chunk p holds sub-block 2p in its low nibbles and 2p+1 in its high
  nibbles; w = d*sc*q - dmin*m.
* Q6_K ("The quantized GEMM", "Q6_K: the same layout and prefetch"): 128 bytes of
  low nibbles, 64 of high 2-bit fields, 16 int8 scales, f16 d; the element map
  inside the two planes is the public GGUF arrangement (a reading the pages leave
  open); w = d*sc*(q6 - 32); padded blocks (224 bytes) carry the same first 210.
* Q5_K: Q4_K's header, 32 bytes of fifth bits, Q4_K-arranged low nibbles.
* Q4_0 / Q8_0 ("03 - Reading minfer's kernels I", section 3.2): groups of eight
  32-weight blocks, f16 d then 16 nibble bytes (w = d*(n - 8)) or 32 int8 (w = d*q).
"""
from __future__ import annotations

import numpy as np

BLOCK = {1: 144, 2: 210, 3: 224, 4: 144, 5: 272, 6: 176}


def _f16(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return (lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)).view(np.float16).astype(np.float64)


def _q4k_scales(s12: np.ndarray):
    """(sc, m) [..., 8] from the 12 packed bytes [..., 12]."""
    s = s12.astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), np.int64)
    m = np.empty_like(sc)
    sc[..., :4] = s[..., 0:4] & 63
    m[..., :4] = s[..., 4:8] & 63
    sc[..., 4:] = (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)
    m[..., 4:] = (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)
    return sc, m


def _q4k_codes(qs: np.ndarray) -> np.ndarray:
    """[..., 256] codes from the 128 code bytes [..., 128]."""
    c = qs.astype(np.int64).reshape(qs.shape[:-1] + (4, 32))
    return np.stack([c & 15, c >> 4], axis=-2).reshape(qs.shape[:-1] + (256,))


def q6k_codes(blocks: np.ndarray) -> np.ndarray:
    """[..., 256] 6-bit codes (0..63) of Q6_K blocks [..., >= 210]."""
    ql = blocks[..., 0:128].astype(np.int64).reshape(blocks.shape[:-1] + (2, 2, 32))   # [h][jq][l]
    qh = blocks[..., 128:192].astype(np.int64).reshape(blocks.shape[:-1] + (2, 32))    # [h][l]
    out = np.empty(blocks.shape[:-1] + (2, 4, 32), np.int64)                           # [h][quad][l]
    for quad in range(4):
        low = ql[..., quad % 2, :]
        low = low & 15 if quad < 2 else low >> 4
        out[..., quad, :] = low | (((qh >> (2 * quad)) & 3) << 4)
    return out.reshape(blocks.shape[:-1] + (256,))


def dequant_blocks(qtype: int, blocks: np.ndarray):
    """(w [..., 256] f64, min [..., 8] f64 or None) of super-blocks / groups [..., BLOCK]:
    min[j] = the value 32-weight block j subtracts from its scaled codes: dmin*m_j
    (Q4_K, Q5_K) or 8*d_j (Q4_0); None where nothing is subtracted (Q6_K, Q8_0)."""
    blocks = np.asarray(blocks, np.uint8)
    if qtype in (1, 6):
        d = _f16(blocks[..., 0], blocks[..., 1])[..., None]
        dmin = _f16(blocks[..., 2], blocks[..., 3])[..., None]
        sc, m = _q4k_scales(blocks[..., 4:16])
        if qtype == 1:
            codes = _q4k_codes(blocks[..., 16:144])
        else:
            hb = blocks[..., 16:48].astype(np.int64)                      # byte l, bit j
            high = np.stack([(hb >> j) & 1 for j in range(8)], axis=-2)   # [..., j, l]
            codes = _q4k_codes(blocks[..., 48:176]) + 16 * high.reshape(blocks.shape[:-1] + (256,))
        scale = np.repeat(d * sc, 32, axis=-1)
        mins = dmin * m
        return scale * codes - np.repeat(mins, 32, axis=-1), mins
    if qtype in (2, 3):
        d = _f16(blocks[..., 208], blocks[..., 209])[..., None]
        sc = blocks[..., 192:208].view(np.int8).astype(np.int64)
        return np.repeat(d * sc, 16, axis=-1) * (q6k_codes(blocks) - 32), None
    if qtype == 4:
        g = blocks.reshape(blocks.shape[:-1] + (8, 18))
        d = _f16(g[..., 0], g[..., 1])[..., None]
        b = g[..., 2:18].astype(np.int64)
        n = np.concatenate([b & 15, b >> 4], axis=-1)                    # elements 0..15, 16..31
        return (d * (n - 8)).reshape(blocks.shape[:-1] + (256,)), 8.0 * d[..., 0]
    if qtype == 5:
        g = blocks.reshape(blocks.shape[:-1] + (8, 34))
        d = _f16(g[..., 0], g[..., 1])[..., None]
        q = g[..., 2:34].view(np.int8).astype(np.int64)
        return (d * q).reshape(blocks.shape[:-1] + (256,)), None
    raise ValueError(f"unknown weight type {qtype}")


def dequant_rows(qtype: int, W: np.ndarray, od: int, idim: int, rows=None):
    """(W_deq [len(rows)][idim] f64, mins [len(rows)][idim/32] f64 or None) of the given
    rows (all rows when rows is None)."""
    nsb = idim // 256
    B = np.asarray(W, np.uint8).reshape(od, nsb, BLOCK[qtype])
    if rows is not None:
        B = B[np.asarray(rows)]
    w, mins = dequant_blocks(qtype, B)
    n = B.shape[0]
    return w.reshape(n, idim), (None if mins is None else mins.reshape(n, nsb * 8))
