"""Seeded synthetic inputs for the quantized matmul (test and benchmark infrastructure).

This module only draws numbers.  It holds none of the matmul's arithmetic: no
super-block decoding, no scale unpacking, no activation quantization.  Both the
CPU oracle harness and the GPU harness take their inputs from here, so the two
sides see byte-identical weights and activations.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the finaliser constants are the
ones Vigna publishes for splitmix64), used as a counter-based generator: draw i
of a stream is mix(base + (i + 1) * GAMMA), so any slice of a stream can be
produced without producing what comes before it.

Block byte layouts follow the GGUF-style super-blocks the matmul consumes:

* Q4_K (144 B per 256 weights): f16 d | f16 dmin | 12 bytes of packed 6-bit
  scales and mins | 128 bytes of 4-bit codes.  The scale bytes and code bytes are
  uniform random bytes.  The 6-bit (scale, min) packing uses each of the 96 bits
  of the 12 scale bytes exactly once, so uniform bytes give 16 independent
  values uniform on {0..63}; uniform code bytes give codes uniform on {0..15}.
* Q6_K (210 B per 256 weights): 128 bytes of low 4-bit fields | 64 bytes of
  high 2-bit fields | 16 int8 group scales | f16 d.  Uniform low/high bytes give
  6-bit codes uniform on {0..63} whatever the element-to-bit map; the group
  scales are drawn uniform on {-32..31}.
* Q5_K (176 B per 256 weights): f16 d | f16 dmin | 12 scale bytes as Q4_K | 32
  bytes of high bits | 128 bytes of low nibbles, all but d and dmin uniform bytes
  (codes uniform on {0..31}).
* Q4_0 (18 B per 32 weights: f16 d | 16 bytes of 4-bit codes) and Q8_0 (34 B per
  32 weights: f16 d | 32 int8 codes), generated in groups of eight blocks (256
  weights, 144 and 272 bytes): uniform code bytes (Q8_0 codes uniform on
  {-128..127}).
* d, dmin: an f32 uniform on [1e-3, 1e-2), rounded to f16 (round to nearest even).
* Activations: f32 N(0, 1) by Box-Muller in f64, rounded to f32; optionally a
  fraction of elements multiplied by a factor (outliers).
"""
from __future__ import annotations

import numpy as np

MASK64 = np.uint64(0xFFFFFFFFFFFFFFFF)
GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
QK = 256  # weights per super-block

TYPE_Q4_K = 1
TYPE_Q6_K = 2
TYPE_Q4_0 = 4
TYPE_Q8_0 = 5
TYPE_Q5_K = 6
Q5K_BLOCK_BYTES = 176
Q40_GROUP_BYTES = 8 * 18
Q80_GROUP_BYTES = 8 * 34

# stream ids inside one seed
STREAM_W = 0
STREAM_X = 1
STREAM_OUTLIER = 2


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (finaliser) on uint64 arrays (wrapping arithmetic)."""
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def stream_base(seed: int, stream: int) -> np.uint64:
    """Starting state of stream `stream` under `seed` (a hash of the pair)."""
    s = np.array([(int(seed) * 0x100000001B3 + int(stream) * 0xD1B54A32D192ED03 + 0x632BE59BD9B4E019)
                  & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    return _mix(s)[0]


def draws(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """Draws start .. start+n-1 of one stream, as uint64."""
    base = stream_base(seed, stream)
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = base + idx * GAMMA
    return _mix(z)


def uniform01(u64: np.ndarray) -> np.ndarray:
    """Top 24 bits of each draw as a float in [0, 1) (exact in f32 and f64)."""
    return (u64 >> np.uint64(40)).astype(np.float64) * (1.0 / 16777216.0)


def _f16_field(u64: np.ndarray, lo: float = 1e-3, hi: float = 1e-2) -> np.ndarray:
    """f32 uniform on [lo, hi), rounded to f16, returned as little-endian u16 bits."""
    v = (lo + uniform01(u64) * (hi - lo)).astype(np.float32)
    return v.astype(np.float16).view(np.uint16)


def _bytes_of(u64: np.ndarray) -> np.ndarray:
    """The little-endian bytes of a [n, k] uint64 array as [n, 8k] uint8."""
    return np.ascontiguousarray(u64).view(np.uint8).reshape(u64.shape[0], -1)


def q4k_blocks(n_blocks: int, seed: int = 0, stream: int = STREAM_W, start_block: int = 0) -> np.ndarray:
    """n_blocks Q4_K super-blocks as a [n_blocks, 144] uint8 array.

    Per block, 20 draws: draw 0 gives d, draw 1 gives dmin, draws 2..19 give 144
    random bytes of which bytes 4..143 (scales and codes) are kept.
    """
    per = 20
    z = draws(seed, stream, n_blocks * per, start=start_block * per).reshape(n_blocks, per)
    out = np.empty((n_blocks, Q4K_BLOCK_BYTES), dtype=np.uint8)
    rnd = _bytes_of(z[:, 2:])  # [n, 144]
    out[:, 4:] = rnd[:, 4:]
    out[:, 0:2] = _f16_field(z[:, 0]).reshape(-1, 1).view(np.uint8).reshape(n_blocks, 2)
    out[:, 2:4] = _f16_field(z[:, 1]).reshape(-1, 1).view(np.uint8).reshape(n_blocks, 2)
    return out


def q6k_blocks(n_blocks: int, seed: int = 0, stream: int = STREAM_W, start_block: int = 0) -> np.ndarray:
    """n_blocks Q6_K super-blocks as a [n_blocks, 210] uint8 array.

    Per block, 27 draws: draw 0 gives d, draws 1..2 give 16 bytes mapped to
    int8 scales uniform on {-32..31}, draws 3..26 give the 192 code bytes.
    """
    per = 27
    z = draws(seed, stream, n_blocks * per, start=start_block * per).reshape(n_blocks, per)
    out = np.empty((n_blocks, Q6K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:192] = _bytes_of(z[:, 3:27])
    sc = (_bytes_of(z[:, 1:3]).astype(np.int16) & 63) - 32
    out[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    out[:, 208:210] = _f16_field(z[:, 0]).reshape(-1, 1).view(np.uint8).reshape(n_blocks, 2)
    return out


def q5k_blocks(n_blocks: int, seed: int = 0, stream: int = STREAM_W, start_block: int = 0) -> np.ndarray:
    """n_blocks Q5_K super-blocks as a [n_blocks, 176] uint8 array.

    Per block, 24 draws: draw 0 gives d, draw 1 gives dmin, draws 2..23 give 176
    random bytes of which bytes 4..175 (scales, high bits, codes) are kept.
    """
    per = 24
    z = draws(seed, stream, n_blocks * per, start=start_block * per).reshape(n_blocks, per)
    out = np.empty((n_blocks, Q5K_BLOCK_BYTES), dtype=np.uint8)
    out[:, 4:] = _bytes_of(z[:, 2:])[:, 4:Q5K_BLOCK_BYTES]
    out[:, 0:2] = _f16_field(z[:, 0]).reshape(-1, 1).view(np.uint8).reshape(n_blocks, 2)
    out[:, 2:4] = _f16_field(z[:, 1]).reshape(-1, 1).view(np.uint8).reshape(n_blocks, 2)
    return out


def b32_groups(qtype: int, n_groups: int, seed: int = 0, stream: int = STREAM_W, start_group: int = 0) -> np.ndarray:
    """n_groups groups of eight Q4_0 or Q8_0 blocks as a [n_groups, 144 or 272] uint8 array.

    Per group, 8 draws give the eight d, then 16 (Q4_0) or 32 (Q8_0) draws give the
    code bytes (16 or 32 per block, in block order).
    """
    cb = 16 if qtype == TYPE_Q4_0 else 32
    bb = cb + 2
    per = 8 + cb
    z = draws(seed, stream, n_groups * per, start=start_group * per).reshape(n_groups, per)
    codes = _bytes_of(z[:, 8:]).reshape(n_groups, 8, cb)
    dbits = _f16_field(z[:, :8].reshape(-1)).reshape(n_groups, 8, 1).view(np.uint8).reshape(n_groups, 8, 2)
    out = np.empty((n_groups, 8, bb), dtype=np.uint8)
    out[:, :, 0:2] = dbits
    out[:, :, 2:] = codes
    return out.reshape(n_groups, 8 * bb)


def block_bytes(qtype: int) -> int:
    """Bytes per 256 weights."""
    if qtype == TYPE_Q4_K:
        return Q4K_BLOCK_BYTES
    if qtype == TYPE_Q6_K:
        return Q6K_BLOCK_BYTES
    if qtype == TYPE_Q5_K:
        return Q5K_BLOCK_BYTES
    if qtype == TYPE_Q4_0:
        return Q40_GROUP_BYTES
    if qtype == TYPE_Q8_0:
        return Q80_GROUP_BYTES
    raise ValueError(f"unknown type {qtype}")


def weights(qtype: int, od: int, idim: int, seed: int = 0, stream: int = STREAM_W) -> np.ndarray:
    """A row-major [od][idim/256] matrix of super-blocks, as a flat uint8 array."""
    if idim % QK:
        raise ValueError("idim must be a multiple of 256")
    nb = od * (idim // QK)
    if qtype in (TYPE_Q4_0, TYPE_Q8_0):
        return b32_groups(qtype, nb, seed=seed, stream=stream).reshape(-1)
    if qtype == TYPE_Q5_K:
        return q5k_blocks(nb, seed=seed, stream=stream).reshape(-1)
    gen = q4k_blocks if qtype == TYPE_Q4_K else q6k_blocks
    return gen(nb, seed=seed, stream=stream).reshape(-1)


def normal_f32(n: int, seed: int = 0, stream: int = STREAM_X, start: int = 0) -> np.ndarray:
    """n N(0,1) values: Box-Muller (cosine branch) in f64 on two draws, rounded to f32."""
    z = draws(seed, stream, 2 * n, start=2 * start).reshape(n, 2)
    u1 = uniform01(z[:, 0])
    u2 = uniform01(z[:, 1])
    r = np.sqrt(-2.0 * np.log1p(-u1))  # 1 - u1 in (0, 1]
    return (r * np.cos(2.0 * np.pi * u2)).astype(np.float32)


def activations(nt: int, idim: int, seed: int = 0, stream: int = STREAM_X,
                outlier_frac: float = 0.0, outlier_scale: float = 20.0,
                outlier_stream: int = STREAM_OUTLIER) -> np.ndarray:
    """Token-major [nt][idim] f32 activations ~ N(0,1).

    With outlier_frac > 0, each element independently (probability outlier_frac,
    decided by its own draw of the outlier stream) is multiplied by outlier_scale.
    """
    x = normal_f32(nt * idim, seed=seed, stream=stream).reshape(nt, idim)
    if outlier_frac > 0.0:
        u = uniform01(draws(seed, outlier_stream, nt * idim)).reshape(nt, idim)
        x = np.where(u < outlier_frac, x * np.float32(outlier_scale), x).astype(np.float32)
    return x


def layer_stream(layer: int, proj: int, kind: int) -> int:
    """Stream id for one projection of one layer in a stacked model (kind: 0 = W, 1 = x)."""
    return 16 + 16 * (8 * int(layer) + int(proj)) + int(kind)
