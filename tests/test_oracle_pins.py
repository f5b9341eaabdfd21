"""Pins for the CPU oracle: it is checked against what the pages and plain
mathematics fix, never against itself.

Pages (by title): "The quantized GEMM" (mojo-dllm kernels page) -- The GPU path;
"llama.cpp MMQ -- quantized-weight int8 tensor-core matmul" -- sections 4, 6, 11.4.

What each pin catches:
* hand-worked scale/min unpack (golden) and the bit-budget property of the
  12-byte packing: index mistakes in the 6-bit unpack, a swapped scale/min;
* designed code-byte pattern: swapped nibble halves, wrong chunk index;
* crafted quantizer blocks (golden): rounding mode, scale constant, s = d*sum(q);
* quantizer invariants: the max element, sign symmetry, power-of-two scaling,
  the rounding error bound;
* element-indexed brute force (tests/bruteforce.py) for the integer dots and
  for the fold identity sum w x = d*sc*dx*sum(q*qx) - dmin*m*s;
* the activation-quantization error bound against the f64 dequantized matmul;
* special cases: Q6_K codes all 32 give exactly 0; one-hot activations read
  single weights through the whole path;
* planted mistakes (OQ_MUTATE builds) must fail at least one pin.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q4, Q6 = oracle.TYPE_Q4_K, oracle.TYPE_Q6_K


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            rows[k.strip()] = v.split()
    return rows


# ---------------------------------------------------------------- pin checks
# Each returns None when the pin holds, else a message.  The test functions
# assert them; the planted-mistake test counts how many fail.

def pin_q4k_scales_golden():
    g = _read_golden("q4k_scales_worked.txt")
    blk = np.zeros(144, np.uint8)
    blk[4:16] = [int(b, 16) for b in g["bytes"]]
    dec = oracle.decode_block(Q4, blk)
    want_sc = [int(v) for v in g["sc"]]
    want_m = [int(v) for v in g["m"]]
    if list(dec["sc"]) != want_sc or list(dec["m"]) != want_m:
        return f"scale/min unpack {list(dec['sc'])} {list(dec['m'])} != {want_sc} {want_m}"
    return None


def _designed_q4k_block(d_bits=0x3C00, dmin_bits=0x0000):
    """A block whose codes follow a known pattern: in code chunk p, byte l has low
    nibble (l + p) % 16 (sub-block 2p) and high nibble (3l + p) % 16 (sub-block 2p+1)."""
    blk = np.zeros(144, np.uint8)
    blk[0], blk[1] = d_bits & 0xFF, d_bits >> 8
    blk[2], blk[3] = dmin_bits & 0xFF, dmin_bits >> 8
    for p in range(4):
        for l in range(32):
            lo, hi = (l + p) % 16, (3 * l + p) % 16
            blk[16 + 32 * p + l] = (hi << 4) | lo
    return blk


def _designed_codes():
    codes = []
    for e in range(256):
        j, l = divmod(e, 32)
        p = j // 2
        codes.append((l + p) % 16 if j % 2 == 0 else (3 * l + p) % 16)
    return codes


def pin_q4k_nibble_pattern():
    dec = oracle.decode_block(Q4, _designed_q4k_block())
    if list(dec["codes"]) != _designed_codes():
        return "code map differs from the designed nibble pattern"
    return None


def _identity_case(qtype, od, idim, nt, seed):
    """O6(i): oracle output vs f64 W_deq . x_deq, x_deq = d*q exactly."""
    W = synth.weights(qtype, od, idim, seed=seed)
    x = synth.activations(nt, idim, seed=seed, outlier_frac=0.05)
    out, mag, (q, d, s) = oracle.matmul(qtype, W, x, od)
    Wd = bf.dequant(qtype, W, od, idim)
    xd = np.repeat(d.astype(np.float64), 32, axis=1) * q.astype(np.float64)
    ref = xd @ Wd.T
    bound = 2.0 ** -24 * np.abs(out) + 1e-12 * mag
    if qtype == Q4:
        bound = bound + 2.0 ** -24 * bf.min_term_mag(W, s, od, idim)
    err = np.abs(out.astype(np.float64) - ref)
    return err, bound, out, ref, (W, x, q, d, s, Wd)


def pin_identity(qtype, seeds=(1, 2)):
    for seed in seeds:
        err, bound, *_ = _identity_case(qtype, 5, 512, 3, seed)
        if not np.all(err <= bound):
            k = np.argmax(err - bound)
            return f"identity fails: err {err.flat[k]:.3e} > bound {bound.flat[k]:.3e}"
    return None


def pin_q6k_code32_zero():
    W = synth.weights(Q6, 4, 512, seed=3).reshape(-1, 210).copy()
    W[:, 0:128] = 0x00          # low nibbles 0
    W[:, 128:192] = 0xAA        # every 2-bit high field = 2, so every code is 32
    x = synth.activations(2, 512, seed=3)
    out, _, _ = oracle.matmul(Q6, W.reshape(-1), x, 4)
    if not np.all(out == 0.0):
        return "codes all 32 must give an exactly zero output"
    return None


ALL_PINS = [pin_q4k_scales_golden, pin_q4k_nibble_pattern, lambda: pin_identity(Q4),
            lambda: pin_identity(Q6), pin_q6k_code32_zero]


# ---------------------------------------------------------------- tests

def test_f16_fields_match_numpy():
    bits = np.concatenate([np.arange(0, 0x7C00, 7, dtype=np.uint32),
                           np.arange(0x8000, 0xFC00, 11, dtype=np.uint32),
                           np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x8001], np.uint32)])
    blk = np.zeros(144, np.uint8)
    for b, b2 in zip(bits, bits[::-1]):
        blk[0], blk[1] = b & 0xFF, b >> 8
        blk[2], blk[3] = b2 & 0xFF, b2 >> 8
        dec = oracle.decode_block(Q4, blk)
        want = float(np.array([b], np.uint16).view(np.float16)[0])
        want2 = float(np.array([b2], np.uint16).view(np.float16)[0])
        assert dec["d"] == want and dec["dmin"] == want2


def test_q4k_scales_worked_example():
    assert pin_q4k_scales_golden() is None


def test_q4k_scale_packing_uses_each_bit_once():
    """The 12 scale bytes carry 16 six-bit fields = 96 bits: flipping any one input
    bit must change exactly one field by exactly one power of two, and distinct
    input bits must land on distinct (field, bit) places."""
    rng = np.random.default_rng(7)
    for trial in range(8):
        base = np.zeros(144, np.uint8)
        base[4:16] = rng.integers(0, 256, 12)
        d0 = oracle.decode_block(Q4, base)
        v0 = np.concatenate([d0["sc"], d0["m"]])
        seen = set()
        for byte in range(12):
            for bit in range(8):
                blk = base.copy()
                blk[4 + byte] ^= 1 << bit
                d1 = oracle.decode_block(Q4, blk)
                v1 = np.concatenate([d1["sc"], d1["m"]])
                diff = np.nonzero(v1 != v0)[0]
                assert diff.size == 1, (byte, bit, diff)
                delta = abs(int(v1[diff[0]]) - int(v0[diff[0]]))
                assert delta & (delta - 1) == 0 and delta < 64
                seen.add((int(diff[0]), delta))
        assert len(seen) == 96


def test_q4k_nibble_pattern():
    assert pin_q4k_nibble_pattern() is None


def test_q4k_header_fields():
    blk = _designed_q4k_block(d_bits=0x4200, dmin_bits=0xB800)  # 3.0, -0.5
    dec = oracle.decode_block(Q4, blk)
    assert dec["d"] == 3.0 and dec["dmin"] == -0.5


def test_q6k_reading_r1_designed_block():
    """Reading R1 (the element-to-bit map the pages leave open; parity unpinned by
    the pages): low byte 64h+32c+l holds c in its low nibble and c+2 in its high
    nibble, and every high 2-bit field of half h is h, so every element's code is
    its quarter index within the half plus 16*h."""
    blk = np.zeros(210, np.uint8)
    for h in range(2):
        for c in range(2):
            for l in range(32):
                blk[64 * h + 32 * c + l] = (((2 + c) % 4) << 4) | c   # quarter c low, c+2 high
        for l in range(32):
            # high 2-bit fields: quarter k gets value h (so code = quarter + 16*h)
            blk[128 + 32 * h + l] = h * 0b01010101
    blk[192:208] = np.arange(16, dtype=np.int8).view(np.uint8) - 8
    blk[208], blk[209] = 0x00, 0x3C
    dec = oracle.decode_block(Q6, blk)
    want = [(e % 128) // 32 + 16 * (e // 128) for e in range(256)]
    assert list(dec["codes"]) == want
    assert list(dec["sc"]) == list(range(-8, 8))
    assert dec["d"] == 1.0
    # and the brute-force helper agrees on the same reading
    assert [bf.q6k_code(blk, e) for e in range(256)] == want


def test_quantize_golden_ties():
    g = _read_golden("quantize_ties.txt")
    for name in ("A", "B", "C"):
        x = np.array([float(v) for v in g[f"{name}.x"]], np.float32).reshape(1, 32)
        q, d, s = oracle.quantize(x)
        assert list(q[0]) == [int(v) for v in g[f"{name}.q"]], name
        assert d[0, 0] == np.float32(float(g[f"{name}.d"][0]))
        assert s[0, 0] == np.float32(float(g[f"{name}.s"][0]))


@pytest.mark.parametrize("seed,scale,outliers", [(0, 1.0, 0.0), (1, 1e-30, 0.0), (2, 3e4, 0.01), (3, 1.0, 0.05)])
def test_quantize_invariants(seed, scale, outliers):
    x = (synth.activations(4, 1024, seed=seed, outlier_frac=outliers) * np.float32(scale)).astype(np.float32)
    q, d, s = oracle.quantize(x)
    xb = x.reshape(4, 32, 32)
    qb = q.reshape(4, 32, 32).astype(np.int32)
    # the largest magnitude maps to +-127 exactly
    k = np.argmax(np.abs(xb), axis=2)
    qmax = np.take_along_axis(qb, k[..., None], axis=2)[..., 0]
    xmax = np.take_along_axis(xb, k[..., None], axis=2)[..., 0]
    assert np.all(qmax == np.where(xmax > 0, 127, -127))
    assert np.all(np.abs(qb) <= 127)
    # rounding error bound: |x - d q| <= d (1/2 + 2^-17)
    err = np.abs(xb.astype(np.float64) - d.reshape(4, 32, 1).astype(np.float64) * qb)
    assert np.all(err <= d.reshape(4, 32, 1).astype(np.float64) * (0.5 + 2.0 ** -17))
    # s is one f32 product of d and the integer code sum
    assert np.array_equal(s, (d * qb.sum(axis=2).astype(np.float32)).astype(np.float32))
    # sign symmetry
    qn, dn, sn = oracle.quantize(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d) and np.array_equal(sn, -s)
    # power-of-two equivariance (stays in the normal range)
    q2, d2, s2 = oracle.quantize((x * np.float32(2.0 ** -3)).astype(np.float32))
    if scale >= 1.0:
        assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(0.125)) and \
            np.array_equal(s2, s * np.float32(0.125))


@pytest.mark.parametrize("qtype", [Q4, Q6])
def test_group_dots_brute_force(qtype):
    od, idim, nt = 3, 512, 2
    W = synth.weights(qtype, od, idim, seed=11)
    x = synth.activations(nt, idim, seed=11)
    q, _, _ = oracle.quantize(x)
    S = oracle.subblock_dots(qtype, W, q, od)
    assert np.array_equal(S.astype(np.int64), bf.group_dots(qtype, W, q, od, idim))


@pytest.mark.parametrize("qtype", [Q4, Q6])
def test_fold_identity(qtype):
    assert pin_identity(qtype, seeds=(1, 2, 3)) is None


@pytest.mark.parametrize("qtype", [Q4, Q6])
def test_activation_quantization_bound(qtype):
    """|out - W_deq . x| <= sum_k d_k (1/2 + 2^-17) sum_{i in k} |w_i| + identity bound."""
    err, bound, out, ref, (W, x, q, d, s, Wd) = _identity_case(qtype, 5, 512, 3, 4)
    exact = x.astype(np.float64) @ Wd.T
    nt, idim = x.shape
    absW = np.abs(Wd).reshape(Wd.shape[0], idim // 32, 32).sum(axis=2)  # [od][blocks]
    act = (d.astype(np.float64) * (0.5 + 2.0 ** -17)) @ absW.T
    tot_err = np.abs(out.astype(np.float64) - exact)
    assert np.all(tot_err <= act + bound)
    ratio = float(np.max(tot_err / (act + bound)))
    assert ratio < 1.0


def test_q6k_codes_32_give_zero():
    assert pin_q6k_code32_zero() is None


def test_one_hot_reads_single_weights():
    """x = e_i reads weight w[r][i] through quantize + dots + fold: the block holding
    i quantizes to code 127 with d = fl(1/127), so out = w * (127 * fl(1/127)) up to
    one rounding of s."""
    od, idim = 3, 512
    blocks = []
    for r in range(od):
        for b in range(2):
            blk = _designed_q4k_block(d_bits=0x3C00 + 0x400 * r, dmin_bits=0x3800)  # d = 1, 2, 4; dmin 0.5
            blk[4:8] = 1 + b        # sc_j = 1 + b for j < 4
            blk[8:12] = 2           # m_j = 2 for j < 4
            blk[12:16] = 0x31 + b   # sc_j = 1 + b, m_j = 3 for j >= 4
            blocks.append(blk)
    W = np.stack(blocks).reshape(-1)
    codes = _designed_codes()
    for i in (0, 37, 255, 256, 300, 511):
        x = np.zeros((1, idim), np.float32)
        x[0, i] = 1.0
        out, _, (q, d, s) = oracle.matmul(Q4, W, x, od)
        b, e = divmod(i, 256)
        j = e // 32
        sc = 1 + b
        m = 2 if j < 4 else 3
        for r in range(od):
            w = (2.0 ** r) * sc * codes[e] - 0.5 * m
            want = w * (127.0 * float(np.float32(1.0) / np.float32(127.0)))
            assert abs(float(out[0, r]) - want) <= 2.0 ** -22 * (abs((2.0 ** r) * sc * codes[e]) + 0.5 * m) + 1e-30


def test_points_match_full():
    od, idim, nt = 7, 768, 3
    for qtype in (Q4, Q6):
        W = synth.weights(qtype, od, idim, seed=5)
        x = synth.activations(nt, idim, seed=5)
        out, mag, (q, d, s) = oracle.matmul(qtype, W, x, od)
        t = np.array([0, 2, 1, 2], np.int32)
        r = np.array([6, 0, 3, 5], np.int32)
        po, pm = oracle.matmul_q8_points(qtype, W, q, d, s, od, t, r)
        assert np.array_equal(po, out[t, r]) and np.array_equal(pm, mag[t, r])


def test_oracle_threads_do_not_change_results():
    od, idim, nt = 16, 512, 3
    W = synth.weights(Q4, od, idim, seed=6)
    x = synth.activations(nt, idim, seed=6)
    n0 = oracle.num_threads()
    oracle.set_num_threads(1)
    a, _, _ = oracle.matmul(Q4, W, x, od)
    oracle.set_num_threads(max(n0, 2))
    b, _, _ = oracle.matmul(Q4, W, x, od)
    oracle.set_num_threads(n0)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mutation", [1, 2, 3, 4, 5])
def test_planted_mistakes_are_caught(mutation, tmp_path):
    """Each planted mistake (swapped nibble halves, Q6_K offset dropped, min term
    dropped, scale/min swapped, Q6_K scale per 32) must fail at least one pin."""
    path = oracle.build(out=str(tmp_path / f"liboracle_m{mutation}.so"), mutate=mutation)
    with oracle.use(path):
        failures = [m for m in (p() for p in ALL_PINS) if m is not None]
    assert failures, f"mutation {mutation} passed every pin"
    # and the real oracle passes all of them
    assert all(p() is None for p in ALL_PINS)


def _pad_q6k(W, fill):
    """210-byte Q6_K blocks to 224-byte blocks, the 14 pad bytes set to `fill`."""
    b = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1, 210)
    out = np.full((b.shape[0], 224), fill, np.uint8)
    out[:, :210] = b
    return out.reshape(-1)


def test_q6k_padded_blocks_equal_unpadded():
    """Q6_K with blocks padded to 224 bytes ("The quantized GEMM", The GPU path:
    the upload pads each Q6_K block so every 16-byte piece is aligned) is the same
    matrix: every oracle entry point gives identical results, whatever the pad
    bytes hold (a wrong block stride or a pad read as data changes them)."""
    od, idim, nt = 5, 768, 3
    W = synth.weights(Q6, od, idim, seed=61)
    Wp = _pad_q6k(W, 0xA7)
    P6 = oracle.TYPE_Q6_K_P224
    x = synth.activations(nt, idim, seed=62, outlier_frac=0.02)
    o, m, (q, d, s) = oracle.matmul(Q6, W, x, od)
    op, mp, _ = oracle.matmul(P6, Wp, x, od)
    assert np.array_equal(o, op) and np.array_equal(m, mp)
    assert np.array_equal(oracle.subblock_dots(Q6, W, q, od), oracle.subblock_dots(P6, Wp, q, od))
    q8, d8, b8 = oracle.quantize_q8k(x)
    assert np.array_equal(oracle.matmul_q8k(Q6, W, q8, d8, b8, od)[0], oracle.matmul_q8k(P6, Wp, q8, d8, b8, od)[0])
    t = np.array([0, 2], np.int32)
    r = np.array([4, 1], np.int32)
    assert np.array_equal(oracle.matmul_q8_points(P6, Wp, q, d, s, od, t, r)[0], o[t, r])
    dec = oracle.decode_block(P6, Wp[224:448])
    ref = oracle.decode_block(Q6, W[210:420])
    assert dec["d"] == ref["d"] and np.array_equal(dec["codes"], ref["codes"]) and np.array_equal(dec["sc"], ref["sc"])
