"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function include/qmm.h declares, sizes follow their closed forms, and argument
validation answers before any device work."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import quantized_matmul_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qmm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _declared()
    assert "qmm_matmul" in names and "qmm_quantize_act" in names
    L = qmm.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qmm.EXPORTS)


def test_weight_bytes_closed_forms():
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q4_K, 1, 256) == 144
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K, 1, 256) == 210
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q4_K, 1024, 4096) == 2_359_296
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q4_K, 12288, 4096) == 28_311_552
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K, 32000, 4096) == 107_520_000
    # "The quantized GEMM", Q6_K paragraph: 6,217,728 Q6_K blocks in the output,
    # 16 attn_v and 16 ffn_down tensors of an 8B model (vocab 126464, hidden 4096,
    # FFN 12288); 12 more bytes each is 74,612,736 bytes (74.6 MB, 71.2 MiB).
    nblk = (qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K, 126464, 4096)
            + 16 * qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K, 4096, 4096)
            + 16 * qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K, 4096, 12288)) // 210
    assert nblk == 6_217_728
    assert nblk * 12 == 74_612_736 and round(nblk * 12 / 2**20, 1) == 71.2
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q6_K_P224, 32000, 4096) == 32000 * 16 * 224
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q4_0, 12288, 4096) == 12288 * 16 * 144
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q8_0, 12288, 4096) == 12288 * 16 * 272
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q5_K, 4096, 4096) == 4096 * 16 * 176
    assert qmm.qmm_weight_bytes(7, 1, 256) == 0
    assert qmm.qmm_weight_bytes(qmm.QMM_TYPE_Q4_K, 1, 300) == 0


def test_act_bytes():
    # q8 plane then d then s, each rounded up to 256 bytes
    assert qmm.qmm_act_bytes(1, 4096) == 4096 + 2 * 512
    assert qmm.qmm_act_bytes(3, 256) == 768 + 2 * 256
    assert qmm.qmm_act_bytes(512, 12288) == 512 * 12288 + 2 * 512 * 384 * 4
    assert qmm.qmm_act_bytes(0, 256) == 0 and qmm.qmm_act_bytes(1, 33) == 0


def test_set_skinny_split_host():
    """The small-batch split setting takes 0, 1, 2, 4, 8 and 16 and refuses anything
    else before touching any state (host only)."""
    try:
        for ks in (1, 2, 4, 8, 16, 0):
            qmm.qmm_set_skinny_split(ks)
        for bad in (3, 5, 32, -1):
            with pytest.raises(qmm.QmmError):
                qmm.qmm_set_skinny_split(bad)
    finally:
        qmm.qmm_set_skinny_split(0)


def test_dispatch_kind_host():
    assert qmm.qmm_nt_switch() == 8
    Q4, Q6 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K
    # Q4_K: the small-batch kernel on 9..16 tokens of any matrix, on 3..8 tokens from
    # 3072 rows, on 5..8 tokens from 2048 rows, on 6..8 tokens from 1024 rows of at
    # most 4096 columns, on 17..32 tokens up to 12288 rows, on 33..48 tokens up to
    # 8192 rows of at most 4096 columns; MMVQ otherwise up to 8 tokens (and 9..16 when
    # the switch is moved), MMQ beyond
    def want(nt, od, idim):
        sk = ((nt <= 16 and (nt >= 9 or (nt >= 3 and od >= 3072) or (nt >= 5 and od >= 2048) or
                             (nt >= 6 and od >= 1024 and idim <= 4096))) or
              (17 <= nt <= 32 and od <= 12288) or (33 <= nt <= 48 and od <= 8192 and idim <= 4096))
        return qmm.QMM_KIND_SKINNY if sk else qmm.QMM_KIND_MMVQ if nt <= 8 else qmm.QMM_KIND_MMQ

    for nt in range(1, 65):
        for od in (64, 1023, 1024, 2048, 3072, 4096, 8192, 12288, 12544, 14336):
            for idim in (4096, 12288):
                assert qmm.qmm_dispatch_kind(Q4, nt, od, idim) == want(nt, od, idim), (nt, od, idim)
        assert qmm.qmm_dispatch_kind(Q4, 3, 3072, 3072) == qmm.QMM_KIND_SKINNY
        assert qmm.qmm_dispatch_kind(Q4, 3, 3071, 4096) == qmm.QMM_KIND_MMVQ
        assert qmm.qmm_dispatch_kind(Q4, 6, 1023, 4096) == qmm.QMM_KIND_MMVQ
        assert qmm.qmm_dispatch_kind(Q4, 6, 1024, 4352) == qmm.QMM_KIND_MMVQ
    assert qmm.qmm_dispatch_kind(Q4, 17, 4096, 4096) == qmm.QMM_KIND_SKINNY
    assert qmm.qmm_dispatch_kind(Q4, 33, 4096, 12288) == qmm.QMM_KIND_MMQ
    assert qmm.qmm_dispatch_kind(Q4, 49, 4096, 4096) == qmm.QMM_KIND_MMQ
    # other types: MMVQ up to 8 tokens; 9..16 tokens on token slices of 8 up to 4096
    # rows, MMQ above
    for nt in range(1, 9):
        assert qmm.qmm_dispatch_kind(Q6, nt, 12288, 4096) == qmm.QMM_KIND_MMVQ
    for nt in (9, 12, 16):
        assert qmm.qmm_dispatch_kind(Q6, nt, 4096, 4096) == qmm.QMM_KIND_MMVQ
        assert qmm.qmm_dispatch_kind(Q6, nt, 64, 12288) == qmm.QMM_KIND_MMVQ
        assert qmm.qmm_dispatch_kind(Q6, nt, 4097, 4096) == qmm.QMM_KIND_MMQ
    for nt in (17, 256, 512):
        assert qmm.qmm_dispatch_kind(Q6, nt, 4096, 4096) == qmm.QMM_KIND_MMQ


def test_streamk_preferred_host():
    """Stream-K for Q4_K and Q6_K MMQ calls: never for a whole number of rounds of 256
    tiles (128 x 64); above 256 tiles when the last round leaves >= 10 % of the
    workgroup slots idle; within one round for K of >= 32 super-blocks (not at 128
    tiles), or Q6_K grids of at most 64 tiles.  Never for vector-kernel or small-batch
    calls or other types."""
    Q4, Q6, P6 = qmm.QMM_TYPE_Q4_K, qmm.QMM_TYPE_Q6_K, qmm.QMM_TYPE_Q6_K_P224
    sp = qmm.qmm_streamk_preferred
    for qt in (Q4, Q6, P6):
        assert sp(qt, 33, 4096, 12288)               # 48 super-blocks, 32 tiles
        assert sp(qt, 17, 4096, 12288) == (qt != Q4)  # the same (Q4_K: small-batch slices)
        assert sp(qt, 448, 4096, 8192)                # 32 super-blocks, 224 tiles
        assert not sp(qt, 256, 4096, 12288)           # 128 tiles: the per-tile split fills one round
        assert not sp(qt, 512, 4096, 12288)           # 256 tiles: one whole round
        assert not sp(qt, 512, 12288, 4096)           # 768 tiles: three rounds
        assert sp(qt, 192, 12288, 4096)               # 288 tiles: 44 % of 512 slots idle
        assert sp(qt, 384, 14336, 4096)               # 672 tiles: 12.5 % of 768 idle
        assert not sp(qt, 128, 32000, 4096)           # 500 tiles: 2.3 % of 512 idle
        assert not sp(qt, 128, 12288, 4096)           # 192 tiles, short K
        assert not sp(qt, 8, 4096, 65536)             # vector kernel
        assert not sp(qt, 12, 4096, 65536)            # vector kernel on slices
        assert sp(qt, 12, 4097, 65536) == (qt != Q4)  # MMQ above 4096 rows (Q4_K: the small-batch kernel)
    assert not sp(Q4, 448, 4096, 7936)                # 31 super-blocks, 224 tiles
    # short K within one round: only Q6_K grids of at most 64 tiles
    assert not sp(Q4, 64, 4096, 4096) and sp(Q6, 64, 4096, 4096) and sp(P6, 128, 4096, 4096)
    assert not sp(Q6, 192, 4096, 4096)                # 96 tiles
    # Q4_K within one round of the 4-wave kernel (257-512 tiles where it runs): per tile
    assert not sp(Q4, 256, 12288, 4096) and sp(Q6, 256, 12288, 4096)   # 384 tiles, the split named
    assert not sp(Q4, 448, 8192, 4096) and sp(Q6, 448, 8192, 4096)     # 448 tiles, 128 x 64 named
    assert sp(Q4, 320, 8192, 4096)                                     # 320 tiles, the split: stream-K
    assert not sp(qmm.QMM_TYPE_Q4_0, 512, 4096, 12288)
    assert not sp(qmm.QMM_TYPE_Q5_K, 512, 4096, 12288)
    n = qmm.qmm_act_bytes(384, 12288)
    assert qmm.qmm_matmul_ws_bytes(Q4, 384, 4096, 12288) == n + qmm.qmm_streamk_ws_bytes()
    assert qmm.qmm_matmul_ws_bytes(Q6, 384, 4096, 12288) == n + qmm.qmm_streamk_ws_bytes()
    assert qmm.qmm_matmul_ws_bytes(Q4, 512, 4096, 12288) == qmm.qmm_act_bytes(512, 12288)
    with pytest.raises(qmm.QmmError):
        qmm.qmm_streamk_preferred(Q4, 512, 4096, 4000)
    with pytest.raises(qmm.QmmError):
        qmm.qmm_dispatch_kind(qmm.QMM_TYPE_Q4_K, 1, 4096, 4000)


def test_validation_before_device_work():
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
    mis = ctypes.c_void_p((1 << 20) + 4)
    big = 1 << 30
    assert L.qmm_matmul(7, p, p, 1, 4, 256, p, p, big, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul(0, p, p, 1, 4, 256, p, p, big, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul(1, None, p, 1, 4, 256, p, p, big, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul(1, p, p, 0, 4, 256, p, p, big, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul(1, p, p, 1, 4, 320, p, p, big, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_matmul(1, p, p, 1, 4, 0, p, p, big, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_matmul(1, mis, p, 1, 4, 256, p, p, big, None) == qmm.QMM_ERR_ALIGN
    assert L.qmm_matmul(1, p, p, 1, 4, 256, p, p, 10, None) == qmm.QMM_ERR_WORKSPACE
    assert L.qmm_matmul_q8(2, p, p, p, mis, 1, 4, 256, p, None) == qmm.QMM_ERR_ALIGN
    assert L.qmm_matmul_q8_kind(0, 1, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul_q8_kind(9, 1, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK, 1, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK, 2, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_TYPE
    # the 32 x 64 per-wave kernel and the small-batch kernel exist for Q4_K only; the
    # small-batch kernel takes any nt (slices of 16 tokens above 16): validation passes
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_WAVE32X64, 2, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_SKINNY, 2, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_SKINNY, 1, p, p, p, p, 17, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_SKINNY, 1, p, p, p, p, 16, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    # the MMQ tile kinds pass validation; without a GPU the device check answers
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_MMQ_64X64_SPLITK, 1, p, p, p, p, 1, 4, 256, p, None) == \
        qmm.QMM_ERR_DEVICE
    # MMVQ takes any nt (slices of 8 tokens above 8): validation passes
    assert L.qmm_matmul_q8_kind(qmm.QMM_KIND_MMVQ, 1, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    assert L.qmm_quantize_act(p, 1, 40, p, p, p, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_group_dots(qmm.QMM_KIND_MMVQ, 1, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul(1, p, p, 1 << 20, 4, 4096, p, p, big, None) == qmm.QMM_ERR_SHAPE


def test_fused_steps_validation_before_device_work():
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)
    mis = ctypes.c_void_p((1 << 20) + 8)
    E = 1e-5
    A, S, AL, D = qmm.QMM_ERR_ARG, qmm.QMM_ERR_SHAPE, qmm.QMM_ERR_ALIGN, qmm.QMM_ERR_DEVICE
    assert L.qmm_add_rmsnorm_quantize(None, p, p, E, 1, 64, p, p, p, None) == A
    assert L.qmm_add_rmsnorm_quantize(p, p, p, -1.0, 1, 64, p, p, p, None) == A
    assert L.qmm_add_rmsnorm_quantize(p, p, p, float("nan"), 1, 64, p, p, p, None) == A
    assert L.qmm_add_rmsnorm_quantize(p, p, p, float("inf"), 1, 64, p, p, p, None) == A
    assert L.qmm_add_rmsnorm_quantize(p, p, p, E, 0, 64, p, p, p, None) == A
    assert L.qmm_add_rmsnorm_quantize(p, p, p, E, 1, 48, p, p, p, None) == S
    assert L.qmm_add_rmsnorm_quantize(p, mis, p, E, 1, 64, p, p, p, None) == AL
    assert L.qmm_rmsnorm_quantize(p, p, E, 1, 0, p, p, p, None) == S
    assert L.qmm_rmsnorm_quantize(p, p, E, 1 << 16, 1 << 15, p, p, p, None) == S
    assert L.qmm_rmsnorm_quantize(p, p, E, 1, 64, p, mis, p, None) == AL
    assert L.qmm_silu_mul_quantize(p, None, 1, 64, p, p, p, None) == A
    assert L.qmm_silu_mul_quantize(p, p, 1, 16, p, p, p, None) == S
    assert L.qmm_residual_add(p, p, 0, 64, None) == A
    assert L.qmm_rmsnorm(p, p, E, 1, 64, mis, None) == AL
    assert L.qmm_silu_mul(p, p, 1, 100, p, None) == S
    # valid arguments reach the device check; eps = 0 is allowed
    import torch
    if not torch.cuda.is_available():
        assert L.qmm_add_rmsnorm_quantize(p, p, p, 0.0, 1, 64, p, p, p, None) == D
        assert L.qmm_rmsnorm_quantize(p, p, E, 3, 32, p, p, p, None) == D
        assert L.qmm_silu_mul_quantize(p, p, 1, 64, p, p, p, None) == D
        assert L.qmm_residual_add(p, p, 1, 64, None) == D
        assert L.qmm_rmsnorm(p, p, E, 1, 64, p, None) == D
        assert L.qmm_silu_mul(p, p, 1, 64, p, None) == D


def test_pad_q6k_validation():
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)
    far = ctypes.c_void_p(1 << 30)
    assert L.qmm_pad_q6k(None, p, 1, None) == qmm.QMM_ERR_ARG
    assert L.qmm_pad_q6k(far, p, 0, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_pad_q6k(far, ctypes.c_void_p((1 << 20) + 8), 1, None) == qmm.QMM_ERR_ALIGN
    assert L.qmm_pad_q6k(ctypes.c_void_p((1 << 20) + 100), p, 4, None) == qmm.QMM_ERR_ARG   # overlap
    import torch
    if not torch.cuda.is_available():
        assert L.qmm_pad_q6k(far, p, 4, None) == qmm.QMM_ERR_DEVICE
        assert L.qmm_matmul_q8(qmm.QMM_TYPE_Q6_K_P224, p, p, p, p, 1, 4, 256, p, None) == qmm.QMM_ERR_DEVICE


def test_q8k_validation():
    """qmm_matmul_q8k and its integer-stage diagnostic take Q4_K, Q5_K and Q6_K in
    both layouts (validation passes; the device check answers here) and refuse the
    32-block types and unknown types; shape, null and alignment errors come first."""
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)
    for t in (1, 2, 3, 6):
        assert L.qmm_matmul_q8k(t, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
        assert L.qmm_q8k_superblock_sums(t, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    for t in (4, 5, 7):
        assert L.qmm_matmul_q8k(t, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul_q8k(2, p, p, p, None, 9, 4, 256, p, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul_q8k(2, p, p, p, p, 9, 4, 320, p, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_matmul_q8k(3, ctypes.c_void_p((1 << 20) + 2), p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_ALIGN
    for kind in (qmm.QMM_KIND_MMQ, qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK):
        assert L.qmm_matmul_q8k_kind(kind, 2, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
    for kind in (0, qmm.QMM_KIND_MMVQ, qmm.QMM_KIND_SKINNY, 9):
        assert L.qmm_matmul_q8k_kind(kind, 2, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_ARG
    # the wave kernels with the scales in the int8 operand exist for Q4_K only
    for kind in (qmm.QMM_KIND_MMQ_WAVE32X64, qmm.QMM_KIND_MMQ_WAVE32X64_SPLITK):
        assert L.qmm_matmul_q8k_kind(kind, 1, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_DEVICE
        for t in (2, 3, 6):
            assert L.qmm_matmul_q8k_kind(kind, t, p, p, p, p, 9, 4, 256, p, None) == qmm.QMM_ERR_TYPE
    # the tile rule: fewest rounds x super-blocks per wave, ties to the larger tile
    assert qmm.qmm_q8k_tile(512, 12288, 4096) == qmm.QMM_KIND_MMQ_128X64
    assert qmm.qmm_q8k_tile(512, 4096, 12288) == qmm.QMM_KIND_MMQ_128X64
    assert qmm.qmm_q8k_tile(256, 4096, 12288) == qmm.QMM_KIND_MMQ_64X64_SPLITK
    assert qmm.qmm_q8k_tile(256, 4096, 4096) == qmm.QMM_KIND_MMQ_64X64_SPLITK
    assert qmm.qmm_q8k_tile(64, 32000, 4096) == qmm.QMM_KIND_MMQ_128X64
    with pytest.raises(qmm.QmmError):
        qmm.qmm_q8k_tile(4, 4, 300)


def test_streamk_validation():
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)
    n = qmm.qmm_streamk_ws_bytes()
    assert n == 256 * 2 * 128 * 64 * 4
    assert L.qmm_matmul_q8_streamk(1, p, p, p, p, 9, 4, 256, p, None, n, None) == qmm.QMM_ERR_ARG
    # Q4_K and Q6_K (both layouts) pass validation (the device check answers here);
    # the 32-block types and Q5_K have no stream-K kernel
    for t in (1, 2, 3):
        assert L.qmm_matmul_q8_streamk(t, p, p, p, p, 9, 4, 256, p, p, n, None) == qmm.QMM_ERR_DEVICE
    for t in (4, 5, 6):
        assert L.qmm_matmul_q8_streamk(t, p, p, p, p, 9, 4, 256, p, p, n, None) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul_q8_streamk(1, p, p, p, p, 9, 4, 256, p, p, n - 1, None) == qmm.QMM_ERR_WORKSPACE
    assert L.qmm_matmul_q8_streamk(1, p, p, p, p, 9, 4, 256, p, ctypes.c_void_p((1 << 20) + 4), n, None) == \
        qmm.QMM_ERR_ALIGN
    assert L.qmm_matmul_q8_streamk(1, p, p, p, p, 9, 4, 300, p, p, n, None) == qmm.QMM_ERR_SHAPE


def test_no_device_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = qmm.lib()
    p = ctypes.c_void_p(1 << 20)
    assert L.qmm_quantize_act(p, 1, 32, p, p, p, None) == qmm.QMM_ERR_DEVICE
    assert L.qmm_matmul(1, p, p, 1, 4, 256, p, p, 1 << 20, None) == qmm.QMM_ERR_DEVICE


def test_strerror():
    for code in range(-7, 1):
        assert qmm.strerror(code) and qmm.strerror(code) != "unknown status"
    assert qmm.strerror(-99) == "unknown status"


def test_product_does_not_import_oracle():
    import sys
    import subprocess
    code = ("import sys; import quantized_matmul_amd; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True)
    src = "".join(open(os.path.join(ROOT, "quantized_matmul_amd", f)).read()
                  for f in os.listdir(os.path.join(ROOT, "quantized_matmul_amd")) if f.endswith(".py"))
    assert "oracle" not in src.replace("no CPU path", "")


def test_mmq_tile_choice():
    """The MMQ tile shape by the cost model (rounds of workgroups x super-blocks per
    wave), on the benchmark shapes and a few small ones; invalid shapes are errors."""
    qmm = pytest.importorskip("quantized_matmul_amd")
    T128, T64, TSPLIT = qmm.QMM_KIND_MMQ_128X64, qmm.QMM_KIND_MMQ_64X64, qmm.QMM_KIND_MMQ_64X64_SPLITK
    # nt = 512: 768 / 256 tiles of 128 x 64 fill the CUs in whole rounds; ties keep the big tile
    assert qmm.qmm_mmq_tile(512, 12288, 4096) == T128
    assert qmm.qmm_mmq_tile(512, 4096, 12288) == T128
    # 256 tokens: too few 128 x 64 tiles; the split over K halves each wave's walk
    assert qmm.qmm_mmq_tile(256, 4096, 4096) == TSPLIT
    assert qmm.qmm_mmq_tile(256, 12288, 4096) == TSPLIT
    assert qmm.qmm_mmq_tile(9, 65, 512) == TSPLIT
    # one super-block: splitting K gains nothing; many tiles: the big tile
    assert qmm.qmm_mmq_tile(33, 131072, 256) == T128
    with pytest.raises(qmm.QmmError):
        qmm.qmm_mmq_tile(9, 65, 300)


def test_noalloc_rejects_calls_beyond_its_scratch():
    """qmm_matmul_noalloc refuses, before any device work, a call whose quantized
    activations exceed QMM_NOALLOC_ACT_BYTES; a call that fits gets past that check
    (and, with no gfx950 device here, stops at the device check)."""
    L = qmm.lib()
    P = ctypes.c_void_p
    fake = P(0x10000)   # non-null, aligned; never dereferenced on these paths
    nt, idim = 2048, 12288
    assert qmm.qmm_act_bytes(nt, idim) > qmm.QMM_NOALLOC_ACT_BYTES
    assert L.qmm_matmul_noalloc(1, fake, fake, nt, 64, idim, fake, None) == qmm.QMM_ERR_SCRATCH
    assert "scratch" in qmm.strerror(qmm.QMM_ERR_SCRATCH)
    assert qmm.qmm_act_bytes(512, 12288) <= qmm.QMM_NOALLOC_ACT_BYTES
    rc = L.qmm_matmul_noalloc(1, fake, fake, 512, 64, 12288, fake, None)
    assert rc != qmm.QMM_ERR_SCRATCH and rc < 0
    assert L.qmm_matmul_noalloc(1, None, fake, 1, 64, 256, fake, None) == qmm.QMM_ERR_ARG
    assert L.qmm_matmul_noalloc(1, fake, fake, 1, 64, 300, fake, None) == qmm.QMM_ERR_SHAPE
    assert L.qmm_matmul_noalloc(1, P(0x10004), fake, 1, 64, 256, fake, None) == qmm.QMM_ERR_ALIGN
