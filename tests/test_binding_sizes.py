"""The Python binding refuses tensors too small for the call before anything reaches
the library (no GPU needed).

The C ABI takes pointers and sizes only, so it cannot tell an undersized buffer from
a large one; a wrong weight type or a short output would let a kernel read or write
past an allocation.  The binding checks every buffer against the call's shape first.
Here the tensors are meta tensors dressed up as device tensors: a correctly sized
call gets past the size checks and is refused by the library itself (null pointers
or no gfx950 device here), an undersized one raises ValueError before it.
"""
from __future__ import annotations

import pytest
import torch

import quantized_matmul_amd as qmm


class _Dev(torch.Tensor):
    @property
    def is_cuda(self):
        return True


def dev(shape, dtype):
    return torch.Tensor._make_subclass(_Dev, torch.empty(shape, dtype=dtype, device="meta"))


@pytest.fixture(autouse=True)
def _null_stream(monkeypatch):
    """No device here: the calls get the null stream instead of torch's current one."""
    import ctypes
    monkeypatch.setattr(qmm, "_stream", lambda stream: ctypes.c_void_p(0))


def _refused_by_size(fn):
    with pytest.raises(ValueError, match="needs at least"):
        fn()


def _passes_size_checks(fn):
    with pytest.raises(qmm.QmmError):
        fn()


U8, I8, F32, I32 = torch.uint8, torch.int8, torch.float32, torch.int32
NT, OD, ID = 3, 40, 512


def OUT():
    return dev((NT, OD), F32)


def q8(nt=NT, idim=ID, nb=None):
    nb = nt * idim // 32 if nb is None else nb
    return dev((nt, idim), I8), dev((nb,), F32), dev((nb,), F32)


def q8k(nt=NT, idim=ID, nd=None, nbs=None):
    return (dev((nt, idim), I8), dev((nt * idim // 256 if nd is None else nd,), F32),
            dev((nt * idim // 16 if nbs is None else nbs,), F32))


@pytest.mark.parametrize("qtype", [1, 2, 3, 4, 5, 6])
def test_weight_size_checked(qtype):
    wb = qmm.qmm_weight_bytes(qtype, OD, ID)
    q, d, s = q8()
    _passes_size_checks(lambda: qmm.qmm_matmul_q8(qtype, dev((wb,), U8), q, d, s, OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8(qtype, dev((wb - 1,), U8), q, d, s, OD))
    _refused_by_size(lambda: qmm.qmm_matmul_q8_kind(2, qtype, dev((wb - 16,), U8), q, d, s, OD))
    _refused_by_size(lambda: qmm.qmm_matmul(qtype, dev((wb - 1,), U8), dev((NT, ID), F32), OD,
                                            workspace=dev((1 << 20,), U8)))
    _refused_by_size(lambda: qmm.qmm_group_dots(1, qtype, dev((wb - 1,), U8), q, OD))


def test_type_mismatch_caught_by_size():
    """Q4_K-sized weights passed as Q6_K (larger blocks) are refused."""
    wb4 = qmm.qmm_weight_bytes(1, OD, ID)
    q, d, s = q8()
    _refused_by_size(lambda: qmm.qmm_matmul_q8(2, dev((wb4,), U8), q, d, s, OD))


def test_activation_planes_checked():
    W = dev((qmm.qmm_weight_bytes(1, OD, ID),), U8)
    q, d, s = q8()
    short = dev((NT * ID // 32 - 1,), F32)
    _refused_by_size(lambda: qmm.qmm_matmul_q8(1, W, q, short, s, OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8(1, W, q, d, short, OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_quantize_act(dev((NT, ID), F32), q, short, s))
    _refused_by_size(lambda: qmm.qmm_quantize_act(dev((NT, ID), F32), dev((NT * ID - 1,), I8), d, s))
    _passes_size_checks(lambda: qmm.qmm_quantize_act(dev((NT, ID), F32), q=q, d=d, s=s))


def test_outputs_checked():
    W = dev((qmm.qmm_weight_bytes(1, OD, ID),), U8)
    q, d, s = q8()
    _refused_by_size(lambda: qmm.qmm_matmul_q8(1, W, q, d, s, OD, out=dev((NT * OD - 1,), F32)))
    _passes_size_checks(lambda: qmm.qmm_matmul_q8(1, W, q, d, s, OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8_kind(1, 1, W, q, d, s, OD, out=dev((NT * OD - 1,), F32)))
    _refused_by_size(lambda: qmm.qmm_matmul(1, W, dev((NT, ID), F32), OD, out=dev((NT * OD - 1,), F32),
                                            workspace=dev((1 << 20,), U8)))
    _refused_by_size(lambda: qmm.qmm_group_dots(1, 1, W, q, OD, S=dev((NT * OD * 2 * 8 - 1,), I32)))
    _refused_by_size(lambda: qmm.qmm_rmsnorm(dev((NT, ID), F32), dev((ID,), F32), 1e-5,
                                             y=dev((NT * ID - 1,), F32)))
    _refused_by_size(lambda: qmm.qmm_silu_mul(dev((NT, ID), F32), dev((NT, ID), F32),
                                              y=dev((NT * ID - 1,), F32)))
    _refused_by_size(lambda: qmm.qmm_pad_q6k(dev((210 * 4,), U8), out=dev((224 * 4 - 1,), U8)))


def test_streamk_checked():
    W = dev((qmm.qmm_weight_bytes(1, OD, ID),), U8)
    q, d, s = q8()
    ws = dev((1 << 20,), U8)
    _refused_by_size(lambda: qmm.qmm_matmul_q8_streamk(1, dev((100,), U8), q, d, s, OD, ws, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8_streamk(1, W, q, d, s, OD, ws, out=dev((1,), F32)))
    _passes_size_checks(lambda: qmm.qmm_matmul_q8_streamk(1, W, q, d, s, OD, ws, out=OUT()))


def test_q8k_planes_checked():
    W = dev((qmm.qmm_weight_bytes(1, OD, ID),), U8)
    q, d, b = q8k()
    _passes_size_checks(lambda: qmm.qmm_matmul_q8k(1, W, q, d, b, OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8k(1, W, *q8k(nd=NT * ID // 256 - 1), OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8k(1, W, *q8k(nbs=NT * ID // 16 - 1), OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_matmul_q8k_kind(2, 1, W, *q8k(nbs=1), OD, out=OUT()))
    _refused_by_size(lambda: qmm.qmm_q8k_superblock_sums(1, W, q, d, b, OD, S=dev((NT * OD * 2 * 2 - 1,), I32)))
    _refused_by_size(lambda: qmm.qmm_quantize_act_q8k(dev((NT, ID), F32), q, d, dev((1,), F32)))
    _refused_by_size(lambda: qmm.qmm_rmsnorm_quantize_q8k(dev((NT, ID), F32), dev((ID,), F32), 1e-5,
                                                          q, dev((1,), F32), b))


def test_fused_outputs_checked():
    x, w = dev((NT, ID), F32), dev((ID,), F32)
    short = dev((1,), F32)
    q, d, s = q8()
    kq, kd, kb = q8k()
    _refused_by_size(lambda: qmm.qmm_rmsnorm_quantize(x, w, 1e-5, q, d, short))
    _refused_by_size(lambda: qmm.qmm_add_rmsnorm_quantize(x, dev((NT, ID), F32), w, 1e-5, q, short, s))
    _refused_by_size(lambda: qmm.qmm_silu_mul_quantize(x, dev((NT, ID), F32), dev((5,), I8), d, s))
    _refused_by_size(lambda: qmm.qmm_silu_mul_quantize_q8k(x, dev((NT, ID), F32), kq, kd, short))
    _refused_by_size(lambda: qmm.qmm_add_rmsnorm_quantize_q8k(x, dev((NT, ID), F32), w, 1e-5, dev((5,), I8), kd, kb))
    _passes_size_checks(lambda: qmm.qmm_rmsnorm_quantize(x, w, 1e-5, q, d, s))


def test_mfma_tile_check_sizes():
    _refused_by_size(lambda: qmm.qmm_mfma_tile_check(1, dev((1023,), I8), dev((1024,), I8)))
    _refused_by_size(lambda: qmm.qmm_mfma_tile_check(2, dev((64,), F32), dev((64,), F32), C=dev((2047,), F32)))
