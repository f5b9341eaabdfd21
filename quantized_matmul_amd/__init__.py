"""quantized_matmul_amd: Python binding of libqmm (the quantized-weight matmul for
MI355X / gfx950).

The binding only marshals arguments: tensors become device pointers, the current
torch stream becomes the hipStream_t, status codes become exceptions.  Every step
of the computation runs in the library's HIP kernels; there is no CPU path.
PyTorch provides device memory and streams.

Entry points mirror include/qmm.h (same names).  Weight types: QMM_TYPE_Q4_K,
QMM_TYPE_Q6_K.  Layouts: W uint8 [od * id/256 * block bytes] row-major super-blocks;
x f32 [nt, id]; q int8 [nt, id]; d, s f32 [nt, id/32]; out f32 [nt, od].
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libqmm binds to the HIP runtime torch already mapped

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

QMM_TYPE_Q4_K = 1
QMM_TYPE_Q6_K = 2
QMM_TYPE_Q6_K_P224 = 3   # Q6_K blocks padded to 224 bytes (qmm_pad_q6k)
QMM_TYPE_Q4_0 = 4        # 18-byte blocks of 32 weights
QMM_TYPE_Q8_0 = 5        # 34-byte blocks of 32 weights
QMM_TYPE_Q5_K = 6        # 176-byte super-blocks (5-bit codes)
QMM_KIND_MMVQ = 1
QMM_KIND_MMQ = 2
QMM_KIND_MMQ_128X64 = 3
QMM_KIND_MMQ_64X64 = 4
QMM_KIND_MMQ_64X64_SPLITK = 5
QMM_KIND_MMQ_WAVE32X64 = 6
QMM_KIND_MMQ_WAVE32X64_SPLITK = 8
QMM_KIND_SKINNY = 7
QMM_OK = 0
QMM_ERR_ARG = -1
QMM_ERR_TYPE = -2
QMM_ERR_SHAPE = -3
QMM_ERR_ALIGN = -4
QMM_ERR_WORKSPACE = -5
QMM_ERR_DEVICE = -6
QMM_ERR_LAUNCH = -7
QMM_ERR_SCRATCH = -8
QMM_NOALLOC_SCRATCH_BYTES = 32 << 20
QMM_NOALLOC_ACT_BYTES = 16 << 20

BLOCK_BYTES = {QMM_TYPE_Q4_K: 144, QMM_TYPE_Q6_K: 210, QMM_TYPE_Q6_K_P224: 224,  # bytes per 256 weights
               QMM_TYPE_Q4_0: 144, QMM_TYPE_Q8_0: 272, QMM_TYPE_Q5_K: 176}

EXPORTS = ("qmm_weight_bytes", "qmm_act_bytes", "qmm_quantize_act", "qmm_matmul", "qmm_matmul_q8",
           "qmm_matmul_q8_kind", "qmm_dispatch_kind", "qmm_mmq_tile", "qmm_nt_switch", "qmm_group_dots",
           "qmm_mfma_tile_check", "qmm_strerror", "qmm_add_rmsnorm_quantize", "qmm_rmsnorm_quantize",
           "qmm_silu_mul_quantize", "qmm_add_rmsnorm_quantize_q8k", "qmm_rmsnorm_quantize_q8k",
           "qmm_silu_mul_quantize_q8k", "qmm_residual_add", "qmm_rmsnorm", "qmm_silu_mul", "qmm_quantize_act_q8k",
           "qmm_matmul_q8k", "qmm_matmul_q8k_kind", "qmm_q8k_tile", "qmm_q8k_superblock_sums", "qmm_pad_q6k", "qmm_streamk_ws_bytes",
           "qmm_matmul_q8_streamk", "qmm_streamk_preferred", "qmm_matmul_noalloc", "qmm_set_skinny_split")


class QmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded libqmm (ctypes).  Raises if the library was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.qmm_weight_bytes.argtypes = [I, I, I]
        L.qmm_weight_bytes.restype = Z
        L.qmm_act_bytes.argtypes = [I, I]
        L.qmm_act_bytes.restype = Z
        L.qmm_quantize_act.argtypes = [P, I, I, P, P, P, P]
        L.qmm_matmul.argtypes = [I, P, P, I, I, I, P, P, Z, P]
        L.qmm_matmul_noalloc.argtypes = [I, P, P, I, I, I, P, P]
        L.qmm_matmul_q8.argtypes = [I, P, P, P, P, I, I, I, P, P]
        L.qmm_matmul_q8_kind.argtypes = [I, I, P, P, P, P, I, I, I, P, P]
        L.qmm_dispatch_kind.argtypes = [I, I, I, I]
        L.qmm_streamk_preferred.argtypes = [I, I, I, I]
        L.qmm_mmq_tile.argtypes = [I, I, I]
        L.qmm_nt_switch.argtypes = []
        L.qmm_set_skinny_split.argtypes = [I]
        L.qmm_group_dots.argtypes = [I, I, P, P, I, I, I, P, P]
        L.qmm_mfma_tile_check.argtypes = [I, P, P, P, P]
        F = ctypes.c_float
        L.qmm_add_rmsnorm_quantize.argtypes = [P, P, P, F, I, I, P, P, P, P]
        L.qmm_rmsnorm_quantize.argtypes = [P, P, F, I, I, P, P, P, P]
        L.qmm_silu_mul_quantize.argtypes = [P, P, I, I, P, P, P, P]
        L.qmm_add_rmsnorm_quantize_q8k.argtypes = [P, P, P, F, I, I, P, P, P, P]
        L.qmm_rmsnorm_quantize_q8k.argtypes = [P, P, F, I, I, P, P, P, P]
        L.qmm_silu_mul_quantize_q8k.argtypes = [P, P, I, I, P, P, P, P]
        L.qmm_residual_add.argtypes = [P, P, I, I, P]
        L.qmm_rmsnorm.argtypes = [P, P, F, I, I, P, P]
        L.qmm_silu_mul.argtypes = [P, P, I, I, P, P]
        L.qmm_quantize_act_q8k.argtypes = [P, I, I, P, P, P, P]
        L.qmm_matmul_q8k.argtypes = [I, P, P, P, P, I, I, I, P, P]
        L.qmm_matmul_q8k_kind.argtypes = [I, I, P, P, P, P, I, I, I, P, P]
        L.qmm_q8k_tile.argtypes = [I, I, I]
        L.qmm_q8k_superblock_sums.argtypes = [I, P, P, P, P, I, I, I, P, P]
        L.qmm_pad_q6k.argtypes = [P, P, ctypes.c_longlong, P]
        L.qmm_streamk_ws_bytes.argtypes = []
        L.qmm_streamk_ws_bytes.restype = Z
        L.qmm_matmul_q8_streamk.argtypes = [I, P, P, P, P, I, I, I, P, P, Z, P]
        L.qmm_strerror.argtypes = [I]
        L.qmm_strerror.restype = ctypes.c_char_p
        for f in ("qmm_quantize_act", "qmm_matmul", "qmm_matmul_noalloc", "qmm_matmul_q8", "qmm_matmul_q8_kind",
                  "qmm_dispatch_kind", "qmm_mmq_tile", "qmm_nt_switch", "qmm_group_dots", "qmm_mfma_tile_check",
                  "qmm_add_rmsnorm_quantize", "qmm_rmsnorm_quantize", "qmm_silu_mul_quantize",
                  "qmm_add_rmsnorm_quantize_q8k", "qmm_rmsnorm_quantize_q8k", "qmm_silu_mul_quantize_q8k",
                  "qmm_residual_add",
                  "qmm_rmsnorm", "qmm_silu_mul", "qmm_quantize_act_q8k", "qmm_matmul_q8k", "qmm_matmul_q8k_kind",
                  "qmm_q8k_tile", "qmm_q8k_superblock_sums", "qmm_pad_q6k", "qmm_matmul_q8_streamk", "qmm_streamk_preferred",
                  "qmm_set_skinny_split"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().qmm_strerror(int(status)).decode()


def _check(rc: int, what: str) -> None:
    if rc != QMM_OK:
        raise QmmError(rc, what)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t: torch.Tensor, dtype, name: str, need: int = 0) -> ctypes.c_void_p:
    """The device pointer of t, after checking its type, placement, layout and that it
    holds at least `need` elements: the library sees only pointers and sizes, so an
    undersized tensor must be refused here, before any launch."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} elements; this call needs at least {need}")
    return ctypes.c_void_p(t.data_ptr())


def _wbytes(qtype: int, od: int, idim: int) -> int:
    """Bytes W must hold (0 for an unknown type or a bad shape: the library then
    returns an error status before any launch)."""
    return qmm_weight_bytes(qtype, od, idim) if od > 0 and idim > 0 else 0


def qmm_weight_bytes(qtype: int, od: int, idim: int) -> int:
    return int(lib().qmm_weight_bytes(qtype, od, idim))


def qmm_act_bytes(nt: int, idim: int) -> int:
    return int(lib().qmm_act_bytes(nt, idim))


def qmm_nt_switch() -> int:
    return int(lib().qmm_nt_switch())


def qmm_set_skinny_split(ks: int) -> None:
    """Force the small-batch kernel's K split (1, 2, 4, 8 or 16 waves; 0 = default).
    Process-wide; the results do not depend on it (tests and tuning)."""
    _check(int(lib().qmm_set_skinny_split(ks)), "qmm_set_skinny_split")


def qmm_dispatch_kind(qtype: int, nt: int, od: int, idim: int) -> int:
    k = int(lib().qmm_dispatch_kind(qtype, nt, od, idim))
    if k < 0:
        raise QmmError(k, "qmm_dispatch_kind")
    return k


def qmm_streamk_preferred(qtype: int, nt: int, od: int, idim: int) -> bool:
    """Whether qmm_matmul runs the stream-K kernel for this call, given a workspace of
    qmm_matmul_ws_bytes()."""
    k = int(lib().qmm_streamk_preferred(qtype, nt, od, idim))
    if k < 0:
        raise QmmError(k, "qmm_streamk_preferred")
    return k == 1


def qmm_matmul_ws_bytes(qtype: int, nt: int, od: int, idim: int) -> int:
    """Workspace bytes for qmm_matmul: the q8 plane, plus the stream-K partial tiles
    where qmm_streamk_preferred."""
    n = qmm_act_bytes(nt, idim)
    return n + (qmm_streamk_ws_bytes() if qmm_streamk_preferred(qtype, nt, od, idim) else 0)


def qmm_mmq_tile(nt: int, od: int, idim: int) -> int:
    """The MMQ tile shape (a QMM_KIND_MMQ_* value) used for this shape."""
    k = int(lib().qmm_mmq_tile(nt, od, idim))
    if k < 0:
        raise QmmError(k, "qmm_mmq_tile")
    return k


def qmm_quantize_act(x: torch.Tensor, q=None, d=None, s=None, stream=None):
    """x f32 [nt, id] -> (q int8 [nt, id], d f32 [nt, id/32], s f32 [nt, id/32])."""
    nt, idim = x.shape
    if q is None:
        q = torch.empty((nt, idim), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((nt, idim // 32), dtype=torch.float32, device=x.device)
    if s is None:
        s = torch.empty((nt, idim // 32), dtype=torch.float32, device=x.device)
    nb = nt * (idim // 32)
    _check(lib().qmm_quantize_act(_dev(x, torch.float32, "x"), nt, idim, _dev(q, torch.int8, "q", nt * idim),
                                  _dev(d, torch.float32, "d", nb), _dev(s, torch.float32, "s", nb), _stream(stream)),
           "qmm_quantize_act")
    return q, d, s


def qmm_streamk_ws_bytes() -> int:
    return int(lib().qmm_streamk_ws_bytes())


def qmm_matmul_q8_streamk(qtype: int, W: torch.Tensor, q: torch.Tensor, d: torch.Tensor, s: torch.Tensor, od: int,
                          workspace: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Stream-K matrix kernel (Q4_K, Q6_K, Q6_K padded): out f32 [nt, od]; workspace uint8 >=
    qmm_streamk_ws_bytes(), any content."""
    nt, idim = q.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=q.device)
    nb = nt * (idim // 32)
    _check(lib().qmm_matmul_q8_streamk(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                       _dev(q, torch.int8, "q"), _dev(d, torch.float32, "d", nb),
                                       _dev(s, torch.float32, "s", nb), nt, od, idim,
                                       _dev(out, torch.float32, "out", nt * od),
                                       _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                       _stream(stream)), "qmm_matmul_q8_streamk")
    return out


def qmm_pad_q6k(W: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Q6_K weights (uint8, 210 bytes per block) -> the padded layout of
    QMM_TYPE_Q6_K_P224 (224 bytes per block, pad bytes zero)."""
    if W.numel() % 210:
        raise ValueError("W must hold whole 210-byte Q6_K blocks")
    nb = W.numel() // 210
    if out is None:
        out = torch.empty(nb * 224, dtype=torch.uint8, device=W.device)
    _check(lib().qmm_pad_q6k(_dev(W, torch.uint8, "W"), _dev(out, torch.uint8, "out", nb * 224), nb,
                             _stream(stream)), "qmm_pad_q6k")
    return out


def qmm_quantize_act_q8k(x: torch.Tensor, q=None, d=None, bsum=None, stream=None):
    """Q8_K activations: x f32 [nt, id] -> (q int8 [nt, id], d f32 [nt, id/256], bsum f32 [nt, id/16])."""
    nt, idim = x.shape
    if q is None:
        q = torch.empty((nt, idim), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((nt, idim // 256), dtype=torch.float32, device=x.device)
    if bsum is None:
        bsum = torch.empty((nt, idim // 16), dtype=torch.float32, device=x.device)
    _check(lib().qmm_quantize_act_q8k(_dev(x, torch.float32, "x"), nt, idim, _dev(q, torch.int8, "q", nt * idim),
                                      _dev(d, torch.float32, "d", nt * (idim // 256)),
                                      _dev(bsum, torch.float32, "bsum", nt * (idim // 16)), _stream(stream)),
           "qmm_quantize_act_q8k")
    return q, d, bsum


def qmm_matmul_q8k(qtype: int, W: torch.Tensor, q: torch.Tensor, d: torch.Tensor, bsum: torch.Tensor, od: int,
                   out=None, stream=None):
    """out f32 [nt, od] from Q8_K activations (Q4_K, Q5_K or Q6_K weights, either Q6_K layout)."""
    nt, idim = q.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=q.device)
    _check(lib().qmm_matmul_q8k(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)), _dev(q, torch.int8, "q"),
                                _dev(d, torch.float32, "d", nt * (idim // 256)),
                                _dev(bsum, torch.float32, "bsum", nt * (idim // 16)), nt, od, idim,
                                _dev(out, torch.float32, "out", nt * od), _stream(stream)), "qmm_matmul_q8k")
    return out


def qmm_matmul_q8k_kind(kind: int, qtype: int, W: torch.Tensor, q: torch.Tensor, d: torch.Tensor,
                        bsum: torch.Tensor, od: int, out=None, stream=None) -> torch.Tensor:
    """qmm_matmul_q8k with the tile shape forced (QMM_KIND_MMQ or one of QMM_KIND_MMQ_*)."""
    nt, idim = q.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=q.device)
    _check(lib().qmm_matmul_q8k_kind(kind, qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                     _dev(q, torch.int8, "q"), _dev(d, torch.float32, "d", nt * (idim // 256)),
                                     _dev(bsum, torch.float32, "bsum", nt * (idim // 16)), nt, od, idim,
                                     _dev(out, torch.float32, "out", nt * od), _stream(stream)),
           "qmm_matmul_q8k_kind")
    return out


def qmm_q8k_tile(nt: int, od: int, idim: int) -> int:
    """The tile shape (a QMM_KIND_MMQ_* value) qmm_matmul_q8k uses for this shape."""
    k = int(lib().qmm_q8k_tile(nt, od, idim))
    if k < 0:
        raise QmmError(k, "qmm_q8k_tile")
    return k


def qmm_q8k_superblock_sums(qtype: int, W: torch.Tensor, q: torch.Tensor, d: torch.Tensor, bsum: torch.Tensor,
                            od: int, S=None, stream=None):
    """Integer stage of qmm_matmul_q8k: S int32 [nt, od, id/256, 2]."""
    nt, idim = q.shape
    if S is None:
        S = torch.empty((nt, od, idim // 256, 2), dtype=torch.int32, device=q.device)
    _check(lib().qmm_q8k_superblock_sums(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                         _dev(q, torch.int8, "q"), _dev(d, torch.float32, "d", nt * (idim // 256)),
                                         _dev(bsum, torch.float32, "bsum", nt * (idim // 16)), nt, od, idim,
                                         _dev(S, torch.int32, "S", nt * od * (idim // 256) * 2), _stream(stream)),
           "qmm_q8k_superblock_sums")
    return S


def _q8_out(x: torch.Tensor, q, d, s):
    nt, idim = x.shape
    if q is None:
        q = torch.empty((nt, idim), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((nt, idim // 32), dtype=torch.float32, device=x.device)
    if s is None:
        s = torch.empty((nt, idim // 32), dtype=torch.float32, device=x.device)
    return q, d, s


def _q8_ptrs(q, d, s, nt: int, idim: int):
    nb = nt * (idim // 32)
    return (_dev(q, torch.int8, "q", nt * idim), _dev(d, torch.float32, "d", nb), _dev(s, torch.float32, "s", nb))


def _q8k_ptrs(q, d, bsum, nt: int, idim: int):
    return (_dev(q, torch.int8, "q", nt * idim), _dev(d, torch.float32, "d", nt * (idim // 256)),
            _dev(bsum, torch.float32, "bsum", nt * (idim // 16)))


def _weight_vec(w: torch.Tensor, idim: int):
    if w.dim() != 1 or w.numel() != idim:
        raise ValueError(f"w must have shape [{idim}]")


def qmm_add_rmsnorm_quantize(h: torch.Tensor, o: torch.Tensor, w: torch.Tensor, eps: float, q=None, d=None,
                             s=None, stream=None):
    """h <- h + o in place, then quantize rmsnorm(h) * w: returns (q, d, s)."""
    nt, idim = h.shape
    if o.shape != h.shape:
        raise ValueError("o must have the shape of h")
    _weight_vec(w, idim)
    q, d, s = _q8_out(h, q, d, s)
    _check(lib().qmm_add_rmsnorm_quantize(_dev(h, torch.float32, "h"), _dev(o, torch.float32, "o"),
                                          _dev(w, torch.float32, "w"), float(eps), nt, idim,
                                          *_q8_ptrs(q, d, s, nt, idim), _stream(stream)), "qmm_add_rmsnorm_quantize")
    return q, d, s


def qmm_rmsnorm_quantize(x: torch.Tensor, w: torch.Tensor, eps: float, q=None, d=None, s=None, stream=None):
    """Quantize rmsnorm(x) * w: returns (q, d, s)."""
    nt, idim = x.shape
    _weight_vec(w, idim)
    q, d, s = _q8_out(x, q, d, s)
    _check(lib().qmm_rmsnorm_quantize(_dev(x, torch.float32, "x"), _dev(w, torch.float32, "w"), float(eps), nt,
                                      idim, *_q8_ptrs(q, d, s, nt, idim), _stream(stream)), "qmm_rmsnorm_quantize")
    return q, d, s


def qmm_silu_mul_quantize(g: torch.Tensor, u: torch.Tensor, q=None, d=None, s=None, stream=None):
    """Quantize silu(g) * u: returns (q, d, s)."""
    nt, idim = g.shape
    if u.shape != g.shape:
        raise ValueError("u must have the shape of g")
    q, d, s = _q8_out(g, q, d, s)
    _check(lib().qmm_silu_mul_quantize(_dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), nt, idim,
                                       *_q8_ptrs(q, d, s, nt, idim), _stream(stream)), "qmm_silu_mul_quantize")
    return q, d, s


def _q8k_out(x: torch.Tensor, q, d, bsum):
    nt, idim = x.shape
    if q is None:
        q = torch.empty((nt, idim), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty((nt, idim // 256), dtype=torch.float32, device=x.device)
    if bsum is None:
        bsum = torch.empty((nt, idim // 16), dtype=torch.float32, device=x.device)
    return q, d, bsum


def qmm_add_rmsnorm_quantize_q8k(h: torch.Tensor, o: torch.Tensor, w: torch.Tensor, eps: float, q=None, d=None,
                                 bsum=None, stream=None):
    """h <- h + o in place, then rmsnorm(h) * w quantized to Q8_K: returns (q, d, bsum)."""
    nt, idim = h.shape
    if o.shape != h.shape:
        raise ValueError("o must have the shape of h")
    _weight_vec(w, idim)
    q, d, bsum = _q8k_out(h, q, d, bsum)
    _check(lib().qmm_add_rmsnorm_quantize_q8k(_dev(h, torch.float32, "h"), _dev(o, torch.float32, "o"),
                                              _dev(w, torch.float32, "w"), float(eps), nt, idim,
                                              *_q8k_ptrs(q, d, bsum, nt, idim), _stream(stream)),
           "qmm_add_rmsnorm_quantize_q8k")
    return q, d, bsum


def qmm_rmsnorm_quantize_q8k(x: torch.Tensor, w: torch.Tensor, eps: float, q=None, d=None, bsum=None, stream=None):
    """rmsnorm(x) * w quantized to Q8_K: returns (q, d, bsum)."""
    nt, idim = x.shape
    _weight_vec(w, idim)
    q, d, bsum = _q8k_out(x, q, d, bsum)
    _check(lib().qmm_rmsnorm_quantize_q8k(_dev(x, torch.float32, "x"), _dev(w, torch.float32, "w"), float(eps),
                                          nt, idim, *_q8k_ptrs(q, d, bsum, nt, idim), _stream(stream)),
           "qmm_rmsnorm_quantize_q8k")
    return q, d, bsum


def qmm_silu_mul_quantize_q8k(g: torch.Tensor, u: torch.Tensor, q=None, d=None, bsum=None, stream=None):
    """silu(g) * u quantized to Q8_K: returns (q, d, bsum)."""
    nt, idim = g.shape
    if u.shape != g.shape:
        raise ValueError("u must have the shape of g")
    q, d, bsum = _q8k_out(g, q, d, bsum)
    _check(lib().qmm_silu_mul_quantize_q8k(_dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), nt, idim,
                                           *_q8k_ptrs(q, d, bsum, nt, idim), _stream(stream)),
           "qmm_silu_mul_quantize_q8k")
    return q, d, bsum


def qmm_residual_add(h: torch.Tensor, o: torch.Tensor, stream=None) -> torch.Tensor:
    """h <- h + o in place; returns h."""
    nt, idim = h.shape
    if o.shape != h.shape:
        raise ValueError("o must have the shape of h")
    _check(lib().qmm_residual_add(_dev(h, torch.float32, "h"), _dev(o, torch.float32, "o"), nt, idim,
                                  _stream(stream)), "qmm_residual_add")
    return h


def qmm_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float, y=None, stream=None) -> torch.Tensor:
    """y = rmsnorm(x) * w (f32); y may be x."""
    nt, idim = x.shape
    _weight_vec(w, idim)
    if y is None:
        y = torch.empty_like(x)
    _check(lib().qmm_rmsnorm(_dev(x, torch.float32, "x"), _dev(w, torch.float32, "w"), float(eps), nt, idim,
                             _dev(y, torch.float32, "y", nt * idim), _stream(stream)), "qmm_rmsnorm")
    return y


def qmm_silu_mul(g: torch.Tensor, u: torch.Tensor, y=None, stream=None) -> torch.Tensor:
    """y = silu(g) * u (f32)."""
    nt, idim = g.shape
    if u.shape != g.shape:
        raise ValueError("u must have the shape of g")
    if y is None:
        y = torch.empty_like(g)
    _check(lib().qmm_silu_mul(_dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), nt, idim,
                              _dev(y, torch.float32, "y", nt * idim), _stream(stream)), "qmm_silu_mul")
    return y


def qmm_matmul(qtype: int, W: torch.Tensor, x: torch.Tensor, od: int, out=None, workspace=None, stream=None):
    """out f32 [nt, od] = quantize(x) then the nt-dispatched kernel."""
    nt, idim = x.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(qmm_matmul_ws_bytes(qtype, nt, od, idim), 1), dtype=torch.uint8,
                                device=x.device)
    _check(lib().qmm_matmul(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)), _dev(x, torch.float32, "x"),
                            nt, od, idim, _dev(out, torch.float32, "out", nt * od),
                            _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)),
           "qmm_matmul")
    return out


def qmm_matmul_noalloc(qtype: int, W: torch.Tensor, x: torch.Tensor, od: int, out=None, stream=None):
    """out f32 [nt, od] = quantize(x) then the nt-dispatched kernel, with the library's
    fixed device scratch as the workspace (the call itself allocates nothing; pass
    `out` to allocate nothing here either).  Calls overlapping on one device race."""
    nt, idim = x.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=x.device)
    _check(lib().qmm_matmul_noalloc(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                    _dev(x, torch.float32, "x"), nt, od, idim,
                                    _dev(out, torch.float32, "out", nt * od), _stream(stream)), "qmm_matmul_noalloc")
    return out


def qmm_matmul_q8(qtype: int, W: torch.Tensor, q: torch.Tensor, d: torch.Tensor, s: torch.Tensor, od: int,
                  out=None, stream=None):
    nt, idim = q.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=q.device)
    nb = nt * (idim // 32)
    _check(lib().qmm_matmul_q8(qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)), _dev(q, torch.int8, "q"),
                               _dev(d, torch.float32, "d", nb), _dev(s, torch.float32, "s", nb), nt, od, idim,
                               _dev(out, torch.float32, "out", nt * od), _stream(stream)), "qmm_matmul_q8")
    return out


def qmm_matmul_q8_kind(kind: int, qtype: int, W, q, d, s, od: int, out=None, stream=None):
    nt, idim = q.shape
    if out is None:
        out = torch.empty((nt, od), dtype=torch.float32, device=q.device)
    nb = nt * (idim // 32)
    _check(lib().qmm_matmul_q8_kind(kind, qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                    _dev(q, torch.int8, "q"), _dev(d, torch.float32, "d", nb),
                                    _dev(s, torch.float32, "s", nb), nt, od, idim,
                                    _dev(out, torch.float32, "out", nt * od), _stream(stream)), "qmm_matmul_q8_kind")
    return out


def qmm_group_dots(kind: int, qtype: int, W: torch.Tensor, q: torch.Tensor, od: int, S=None, stream=None):
    """int32 [nt, od, id/256, 8 or 16] per-scale-group integer dots from kernel `kind`."""
    nt, idim = q.shape
    ng = 16 if qtype in (QMM_TYPE_Q6_K, QMM_TYPE_Q6_K_P224) else 8
    if S is None:
        S = torch.empty((nt, od, idim // 256, ng), dtype=torch.int32, device=q.device)
    _check(lib().qmm_group_dots(kind, qtype, _dev(W, torch.uint8, "W", _wbytes(qtype, od, idim)),
                                _dev(q, torch.int8, "q"), nt, od, idim,
                                _dev(S, torch.int32, "S", nt * od * (idim // 256) * ng), _stream(stream)),
           "qmm_group_dots")
    return S


def qmm_mfma_tile_check(kind: int, A: torch.Tensor, B: torch.Tensor, C=None, stream=None):
    """One MFMA tile in the MMQ kernels' lane mapping (see include/qmm.h)."""
    if C is None:
        if kind == 1:
            C = torch.empty((32, 32), dtype=torch.int32, device=A.device)
        elif kind == 2:
            C = torch.empty((2, 32, 32), dtype=torch.float32, device=A.device)
        else:
            C = torch.empty((32, 32), dtype=torch.float32, device=A.device)
    dt = torch.int8 if kind == 1 else torch.float32
    ct = torch.int32 if kind == 1 else torch.float32
    na, nc = {1: (1024, 1024), 2: (64, 2048), 3: (64, 1024)}.get(int(kind), (0, 0))
    _check(lib().qmm_mfma_tile_check(int(kind), _dev(A, dt, "A", na), _dev(B, dt, "B", na), _dev(C, ct, "C", nc),
                                     _stream(stream)), "qmm_mfma_tile_check")
    return C
