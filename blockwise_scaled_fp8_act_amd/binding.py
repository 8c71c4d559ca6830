"""Thin ctypes binding of libbsfp8.so (the gfx950 HIP library); declarations in include/blockwise_fp8.h.

Argument marshalling only: every step runs in the HIP kernels. torch provides device memory and the
current stream. There is no CPU fallback: if the library is missing, loading raises.

Tensor conventions (torch, on the GPU):
  bf16 inputs       torch.bfloat16 (or int16/uint16 holding bf16 bits)
  fp8 codes         torch.uint8 (``.view(torch.float8_e4m3fn)`` gives the same bytes as fp8);
                    with ``fmt="e4m3fnuz"`` (or torch.float8_e4m3fnuz) the codes are
                    float8_e4m3fnuz and FP8_MAX is 240 instead of 448
  LHS scales a_s    torch.float32 of shape (Kb, M), C-contiguous == column-major [M, Kb], ld M
  RHS scales s      torch.float32 (Kb, N) row-major
  weight scales s   torch.float32 (Nb, Kb) row-major
  GEMM output       torch.bfloat16 [M, N]
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsfp8.so")
BLOCK = 128

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64

_lib = None


class Bsfp8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().bsfp8_status_string(status).decode()
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


def lib():
    """Load libbsfp8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m blockwise_scaled_fp8_act_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.bsfp8_status_string.argtypes = [ctypes.c_int]
        L.bsfp8_status_string.restype = ctypes.c_char_p
        L.quantize_lhs.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]
        L.quantize_rhs.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]
        L.quantize_weight_128x128.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]
        L.gemm_1x128_128x128.argtypes = [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _i64,
                                         _i64, _i64, _i64, _vp]
        L.gemm_1x128_128x128_noalloc.argtypes = L.gemm_1x128_128x128.argtypes
        L.gemm_1x128_128x1.argtypes = [_vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i64,
                                       _vp]
        L.encode_e4m3_f32.argtypes = [_vp, _vp, _i64, _vp]
        L.quantize_lhs_and_rhs.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp]
        L.gemm_1x128_128x128_grouped.argtypes = [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _i64,
                                                 _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp]
        L.gemm_1x128_128x1_grouped.argtypes = [_vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64,
                                               _i64, _i64, _i64, _i64, _vp, _vp]
        L.quantize_rhs_grouped.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp]
        L.quantize_rhs_grouped_fnuz.argtypes = L.quantize_rhs_grouped.argtypes
        L.quantize_lhs_and_weight.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _i64,
                                              _i64, _vp, _i64, _vp, _i64, _vp, _vp]
        for f in ("quantize_lhs", "quantize_rhs", "quantize_weight_128x128", "gemm_1x128_128x128",
                  "gemm_1x128_128x1", "quantize_lhs_and_rhs", "encode_e4m3_f32",
                  "quantize_lhs_and_weight"):
            fz = getattr(L, f.replace("e4m3", "e4m3fnuz") if f.startswith("encode") else f + "_fnuz")
            fz.argtypes = getattr(L, f).argtypes
        for f in ("quantize_lhs", "quantize_rhs", "quantize_weight_128x128", "gemm_1x128_128x128",
                  "gemm_1x128_128x1", "encode_e4m3_f32", "quantize_lhs_and_rhs",
                  "gemm_1x128_128x128_grouped", "gemm_1x128_128x1_grouped",
                  "gemm_1x128_128x128_noalloc", "quantize_rhs_grouped", "quantize_rhs_grouped_fnuz",
                  "quantize_lhs_fnuz", "quantize_rhs_fnuz", "quantize_weight_128x128_fnuz",
                  "gemm_1x128_128x128_fnuz", "gemm_1x128_128x1_fnuz", "encode_e4m3fnuz_f32",
                  "quantize_lhs_and_rhs_fnuz", "quantize_lhs_and_weight",
                  "quantize_lhs_and_weight_fnuz"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


# the current stream's handle without building a torch.cuda.Stream object (0.1 against ~3 us per
# call), where this torch provides it
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    if stream is None:
        if _raw_stream is not None:
            return _vp(_raw_stream(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _ld(t):
    """Row stride (elements) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.stride(0)


_fns = {}


def _call(fn, *args):
    f = _fns.get(fn)
    if f is None:
        f = _fns[fn] = getattr(lib(), fn)
    rc = f(*args)
    if rc != 0:
        raise Bsfp8Error(fn, rc)


def cdiv(a, b):
    return (a + b - 1) // b


FORMATS = ("e4m3fn", "e4m3fnuz")


def fp8_format(fmt) -> str:
    """Normalise an FP8 element-format choice: "e4m3fn" / "e4m3fnuz" or the torch dtypes
    torch.float8_e4m3fn / torch.float8_e4m3fnuz."""
    if fmt is torch.float8_e4m3fn:
        return "e4m3fn"
    if fmt is torch.float8_e4m3fnuz:
        return "e4m3fnuz"
    if fmt in FORMATS:
        return fmt
    raise ValueError(f"unsupported FP8 format {fmt!r}: expected one of {FORMATS} or the matching "
                     "torch float8 dtype")


def _entry(fn, fmt):
    return fn + "_fnuz" if fp8_format(fmt) == "e4m3fnuz" else fn


# ---------------------------------------------------------------- argument checks
# Every tensor is checked before the library is called: dtype, rank, shape, row contiguity, and
# last that it lives on the current GPU (the library works on the current device), so a wrong
# argument raises TypeError / ValueError here instead of reaching a kernel.

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_CODES = {"e4m3fn": (torch.uint8, torch.float8_e4m3fn), "e4m3fnuz": (torch.uint8, torch.float8_e4m3fnuz)}


def _on_gpu(name, t, dev=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
    if dev is None:
        dev = torch.cuda.current_device()
    if t.get_device() != dev:
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{dev}")


def _matrix(name, t, dtypes, shape=None):
    """A 2-D tensor of one of ``dtypes`` with contiguous rows; ``shape`` entries of None are free."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if shape is not None and any(w is not None and g != w for g, w in zip(t.shape, shape)):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{tuple('*' if w is None else w for w in shape)}")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have contiguous rows (stride {t.stride()})")
    return t


def _dense(name, t, dtype, shape):
    """A C-contiguous tensor of ``dtype`` and exactly ``shape``."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _codes(name, t, fmt, shape=None):
    return _matrix(name, t, _CODES[fp8_format(fmt)], shape)


def _gpu(**tensors):
    dev = None
    for name, t in tensors.items():
        if t is not None:
            if not t.is_cuda:
                raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
            if dev is None:
                dev = torch.cuda.current_device()
            _on_gpu(name, t, dev)


def _strided_scales(name, t, Nb, Kb, nb, kb):
    """fp32 scales read at t[nb_i * nb + kb_i * kb] for nb_i < Nb, kb_i < Kb (flat, from t's start)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 tensor")
    if nb < 0 or kb < 0:
        raise ValueError(f"{name} strides must be >= 0, got ({nb}, {kb})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (its strides are passed separately)")
    need = (Nb - 1) * nb + (Kb - 1) * kb + 1 if Nb > 0 and Kb > 0 else 0
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} floats, the strides ({nb}, {kb}) read {need}")


def quantize_lhs(x, q=None, a_s=None, stream=None, fmt="e4m3fn"):
    """1x128 row-wise quantization of x [M, K]. Returns (q [M, K] uint8, a_s (Kb, M) fp32)."""
    M, K = _matrix("x", x, _BF16).shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if a_s is None:
        a_s = torch.empty((cdiv(K, BLOCK), M), dtype=torch.float32, device=x.device)
    _codes("q", q, fmt, (M, K))
    _dense("a_s", a_s, torch.float32, (cdiv(K, BLOCK), M))
    _gpu(x=x, q=q, a_s=a_s)
    _call(_entry("quantize_lhs", fmt), _ptr(x), M, K, _ld(x), _ptr(q), _ld(q), _ptr(a_s),
          _stream(stream))
    return q, a_s


def quantize_rhs(x, qT=None, s=None, stream=None, fmt="e4m3fn"):
    """128x1 column-wise quantization of x [K, N]. Returns (qT [N, K] uint8, s (Kb, N) fp32)."""
    K, N = _matrix("x", x, _BF16).shape
    if qT is None:
        qT = torch.empty((N, K), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((cdiv(K, BLOCK), N), dtype=torch.float32, device=x.device)
    _codes("qT", qT, fmt, (N, K))
    _dense("s", s, torch.float32, (cdiv(K, BLOCK), N))
    _gpu(x=x, qT=qT, s=s)
    _call(_entry("quantize_rhs", fmt), _ptr(x), K, N, _ld(x), _ptr(qT), _ld(qT), _ptr(s),
          _stream(stream))
    return qT, s


def quantize_lhs_and_rhs(x, q=None, a_s=None, qT=None, s=None, stream=None, fmt="e4m3fn"):
    """Both activation quantizations of x [R, C] in one pass. Returns (q [R, C], a_s (Kb_C, R),
    qT [C, R], s (Kb_R, C)): the outputs of quantize_lhs(x) and of quantize_rhs(x)."""
    R, C = _matrix("x", x, _BF16).shape
    if q is None:
        q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    if a_s is None:
        a_s = torch.empty((cdiv(C, BLOCK), R), dtype=torch.float32, device=x.device)
    if qT is None:
        qT = torch.empty((C, R), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((cdiv(R, BLOCK), C), dtype=torch.float32, device=x.device)
    _codes("q", q, fmt, (R, C))
    _dense("a_s", a_s, torch.float32, (cdiv(C, BLOCK), R))
    _codes("qT", qT, fmt, (C, R))
    _dense("s", s, torch.float32, (cdiv(R, BLOCK), C))
    _gpu(x=x, q=q, a_s=a_s, qT=qT, s=s)
    _call(_entry("quantize_lhs_and_rhs", fmt), _ptr(x), R, C, _ld(x), _ptr(q), _ld(q), _ptr(a_s),
          _ptr(qT), _ld(qT), _ptr(s), _stream(stream))
    return q, a_s, qT, s


def quantize_lhs_and_weight(x, w, qx=None, sx=None, qw=None, qwT=None, sw=None, want_qT=False,
                            stream=None, fmt="e4m3fn"):
    """quantize_lhs(x) and quantize_weight_128x128(w) in one launch (the two quantizations of a
    linear layer's forward step). Returns (qx [M, K], sx (Kb, M), qw [N, Kw], qwT [Kw, N] or None,
    sw (Nb, Kbw)), byte-identical to the two separate calls."""
    M, K = _matrix("x", x, _BF16).shape
    N, Kw = _matrix("w", w, _BF16).shape
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sx is None:
        sx = torch.empty((cdiv(K, BLOCK), M), dtype=torch.float32, device=x.device)
    if qw is None:
        qw = torch.empty((N, Kw), dtype=torch.uint8, device=w.device)
    if qwT is None and want_qT:
        qwT = torch.empty((Kw, N), dtype=torch.uint8, device=w.device)
    if sw is None:
        sw = torch.empty((cdiv(N, BLOCK), cdiv(Kw, BLOCK)), dtype=torch.float32, device=w.device)
    _codes("qx", qx, fmt, (M, K))
    _dense("sx", sx, torch.float32, (cdiv(K, BLOCK), M))
    _codes("qw", qw, fmt, (N, Kw))
    if qwT is not None:
        _codes("qwT", qwT, fmt, (Kw, N))
    _dense("sw", sw, torch.float32, (cdiv(N, BLOCK), cdiv(Kw, BLOCK)))
    _gpu(x=x, w=w, qx=qx, sx=sx, qw=qw, qwT=qwT, sw=sw)
    ldqwT = _ld(qwT) if qwT is not None else 0
    _call(_entry("quantize_lhs_and_weight", fmt), _ptr(x), M, K, _ld(x), _ptr(qx), _ld(qx), _ptr(sx),
          _ptr(w), N, Kw, _ld(w), _ptr(qw), _ld(qw), _ptr(qwT), ldqwT, _ptr(sw), _stream(stream))
    return qx, sx, qw, qwT, sw


def quantize_weight_128x128(w, q=None, qT=None, s=None, want_qT=True, stream=None,
                            fmt="e4m3fn"):
    """128x128 block quantization of w [N, K]. Returns (q [N, K], qT [K, N] or None, s (Nb, Kb))."""
    N, K = _matrix("w", w, _BF16).shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if qT is None and want_qT:
        qT = torch.empty((K, N), dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((cdiv(N, BLOCK), cdiv(K, BLOCK)), dtype=torch.float32, device=w.device)
    _codes("q", q, fmt, (N, K))
    if qT is not None:
        _codes("qT", qT, fmt, (K, N))
    _dense("s", s, torch.float32, (cdiv(N, BLOCK), cdiv(K, BLOCK)))
    _gpu(w=w, q=q, qT=qT, s=s)
    ldqT = _ld(qT) if qT is not None else 0
    _call(_entry("quantize_weight_128x128", fmt), _ptr(w), N, K, _ld(w), _ptr(q), _ld(q), _ptr(qT),
          ldqT, _ptr(s), _stream(stream))
    return q, qT, s


def _gemm_operands(a, a_s, b, K, fmt):
    """Checks A [M, >= K] and B [N, >= K] codes and a_s (Kb, M); returns (M, N, K)."""
    _codes("a", a, fmt)
    _codes("b", b, fmt)
    M, N = a.shape[0], b.shape[0]
    K = a.shape[1] if K is None else int(K)
    if K < 0 or K > a.shape[1] or K > b.shape[1]:
        raise ValueError(f"K = {K} must lie in [0, min(a.shape[1], b.shape[1])] = [0, {min(a.shape[1], b.shape[1])}]")
    if K > 0:
        _dense("a_s", a_s, torch.float32, (cdiv(K, BLOCK), M))
    return M, N, K


def _gemm_rest(a, a_s, b, b_s, nb, kb, c, M, N, K):
    """Checks the B scales (128x128 through strides nb, kb; 128x1 (Kb, N) when nb is None) and C,
    then that every tensor the call reads or writes is on the current GPU."""
    if K > 0:
        if nb is None:
            _dense("b_s", b_s, torch.float32, (cdiv(K, BLOCK), N))
        else:
            _strided_scales("b_s", b_s, cdiv(N, BLOCK), cdiv(K, BLOCK), nb, kb)
    _matrix("c", c, (torch.bfloat16,), (M, N))
    _gpu(a=a, b=b, c=c, a_s=a_s if K > 0 else None, b_s=b_s if K > 0 else None)


def gemm_1x128_128x128(a, a_s, b, b_s, bs_stride_nb=None, bs_stride_kb=None, c=None, K=None,
                       stream=None, fmt="e4m3fn"):
    """C = A B^T, A [M, K] codes with a_s (Kb, M); B [N, K] codes with 128x128 scales.
    ``b_s`` is addressed as b_s[nb * bs_stride_nb + kb * bs_stride_kb]; the default strides treat it
    as the weight quantizer's (Nb, Kb) tensor. ``fmt`` is the element format of both operands."""
    M, N, K = _gemm_operands(a, a_s, b, K, fmt)
    if bs_stride_nb is None:
        bs_stride_nb, bs_stride_kb = b_s.stride(0), b_s.stride(1)
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _gemm_rest(a, a_s, b, b_s, bs_stride_nb, bs_stride_kb, c, M, N, K)
    _call(_entry("gemm_1x128_128x128", fmt), _ptr(a), _ld(a), _ptr(a_s), _ptr(b), _ld(b), _ptr(b_s),
          bs_stride_nb, bs_stride_kb, _ptr(c), _ld(c), M, N, K, _stream(stream))
    return c


def gemm_1x128_128x128_noalloc(a, a_s, b, b_s, c, bs_stride_nb=None, bs_stride_kb=None, K=None,
                               stream=None):
    """gemm_1x128_128x128 (e4m3fn) into a caller-provided ``c``, with the K-split partial tiles in
    the library's static scratch: the call allocates no device memory."""
    M, N, K = _gemm_operands(a, a_s, b, K, "e4m3fn")
    if bs_stride_nb is None:
        bs_stride_nb, bs_stride_kb = b_s.stride(0), b_s.stride(1)
    _gemm_rest(a, a_s, b, b_s, bs_stride_nb, bs_stride_kb, c, M, N, K)
    _call("gemm_1x128_128x128_noalloc", _ptr(a), _ld(a), _ptr(a_s), _ptr(b), _ld(b), _ptr(b_s),
          bs_stride_nb, bs_stride_kb, _ptr(c), _ld(c), M, N, K, _stream(stream))
    return c


def gemm_1x128_128x1(a, a_s, b, b_s, c=None, K=None, stream=None, fmt="e4m3fn"):
    """C = A B^T, A [M, K] codes with a_s (Kb, M); B [N, K] codes with per-column b_s (Kb, N).
    ``fmt`` is the element format of both operands."""
    M, N, K = _gemm_operands(a, a_s, b, K, fmt)
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _gemm_rest(a, a_s, b, b_s, None, None, c, M, N, K)
    _call(_entry("gemm_1x128_128x1", fmt), _ptr(a), _ld(a), _ptr(a_s), _ptr(b), _ld(b), _ptr(b_s),
          _ptr(c), _ld(c), M, N, K, _stream(stream))
    return c


def _flat_f32(x):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    return x


def _flat_codes(q, n):
    if not isinstance(q, torch.Tensor) or q.dtype != torch.uint8 or not q.is_contiguous() or q.numel() != n:
        raise ValueError(f"q must be a contiguous uint8 tensor of {n} elements")


def encode_e4m3_f32(x, q=None, stream=None):
    """Element conversion of fp32 values to e4m3fn codes (clamped to +-448, RNE)."""
    n = _flat_f32(x).numel()
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _flat_codes(q, n)
    _gpu(x=x, q=q)
    _call("encode_e4m3_f32", _ptr(x), _ptr(q), n, _stream(stream))
    return q


def encode_e4m3fnuz_f32(x, q=None, stream=None):
    """The quantizers' float8_e4m3fnuz conversion (RNE) of fp32 values with
    |x| <= 240 (1 + 2^-21)."""
    n = _flat_f32(x).numel()
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _flat_codes(q, n)
    _gpu(x=x, q=q)
    _call("encode_e4m3fnuz_f32", _ptr(x), _ptr(q), n, _stream(stream))
    return q


def _offsets(offsets, E):
    if not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.int64:
        raise TypeError("offsets must be an int64 tensor")
    if offsets.dim() != 1 or offsets.numel() < E + 1 or not offsets.is_contiguous():
        raise ValueError(f"offsets must be a contiguous 1-D tensor of at least E + 1 = {E + 1} boundaries")


def gemm_1x128_128x128_grouped(a, a_s, b, b_s, offsets, E, b_stride, bs_stride, bs_stride_nb,
                               bs_stride_kb, ldb=None, c=None, N=None, stream=None):
    """Expert-grouped C = A B_e^T over the row ranges [offsets[e], offsets[e+1]) of A and C.
    a [M, K] codes with a_s (Kb, M); B_e starts b_stride bytes after B_(e-1) in ``b`` (a uint8
    tensor, rows of stride ldb, default its row stride); scales of expert e start bs_stride floats
    after those of e-1 in ``b_s`` and are addressed with (bs_stride_nb, bs_stride_kb); ``offsets``
    is an int64 device tensor of E + 1 boundaries. N defaults to b's row count when b holds the
    experts' rows stacked ([E*N, K])."""
    M, K = _codes("a", a, "e4m3fn").shape
    _codes("b", b, "e4m3fn")
    if ldb is None:
        ldb = _ld(b)
    if N is None:
        N = b.shape[0] // E
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _dense("a_s", a_s, torch.float32, (cdiv(K, BLOCK), M))
    if not isinstance(b_s, torch.Tensor) or b_s.dtype != torch.float32 or not b_s.is_contiguous():
        raise TypeError("b_s must be a contiguous float32 tensor")
    _offsets(offsets, E)
    _matrix("c", c, (torch.bfloat16,), (M, N))
    _gpu(a=a, a_s=a_s, b=b, b_s=b_s, offsets=offsets, c=c)
    _call("gemm_1x128_128x128_grouped", _ptr(a), _ld(a), _ptr(a_s), _ptr(b), ldb, b_stride,
          _ptr(b_s), bs_stride, bs_stride_nb, bs_stride_kb, _ptr(offsets), E, _ptr(c), _ld(c), M, N,
          K, _stream(stream))
    return c


def gemm_1x128_128x1_grouped(a, a_s, b, b_s, offsets, E, c=None, status=None, stream=None):
    """Per-expert C_e = A_e B_e^T over the token (column) ranges [offsets[e], offsets[e+1]) of
    A [M, K] and B [N, K] (128x1 codes over all tokens, scales (Kb, M) and (Kb, N)); returns
    c [E, M, N] bf16. Every boundary must be a multiple of 128 (quantize_rhs_grouped's padded
    offsets are); an expert whose range is not gets NaN outputs and sets ``status`` (an int32 GPU
    tensor, optional) to 1."""
    M, K = _codes("a", a, "e4m3fn").shape
    N = _codes("b", b, "e4m3fn", (None, K)).shape[0]
    if c is None:
        c = torch.empty((E, M, N), dtype=torch.bfloat16, device=a.device)
    _dense("a_s", a_s, torch.float32, (cdiv(K, BLOCK), M))
    _dense("b_s", b_s, torch.float32, (cdiv(K, BLOCK), N))
    _offsets(offsets, E)
    if not isinstance(c, torch.Tensor) or c.dtype != torch.bfloat16:
        raise TypeError("c must be a bfloat16 tensor")
    if c.dim() != 3 or tuple(c.shape) != (E, M, N) or (c.stride(2) != 1 and N > 1):
        raise ValueError(f"expected c [E, M, N] = {(E, M, N)} with contiguous rows, got {tuple(c.shape)}")
    if status is not None and (not isinstance(status, torch.Tensor) or status.dtype != torch.int32
                               or status.numel() < 1):
        raise TypeError("status must be an int32 tensor of at least one element")
    _gpu(a=a, a_s=a_s, b=b, b_s=b_s, offsets=offsets, c=c, status=status)
    _call("gemm_1x128_128x1_grouped", _ptr(a), _ld(a), _ptr(a_s), _ptr(b), _ld(b), _ptr(b_s),
          _ptr(offsets), E, _ptr(c), c.stride(1), c.stride(0), M, N, K, _ptr(status), _stream(stream))
    return c


def quantize_rhs_grouped(x, offsets, E, qT=None, s=None, padded_offsets=None, stream=None, fmt="e4m3fn"):
    """128x1 quantization of expert-grouped tokens x [T, N] (expert e owns rows
    [offsets[e], offsets[e+1])) with groups restarting at every expert's first token, in the
    128-padded token layout. Returns (qT [N, 128 G], s (G, N), padded_offsets [E + 1] int64) with
    G = ceil(T / 128) + E; columns and scale rows past padded_offsets[E] are not written."""
    T, N = _matrix("x", x, _BF16).shape
    _offsets(offsets, E)
    G = cdiv(T, BLOCK) + E
    if qT is None:
        qT = torch.empty((N, G * BLOCK), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((G, N), dtype=torch.float32, device=x.device)
    if padded_offsets is None:
        padded_offsets = torch.empty(E + 1, dtype=torch.int64, device=x.device)
    _codes("qT", qT, fmt, (N, None))
    if qT.shape[1] < G * BLOCK:
        raise ValueError(f"qT needs at least 128 (ceil(T/128) + E) = {G * BLOCK} columns, has {qT.shape[1]}")
    _dense("s", s, torch.float32, (G, N))
    _offsets(padded_offsets, E)
    _gpu(x=x, offsets=offsets, qT=qT, s=s, padded_offsets=padded_offsets)
    _call(_entry("quantize_rhs_grouped", fmt), _ptr(x), T, N, _ld(x), _ptr(offsets), E, _ptr(qT), _ld(qT),
          _ptr(s), _ptr(padded_offsets), _stream(stream))
    return qT, s, padded_offsets
