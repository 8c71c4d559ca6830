"""Blockwise-scaled FP8 oracle (CPU): plain reference for the quantize + scaled-GEMM path.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. The product path (the HIP library and its Python
binding) never imports it, and it imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, IEEE binary32 for the quantizer steps, fp64 for the
GEMM); this module only builds/loads it with gcc and marshals numpy arrays. The SQNR helpers below
follow the GEMM-correctness table of "Enable blockwise FP8 dense training kernels on ROCm"
(FP8 GEMM compared with a BF16 matmul by SQNR in dB).

Array conventions:
  bf16 tensors are ``np.uint16`` bit patterns; fp8 tensors are ``np.uint8`` codes in the format
  ``fmt`` names: ``"e4m3fn"`` (default; finfo max 448) or ``"e4m3fnuz"`` (finfo max 240).
  ``a_s`` of the LHS quantizer is column-major [M, Kb]; it is returned as a C-contiguous numpy
  array of shape (Kb, M), which has the same bytes (element (m, kb) at kb * M + m).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
BLOCK = 128

_CFLAGS = [
    "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fexcess-precision=standard",
    "-fopenmp", "-fPIC", "-shared", "-Wall",
]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (seconds)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", *_CFLAGS, os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int

FORMATS = {"e4m3fn": 0, "e4m3fnuz": 1}
FP8_MAX = {"e4m3fn": 448.0, "e4m3fnuz": 240.0}


def _fmt(fmt: str) -> int:
    if fmt not in FORMATS:
        raise ValueError(f"unknown fp8 format {fmt!r}; expected one of {sorted(FORMATS)}")
    return FORMATS[fmt]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode_array.argtypes = [_f32p, _u8p, _i64]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_encode_bits.argtypes = [ctypes.c_uint32, _u8p, _i64]
        L.oracle_e4m3_encode_bits.restype = None
        L.oracle_e4m3fnuz_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3fnuz_encode.restype = ctypes.c_uint8
        L.oracle_e4m3fnuz_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fnuz_decode.restype = ctypes.c_double
        L.oracle_fp8_encode_array.argtypes = [_int, _f32p, _u8p, _i64]
        L.oracle_fp8_encode_array.restype = None
        L.oracle_fp8_encode_bits.argtypes = [_int, ctypes.c_uint32, _u8p, _i64]
        L.oracle_fp8_encode_bits.restype = None
        L.oracle_quantize_lhs.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _f32p, _int]
        L.oracle_quantize_rhs.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _f32p, _int]
        L.oracle_quantize_weight_128x128.argtypes = [
            _u16p, _i64, _i64, _i64, _u8p, _i64, _u8p, _i64, _f32p, _int]
        L.oracle_gemm_1x128_128x128.argtypes = [
            _u8p, _i64, _f32p, _u8p, _i64, _f32p, _i64, _i64, _i64, _i64, _i64, _i64p, _i64, _f64p,
            _int]
        L.oracle_gemm_1x128_128x1.argtypes = [
            _u8p, _i64, _f32p, _u8p, _i64, _f32p, _i64, _i64, _i64, _i64p, _i64, _f64p, _int]
        L.oracle_set_num_threads.argtypes = [_int]
        L.oracle_set_num_threads.restype = None
        for f in ("oracle_quantize_lhs", "oracle_quantize_rhs", "oracle_quantize_weight_128x128",
                  "oracle_gemm_1x128_128x128", "oracle_gemm_1x128_128x1", "oracle_num_threads"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(arr, t):
    return arr.ctypes.data_as(t)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (for single-thread timings)."""
    lib().oracle_set_num_threads(int(n))


def cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


# ------------------------------------------------------------------ codec

def e4m3_encode(v) -> np.ndarray:
    """Round-to-nearest-even, saturating e4m3fn encode of fp32 values (finite inputs)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(v, _f32p), _p(out, _u8p), v.size)
    return out


def e4m3_encode_bits(first: int, n: int) -> np.ndarray:
    """Codes of the fp32 bit patterns first .. first+n-1 (NaN patterns give 0xFF)."""
    out = np.empty(n, dtype=np.uint8)
    lib().oracle_e4m3_encode_bits(ctypes.c_uint32(first), _p(out, _u8p), n)
    return out


def e4m3_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().oracle_e4m3_decode(i) for i in range(256)], dtype=np.float64)
    return table[codes]


def fp8_encode(v, fmt: str = "e4m3fn") -> np.ndarray:
    """Round-to-nearest-even, saturating encode of fp32 values (finite inputs) in either format."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_fp8_encode_array(_fmt(fmt), _p(v, _f32p), _p(out, _u8p), v.size)
    return out


def fp8_encode_bits(first: int, n: int, fmt: str = "e4m3fn") -> np.ndarray:
    """Codes of the fp32 bit patterns first .. first+n-1 (NaN patterns give 0xFF)."""
    out = np.empty(n, dtype=np.uint8)
    lib().oracle_fp8_encode_bits(_fmt(fmt), ctypes.c_uint32(first), _p(out, _u8p), n)
    return out


def fp8_decode(codes, fmt: str = "e4m3fn") -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    dec = lib().oracle_e4m3fnuz_decode if _fmt(fmt) == 1 else lib().oracle_e4m3_decode
    table = np.array([dec(i) for i in range(256)], dtype=np.float64)
    return table[codes]


# ------------------------------------------------------------------ quantizers

def quantize_lhs(x: np.ndarray, fmt: str = "e4m3fn"):
    """1x128 row-wise groups of x [M, K] (bf16 bits). Returns (q [M, K], a_s as (Kb, M))."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    M, K = x.shape
    Kb = cdiv(K, BLOCK)
    q = np.zeros((M, K), dtype=np.uint8)
    a_s = np.zeros((Kb, M), dtype=np.float32)
    _check(lib().oracle_quantize_lhs(_p(x, _u16p), M, K, K, _p(q, _u8p), K, _p(a_s, _f32p),
                                    _fmt(fmt)), "quantize_lhs")
    return q, a_s


def quantize_rhs(x: np.ndarray, fmt: str = "e4m3fn"):
    """128x1 column-wise groups of x [K, N] (bf16 bits). Returns (qT [N, K], s [Kb, N])."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    K, N = x.shape
    Kb = cdiv(K, BLOCK)
    qT = np.zeros((N, K), dtype=np.uint8)
    s = np.zeros((Kb, N), dtype=np.float32)
    _check(lib().oracle_quantize_rhs(_p(x, _u16p), K, N, N, _p(qT, _u8p), K, _p(s, _f32p),
                                    _fmt(fmt)), "quantize_rhs")
    return qT, s


def quantize_rhs_grouped(x: np.ndarray, offsets, fmt: str = "e4m3fn"):
    """128x1 groups of expert-grouped tokens x [T, N] (bf16 bits) that restart at every expert's
    first token: expert e owns rows [offsets[e], offsets[e+1]) (clamped into [0, T] and to
    non-decreasing order) and is quantized on its own by quantize_rhs -- the per-expert act_quant_rhs
    the MoE weight gradient needs ("Enable blockwise FP8 dense training kernels on ROCm",
    description: the MoE path; the pages list no kernel for it, so this is the plainest reading).
    The results go into the 128-padded token layout: P[e] = sum over the experts before e of their
    token counts rounded up to a multiple of 128. Returns (qT [N, 128 G], s [G, N], P [E + 1]) with
    G = ceil(T / 128) + E: column P[e] + t of qT holds expert e's token t, row P[e] / 128 + g of s
    its group g; everything else (padding and the unused tail) is zero."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T, N = x.shape
    offsets = [int(v) for v in offsets]
    E = len(offsets) - 1
    G = cdiv(T, BLOCK) + E
    qT = np.zeros((N, G * BLOCK), dtype=np.uint8)
    s = np.zeros((G, N), dtype=np.float32)
    P = np.zeros(E + 1, dtype=np.int64)
    prev = pos = 0
    for e in range(E):
        a = min(max(offsets[e], prev), T)
        b = min(max(offsets[e + 1], a), T)
        prev = b
        P[e] = pos
        if b > a:
            q_e, s_e = quantize_rhs(x[a:b], fmt)
            qT[:, pos:pos + (b - a)] = q_e
            s[pos // BLOCK:pos // BLOCK + s_e.shape[0]] = s_e
        pos += cdiv(b - a, BLOCK) * BLOCK
    P[E] = pos
    return qT, s, P


def quantize_weight_128x128(w: np.ndarray, want_qT: bool = True, fmt: str = "e4m3fn"):
    """128x128 blocks of w [N, K] (bf16 bits). Returns (q [N, K], qT [K, N] or None, s [Nb, Kb])."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    N, K = w.shape
    q = np.zeros((N, K), dtype=np.uint8)
    qT = np.zeros((K, N), dtype=np.uint8) if want_qT else None
    s = np.zeros((cdiv(N, BLOCK), cdiv(K, BLOCK)), dtype=np.float32)
    qTp = _p(qT, _u8p) if want_qT else None
    _check(lib().oracle_quantize_weight_128x128(_p(w, _u16p), N, K, K, _p(q, _u8p), K, qTp, N,
                                                _p(s, _f32p), _fmt(fmt)),
           "quantize_weight_128x128")
    return q, qT, s


# ------------------------------------------------------------------ GEMMs

def _rows_arg(rows, M):
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    return np.ascontiguousarray(rows, dtype=np.int64)


def gemm_1x128_128x128(a, a_s, b, b_s, bs_stride_nb, bs_stride_kb, rows=None,
                       fmt: str = "e4m3fn") -> np.ndarray:
    """fp64 C rows for A [M, K] codes, a_s (Kb, M), B [N, K] codes, 128x128 b_s via strides."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    rows = _rows_arg(rows, M)
    out = np.zeros((rows.size, N), dtype=np.float64)
    _check(lib().oracle_gemm_1x128_128x128(
        _p(a, _u8p), K, _p(a_s, _f32p), _p(b, _u8p), K, _p(b_s, _f32p),
        bs_stride_nb, bs_stride_kb, M, N, K, _p(rows, _i64p), rows.size, _p(out, _f64p),
        _fmt(fmt)), "gemm_1x128_128x128")
    return out


def gemm_1x128_128x1(a, a_s, b, b_s, rows=None, fmt: str = "e4m3fn") -> np.ndarray:
    """fp64 C rows for A [M, K] codes, a_s (Kb, M), B [N, K] codes, per-column b_s [Kb, N]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K
    rows = _rows_arg(rows, M)
    out = np.zeros((rows.size, N), dtype=np.float64)
    _check(lib().oracle_gemm_1x128_128x1(
        _p(a, _u8p), K, _p(a_s, _f32p), _p(b, _u8p), K, _p(b_s, _f32p),
        M, N, K, _p(rows, _i64p), rows.size, _p(out, _f64p), _fmt(fmt)),
        "gemm_1x128_128x1")
    return out


# ------------------------------------------------------------------ accuracy metrics

def bf16_bits_to_f64(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.uint16)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def matmul_bf16_f64(a_bits, b_bits_nk, rows=None) -> np.ndarray:
    """fp64 reference C = A @ B^T of the original bf16 operands (B given as [N, K])."""
    a = bf16_bits_to_f64(a_bits if rows is None else np.asarray(a_bits)[rows])
    b = bf16_bits_to_f64(b_bits_nk)
    return a @ b.T


def sqnr_db(ref, test) -> float:
    """20 log10(||ref||_F / ||ref - test||_F)."""
    ref = np.asarray(ref, dtype=np.float64)
    test = np.asarray(test, dtype=np.float64)
    err = np.linalg.norm(ref - test)
    if err == 0.0:
        return float("inf")
    return float(20.0 * np.log10(np.linalg.norm(ref) / err))


def gemm_tolerance_report(c, c_oracle) -> dict:
    """Elementwise bound |C - C_o| <= 2e-2 (|C_o| + 1) and relative Frobenius error."""
    c = np.asarray(c, dtype=np.float64)
    c_oracle = np.asarray(c_oracle, dtype=np.float64)
    diff = np.abs(c - c_oracle)
    bound = 2e-2 * (np.abs(c_oracle) + 1.0)
    nf = np.linalg.norm(c_oracle)
    rel_f = float(np.linalg.norm(c - c_oracle) / nf) if nf > 0 else float(np.linalg.norm(c))
    return {
        "max_excess": float(np.max(diff - bound)) if diff.size else 0.0,
        "n_bad": int(np.count_nonzero(diff > bound)),
        "rel_frobenius": rel_f,
        "ok": bool(np.all(diff <= bound) and rel_f <= 4e-3),
    }
