"""C-ABI library checks that need no GPU: it loads, exports every declared entry point, and rejects
bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from blockwise_scaled_fp8_act_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "blockwise_fp8.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from blockwise_scaled_fp8_act_amd import build
        build.build()
    return binding.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert set(names) >= {"quantize_lhs", "quantize_rhs", "quantize_weight_128x128",
                          "gemm_1x128_128x128", "gemm_1x128_128x1", "bsfp8_status_string",
                          "encode_e4m3_f32", "quantize_lhs_and_rhs",
                          "gemm_1x128_128x128_grouped", "gemm_1x128_128x1_grouped",
                          "quantize_lhs_fnuz", "quantize_rhs_fnuz", "quantize_weight_128x128_fnuz",
                          "quantize_lhs_and_rhs_fnuz", "gemm_1x128_128x128_fnuz",
                          "gemm_1x128_128x1_fnuz", "encode_e4m3fnuz_f32",
                          "quantize_lhs_and_weight", "quantize_lhs_and_weight_fnuz",
                          "quantize_rhs_grouped", "quantize_rhs_grouped_fnuz",
                          "gemm_1x128_128x128_noalloc"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(6):
        assert L.bsfp8_status_string(code) != b"unknown status"
    assert L.bsfp8_status_string(99) == b"unknown status"


P = ctypes.c_void_p(16 * 1024)  # a fake, 16-byte aligned address: never dereferenced on these paths


def test_quantizers_reject_bad_arguments(L):
    assert L.quantize_lhs(None, 4, 128, 128, P, 128, P, None) == 1
    assert L.quantize_lhs(P, -1, 128, 128, P, 128, P, None) == 1
    assert L.quantize_lhs(P, 4, 128, 127, P, 128, P, None) == 1      # ldx < K
    assert L.quantize_lhs(P, 4, 128, 128, P, 100, P, None) == 1      # ldq < K
    assert L.quantize_lhs(P, 4, 128, 128, P, 128, None, None) == 1
    assert L.quantize_rhs(P, 128, 64, 63, P, 128, P, None) == 1      # ldx < N
    assert L.quantize_rhs(P, 128, 64, 64, P, 100, P, None) == 1      # ldqT < K
    assert L.quantize_weight_128x128(P, 64, 64, 64, P, 64, P, 10, P, None) == 1  # ldqT < N
    assert L.quantize_weight_128x128(P, 64, 64, 64, None, 64, None, 0, P, None) == 1


def test_fused_quantizer_rejects_bad_arguments(L):
    f = L.quantize_lhs_and_rhs
    assert f(P, -1, 4, 4, P, 4, P, P, 0, P, None) == 1            # negative size
    assert f(P, 3, 64, 63, P, 64, P, P, 3, P, None) == 1          # ldx < C
    assert f(P, 3, 64, 64, P, 60, P, P, 3, P, None) == 1          # ldq < C
    assert f(P, 3, 64, 64, P, 64, P, P, 2, P, None) == 1          # ldqT < R
    assert f(P, 3, 64, 64, P, 64, None, P, 3, P, None) == 1       # a_s null
    assert f(P, 3, 64, 64, P, 64, P, None, 3, P, None) == 1       # qT null
    assert f(None, 0, 64, 64, None, 64, None, None, 0, None, None) == 0   # empty


def test_grouped_gemms_reject_bad_arguments(L):
    g = L.gemm_1x128_128x128_grouped
    #      a   lda  a_s b  ldb  bstr a_s  bss nb kb off E  c  ldc  M    N    K
    assert g(P, 128, P, P, 128, 0, P, 0, 1, 1, P, -1, P, 64, 256, 64, 128, None) == 1     # E < 0
    assert g(P, 144, P, P, 144, 0, P, 0, 1, 1, P, 2, P, 64, 256, 64, 130, None) == 1      # K % 128
    assert g(P, 128, P, P, 128, 0, P, 0, 1, 1, None, 2, P, 64, 256, 64, 128, None) == 1   # offsets
    assert g(P, 128, P, P, 128, 8, P, 0, 1, 1, P, 2, P, 64, 256, 64, 128, None) == 2      # b_stride % 16
    assert g(P, 128, P, P, 128, 0, P, -1, 1, 1, P, 2, P, 64, 256, 64, 128, None) == 1     # bs_stride < 0
    assert g(None, 0, None, None, 0, 0, None, 0, 0, 0, None, 0, None, 0, 5, 5, 128, None) == 0  # E = 0
    h = L.gemm_1x128_128x1_grouped
    #      a   lda  a_s b  ldb  b_s off E  c  ldc cstr    M   N   K  status
    assert h(P, 256, P, P, 256, P, P, 2, P, 64, 64 * 64, 64, 64, 130, None, None) == 1    # K % 128
    assert h(P, 256, P, P, 256, P, P, 2, P, 64, 100, 64, 64, 256, None, None) == 1        # outputs overlap
    assert h(P, 256, P, P, 256, P, None, 2, P, 64, 64 * 64, 64, 64, 256, None, None) == 1  # offsets
    assert h(None, 0, None, None, 0, None, None, 0, None, 0, 0, 3, 4, 256, None, None) == 0  # E = 0


def test_grouped_quantizer_rejects_bad_arguments(L):
    for f in (L.quantize_rhs_grouped, L.quantize_rhs_grouped_fnuz):
        #        x   T    N   ldx off E  qT  ldqT s  padded
        assert f(P, 300, 64, 64, P, 2, P, 624, P, P, None) == 1     # ldqT < 128 (ceil(T/128) + E) = 640
        assert f(P, 300, 64, 63, P, 2, P, 768, P, P, None) == 1     # ldx < N
        assert f(P, 300, 64, 64, None, 2, P, 768, P, P, None) == 1  # offsets
        assert f(P, 300, 64, 64, P, 2, P, 768, P, None, None) == 1  # padded offsets
        assert f(P, -1, 64, 64, P, 2, P, 768, P, P, None) == 1      # negative size
        assert f(P, 300, 64, 64, P, -1, P, 768, P, P, None) == 1    # negative E
        assert f(P, 128 * 65535, 64, 64, P, 1, P, 1 << 30, P, P, None) == 1  # more groups than the grid holds


def test_empty_problems_are_noops(L):
    assert L.quantize_lhs(None, 0, 128, 128, None, 128, None, None) == 0
    assert L.quantize_lhs(None, 4, 0, 0, None, 0, None, None) == 0
    assert L.quantize_rhs(None, 0, 5, 5, None, 0, None, None) == 0
    assert L.quantize_weight_128x128(None, 0, 0, 0, None, 0, None, 0, None, None) == 0
    assert L.gemm_1x128_128x128(None, 0, None, None, 0, None, 1, 1, None, 0, 0, 5, 7, None) == 0
    assert L.gemm_1x128_128x1(None, 0, None, None, 0, None, None, 0, 3, 0, 7, None) == 0
    assert L.encode_e4m3_f32(None, None, 0, None) == 0


def test_gemms_reject_bad_arguments(L):
    g = L.gemm_1x128_128x128
    assert g(P, 128, P, P, 128, P, 1, 1, P, 63, 4, 64, 128, None) == 1       # ldc < N
    assert g(P, 100, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 1       # lda < K
    assert g(P, 144, P, P, 136, P, 1, 1, P, 64, 4, 64, 130, None) == 2       # ldb % 16
    odd = ctypes.c_void_p(16 * 1024 + 8)
    assert g(odd, 128, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 2     # a misaligned
    assert g(P, 128, None, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 1    # a_s null
    assert g(P, 128, P, P, 128, P, -1, 1, P, 64, 4, 64, 128, None) == 1      # negative stride
    assert g(P, 128, P, P, 128, P, 1, 1, P, 64, -4, 64, 128, None) == 1
    h = L.gemm_1x128_128x1
    assert h(P, 128, P, P, 128, None, P, 64, 4, 64, 128, None) == 1          # b_s null
    assert h(P, 128, P, P, 120, P, P, 64, 4, 64, 128, None) == 1             # ldb < K
    assert L.encode_e4m3_f32(odd, P, 16, None) == 2


def test_gemm_size_limits_at_2_31(L):
    """Every operand and scale read goes through a buffer resource of at most 2^31 bytes: the
    largest admissible sizes pass validation (status 3 or 4 here: no GPU), one step past them is
    EINVAL before any HIP call."""
    g, h = L.gemm_1x128_128x128, L.gemm_1x128_128x1
    passed = lambda rc: rc not in (1, 2)                 # noqa: E731
    ld = 2 ** 31 // 256                                  # 256 rows of ld bytes: exactly 2^31
    assert passed(g(P, ld, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None))
    assert g(P, ld + 16, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 1
    assert g(P, 128, P, P, ld + 16, P, 1, 1, P, 64, 4, 64, 128, None) == 1
    M = 65535 * 128                                      # the most rows the grid takes
    assert passed(g(P, 8192, P, P, 8192, P, 64, 1, P, 64, M, 64, 8192, None))   # 4 M Kb < 2^31
    assert g(P, 8320, P, P, 8320, P, 65, 1, P, 64, M, 64, 8320, None) == 1      # 4 M Kb > 2^31
    assert g(P, 128, P, P, 128, P, 1, 1, P, 64, M + 128, 64, 128, None) == 1    # ceil(M/128) > 65535
    N = 2 ** 24
    assert passed(h(P, 4096, P, P, 4096, P, P, N, 4, N, 4096, None))            # 4 N Kb = 2^31
    assert h(P, 4224, P, P, 4224, P, P, N, 4, N, 4224, None) == 1               # 4 N Kb > 2^31
    # 128x128 B scales: the floats the strides span, times 4, at most 2^31
    assert passed(g(P, 128, P, P, 128, P, 2 ** 29 - 1, 1, P, 256, 4, 256, 128, None))
    assert g(P, 128, P, P, 128, P, 2 ** 29, 1, P, 256, 4, 256, 128, None) == 1


def test_fnuz_variants_validate_like_their_e4m3fn_twins(L):
    """Each *_fnuz entry point takes its twin's arguments and rejects the same bad ones, before any
    HIP call; empty problems are no-ops."""
    assert L.quantize_lhs_fnuz(None, 4, 128, 128, P, 128, P, None) == 1
    assert L.quantize_lhs_fnuz(P, 4, 128, 127, P, 128, P, None) == 1
    assert L.quantize_lhs_fnuz(P, 0, 128, 128, P, 128, P, None) == 0
    assert L.quantize_rhs_fnuz(P, 128, 64, 63, P, 128, P, None) == 1
    assert L.quantize_rhs_fnuz(P, 128, 0, 64, P, 128, P, None) == 0
    assert L.quantize_weight_128x128_fnuz(P, 64, 64, 64, P, 64, P, 10, P, None) == 1
    assert L.quantize_lhs_and_rhs_fnuz(P, 64, 64, 64, P, 64, P, P, 63, P, None) == 1  # ldqT < R
    assert L.quantize_lhs_and_rhs_fnuz(P, 0, 64, 64, P, 64, P, P, 64, P, None) == 0
    odd = ctypes.c_void_p(16 * 1024 + 8)
    # gemm_1x128_128x128_fnuz(a, lda, a_s, b, ldb, b_s, nb, kb, c, ldc, M, N, K, stream)
    assert L.gemm_1x128_128x128_fnuz(P, 100, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 1
    assert L.gemm_1x128_128x128_fnuz(odd, 128, P, P, 128, P, 1, 1, P, 64, 4, 64, 128, None) == 2
    assert L.gemm_1x128_128x128_fnuz(P, 128, P, P, 128, P, -1, 1, P, 64, 4, 64, 128, None) == 1
    assert L.gemm_1x128_128x128_fnuz(P, 128, P, P, 128, P, 1, 1, P, 64, 0, 64, 128, None) == 0
    # gemm_1x128_128x1_fnuz(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K, stream)
    assert L.gemm_1x128_128x1_fnuz(P, 128, P, P, 128, None, P, 64, 4, 64, 128, None) == 1
    assert L.gemm_1x128_128x1_fnuz(P, 128, P, P, 144, P, P, 63, 4, 64, 128, None) == 1  # ldc < N
    assert L.gemm_1x128_128x1_fnuz(P, 128, P, P, 120, P, P, 64, 4, 64, 128, None) == 1  # ldb < K
    assert L.encode_e4m3fnuz_f32(odd, P, 16, None) == 2
    assert L.encode_e4m3fnuz_f32(None, None, 0, None) == 0


def test_fused_step_quantizer_rejects_bad_arguments(L):
    # quantize_lhs_and_weight(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, s)
    for f in (L.quantize_lhs_and_weight, L.quantize_lhs_and_weight_fnuz):
        assert f(P, -1, 128, 128, P, 128, P, P, 64, 64, 64, P, 64, None, 0, P, None) == 1
        assert f(P, 4, 128, 127, P, 128, P, P, 64, 64, 64, P, 64, None, 0, P, None) == 1  # ldx < K
        assert f(P, 4, 128, 128, P, 128, None, P, 64, 64, 64, P, 64, None, 0, P, None) == 1
        assert f(P, 4, 128, 128, P, 128, P, P, 64, 64, 63, P, 64, None, 0, P, None) == 1  # ldw < Kw
        assert f(P, 4, 128, 128, P, 128, P, P, 64, 64, 64, P, 64, P, 10, P, None) == 1   # ldqwT < N
        assert f(P, 4, 128, 128, P, 128, P, None, 64, 64, 64, P, 64, None, 0, P, None) == 1
        assert f(P, 0, 128, 128, P, 128, P, P, 0, 64, 64, P, 64, None, 0, P, None) == 0  # both empty


def test_header_is_plain_c(tmp_path):
    """include/blockwise_fp8.h declares a C ABI: it compiles as C99 and as C++ without warnings, and
    a C caller links against the library's exported symbols."""
    import subprocess
    src = tmp_path / "use.c"
    src.write_text(
        '#include "blockwise_fp8.h"\n'
        "#include <stdio.h>\n"
        "int main(void) {\n"
        "    /* argument checks only: no GPU work is launched */\n"
        "    int rc = quantize_lhs(0, 4, 128, 128, 0, 128, 0, 0);\n"
        '    printf("%d %s\\n", rc, bsfp8_status_string(rc));\n'
        "    return rc == BSFP8_EINVAL ? 0 : 1;\n"
        "}\n")
    inc = os.path.join(ROOT, "include")
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-Werror", "-x", "c" if cc == "gcc" else "c++",
                            "-I", inc, "-c", str(src), "-o", str(tmp_path / f"use_{cc}.o")],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    exe = tmp_path / "use"
    r = subprocess.run(["gcc", str(tmp_path / "use_gcc.o"), binding.LIB_PATH,
                        f"-Wl,-rpath,{os.path.dirname(binding.LIB_PATH)}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("1 invalid argument"), (r.stdout, r.stderr)
