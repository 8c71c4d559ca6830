// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI validates first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "schedule.hpp"

namespace bsfp8 {

// fnuz: float8_e4m3fnuz codes (FP8_MAX 240) instead of float8_e4m3fn (FP8_MAX 448).
// strip_loads: 0 = automatic (row strips of sched::lhs_strip_loads pieces per thread where the
// alignment allows, else tiles); 1, 2, 4, 8 or 16 = row strips of that many where the alignment
// allows; -1 = always the tile kernel.
hipError_t launch_quantize_lhs(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                               int64_t ldq, float* a_s, bool fnuz, int strip_loads, hipStream_t stream);
hipError_t launch_quantize_dual(const uint16_t* x, int64_t R, int64_t C, int64_t ldx, uint8_t* q,
                                int64_t ldq, float* a_s, uint8_t* qT, int64_t ldqT, float* s,
                                bool fnuz, hipStream_t stream);
// 128x1 groups that restart at every expert's first token, written in the 128-padded token layout
// (see quantize_rhs_grouped_kernel); padded: E + 1 padded boundaries (device memory, written).
hipError_t launch_quantize_rhs_grouped(const uint16_t* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets,
                                      int64_t E, uint8_t* qT, int64_t ldqT, float* s, int64_t* padded, bool fnuz,
                                      hipStream_t stream);
hipError_t launch_quantize_rhs(const uint16_t* x, int64_t K, int64_t N, int64_t ldx, uint8_t* qT,
                               int64_t ldqT, float* s, bool fnuz, hipStream_t stream);
hipError_t launch_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                  int64_t ldq, uint8_t* qT, int64_t ldqT, float* s, bool fnuz,
                                  hipStream_t stream);
// quantize_lhs(x) and quantize_weight_128x128(w) in one launch
hipError_t launch_quantize_step(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* qx,
                                int64_t ldqx, float* sx, const uint16_t* w, int64_t N, int64_t Kw,
                                int64_t ldw, uint8_t* qw, int64_t ldqw, uint8_t* qwT, int64_t ldqwT,
                                float* sw, bool fnuz, hipStream_t stream);
hipError_t launch_encode(const float* x, uint8_t* q, int64_t n, bool fnuz, hipStream_t stream);

// b-scale addressing of the GEMM: kind 0 = one scale per (K-block, 128-column block) at
// b_s[nb * stride_nb + kb * stride_kb]; kind 1 = one scale per (K-block, column) at b_s[kb * N + n].
struct BScale {
    const float* ptr;
    int64_t stride_nb;
    int64_t stride_kb;
    int per_column;
};

// Compute units of the current device (cached per device after the first query).
int device_cus();

// SplitPlan, gemm_split_plan and gemm_split_plan_forced: schedule.hpp.

// The allocation-free GEMM's scratch: a device array of gemm_scratch_bytes() bytes per device;
// gemm_scratch gives its address on the current device (looked up once per device).
int64_t gemm_scratch_bytes();
hipError_t gemm_scratch(float** out);

// fnuz: both operands hold float8_e4m3fnuz codes (general kernel, f16 matrix instructions).
// plan.S > 1 needs `workspace` (plan.bytes, 256-byte aligned, device memory) for the partial tiles.
hipError_t launch_gemm(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                       int64_t ldb, BScale bs, uint16_t* c, int64_t ldc, int64_t M, int64_t N,
                       int64_t K, bool fnuz, const SplitPlan& plan, float* workspace, int cus,
                       hipStream_t stream);

// Expert-grouped GEMMs (fast kernel; K % 128 == 0). offsets: E + 1 device int64 boundaries.
hipError_t launch_gemm_grouped_rows(const uint8_t* a, int64_t lda, const float* a_s,
                                    const uint8_t* b, int64_t ldb, int64_t b_stride, BScale bs,
                                    int64_t bs_stride, const int64_t* offsets, int64_t E,
                                    uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                    hipStream_t stream);
hipError_t launch_gemm_grouped_k(const uint8_t* a, int64_t lda, const float* a_s, const uint8_t* b,
                                 int64_t ldb, const float* b_s, const int64_t* offsets, int64_t E,
                                 uint16_t* c, int64_t ldc, int64_t c_stride, int64_t M, int64_t N,
                                 int64_t K, int32_t* status, hipStream_t stream);

}  // namespace bsfp8
