// C ABI of the blockwise FP8 library: argument validation (before any HIP call), a per-device
// gfx950 check, and launches on the caller's stream. Declarations and contracts: blockwise_fp8.h.
#include "blockwise_fp8.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.hpp"

namespace {

constexpr int64_t kGroupEdge = 128;
constexpr int64_t kMaxGridY = 65535;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 0 = unknown, 1 = gfx950, 2 = other. Indexed by HIP device ordinal.
std::atomic<int> g_arch_state[64];

int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return BSFP8_EHIP;
    if (dev < 0 || dev >= 64) return BSFP8_EDEVICE;
    int st = g_arch_state[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return BSFP8_EHIP;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? BSFP8_OK : BSFP8_EDEVICE;
}

int finish(hipError_t e) { return e == hipSuccess ? BSFP8_OK : BSFP8_EHIP; }

// Compute units per device ordinal, queried once (0 = not yet known).
std::atomic<int> g_cus[64];

}  // namespace

int bsfp8::device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = g_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        g_cus[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The GEMM kernels read every operand and scale tensor through buffer resources of at most 2^31
// bytes (a 256-row band of an operand, a whole scale tensor), so that an out-of-range lane offset
// (2^31 plus a per-K-block advance below 2^31) is always past the end.
constexpr int64_t kMaxRange = 0x80000000LL;
constexpr int64_t kMaxOperandLd = kMaxRange / 256;

int validate_gemm(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                  const float* b_s, const void* c, int64_t ldc, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0) return BSFP8_EINVAL;
    if (M == 0 || N == 0) return BSFP8_OK;
    if (c == nullptr || ldc < N) return BSFP8_EINVAL;
    if (cdiv(M, kGroupEdge) > kMaxGridY) return BSFP8_EINVAL;
    if (K == 0) return BSFP8_OK;
    if (a == nullptr || b == nullptr || a_s == nullptr || b_s == nullptr) return BSFP8_EINVAL;
    if (lda < K || ldb < K) return BSFP8_EINVAL;
    if (lda > kMaxOperandLd || ldb > kMaxOperandLd) return BSFP8_EINVAL;
    if (4 * M * cdiv(K, kGroupEdge) > kMaxRange) return BSFP8_EINVAL;
    if (!aligned16(a) || !aligned16(b) || (lda % 16) != 0 || (ldb % 16) != 0) return BSFP8_EALIGN;
    return BSFP8_OK;
}

// Split-K workspaces (shapes whose output tiles cannot fill the chip) come from a per-device
// stream-ordered memory pool whose memory is never returned to the system, so a call allocates
// from the driver only until the pool has grown to its largest workspace, and calls on different
// streams never share a buffer.
constexpr int64_t kMaxSplitWorkspace = 256LL << 20;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[64];

hipError_t device_pool(hipMemPool_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (g_pools[dev] == nullptr) {
        hipMemPoolProps props;
        std::memset(&props, 0, sizeof(props));
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t pool = nullptr;
        if ((e = hipMemPoolCreate(&pool, &props)) != hipSuccess) return e;
        uint64_t keep = UINT64_MAX;
        if ((e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) return e;
        g_pools[dev] = pool;
    }
    *out = g_pools[dev];
    return hipSuccess;
}

// BSFP8_GEMM_SPLIT, BSFP8_GEMM_TILE_M, BSFP8_GEMM_TILE_N, BSFP8_GEMM_THIN_STAGES and
// BSFP8_GEMM_THIN_WAVES (environment, read at each call): a slice count (1 = never split), a tile
// height (256 or 128: the fast kernel; 64: the thin kernel), the thin kernel's tile width (32, 64 or
// 128), its LDS stages (2, 3, 4, 6, 8 or 12, as far as the tile's stages fit the LDS) and its waves
// per workgroup (4, or 8 for tiles of 64 or 128 columns; other values fail with BSFP8_EHIP) that
// replace the automatic choices of gemm_split_plan, so tests and benchmarks can run every schedule
// on any shape. Unset or empty: automatic.
int env_int(const char* name) {
    const char* v = std::getenv(name);
    if (v == nullptr || *v == 0) return 0;
    const long s = std::strtol(v, nullptr, 10);
    return s < 1 ? 1 : (s > 65535 ? 65535 : static_cast<int>(s));
}

// The GEMM with its K split when the plan asks for it. The workspace is allocated and freed in
// stream order around the two kernels, or, with use_scratch, is the library's static scratch
// (nothing allocated; a plan larger than the scratch is BSFP8_ESCRATCH).
int run_gemm(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
             bsfp8::BScale bs, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, bool fnuz,
             bool use_scratch, hipStream_t stream) {
    const int cus = bsfp8::device_cus();
    const int forced_s = env_int("BSFP8_GEMM_SPLIT"), forced_bm = env_int("BSFP8_GEMM_TILE_M");
    const int forced_bn = env_int("BSFP8_GEMM_TILE_N");
    bsfp8::SplitPlan plan =
        forced_s || forced_bm || forced_bn
            ? bsfp8::gemm_split_plan_forced(M, N, K, fnuz, cus, forced_s, forced_bm, forced_bn, kMaxSplitWorkspace)
            : bsfp8::gemm_split_plan(M, N, K, fnuz, cus, kMaxSplitWorkspace);
    if (plan.bm == bsfp8::geom::kThinBM) {
        plan.stages = env_int("BSFP8_GEMM_THIN_STAGES");
        plan.waves = env_int("BSFP8_GEMM_THIN_WAVES");
    }
    // A partial last round of 256 x 256 tiles: the leading columns as one GEMM, the tail columns
    // with K split (schedule.hpp, gemm_column_split). Automatic schedules with 128 x 128 B scales
    // only; BSFP8_GEMM_COLUMN_SPLIT=0 turns it off.
    const char* col_env = std::getenv("BSFP8_GEMM_COLUMN_SPLIT");
    const bool col_off = col_env != nullptr && col_env[0] == '0';
    if (!fnuz && !bs.per_column && !forced_s && !forced_bm && !forced_bn && !col_off) {
        const bsfp8::ColumnSplit cs = bsfp8::gemm_column_split(M, N, K, cus, kMaxSplitWorkspace);
        if (cs.n1 > 0 && (!use_scratch || cs.tail.bytes <= bsfp8::gemm_scratch_bytes())) {
            float* ws = nullptr;
            hipMemPool_t pool = nullptr;
            if (use_scratch) {
                if (bsfp8::gemm_scratch(&ws) != hipSuccess) return BSFP8_EHIP;
            } else {
                if (device_pool(&pool) != hipSuccess) return BSFP8_EHIP;
                if (hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(cs.tail.bytes), pool,
                                           stream) != hipSuccess)
                    return BSFP8_EHIP;
            }
            const uint8_t* a8 = static_cast<const uint8_t*>(a);
            const uint8_t* b8 = static_cast<const uint8_t*>(b);
            uint16_t* c16 = static_cast<uint16_t*>(c);
            hipError_t e = bsfp8::launch_gemm(a8, lda, a_s, b8, ldb, bs, c16, ldc, M, cs.n1, K, false, plan, nullptr,
                                              cus, stream);
            if (e == hipSuccess) {
                bsfp8::BScale bs_tail = bs;
                bs_tail.ptr = bs.ptr + (cs.n1 / bsfp8::geom::kBlockK) * bs.stride_nb;
                e = bsfp8::launch_gemm(a8, lda, a_s, b8 + cs.n1 * ldb, ldb, bs_tail, c16 + cs.n1, ldc, M, N - cs.n1, K,
                                       false, cs.tail, ws, cus, stream);
            }
            const hipError_t f = (!use_scratch && ws != nullptr) ? hipFreeAsync(ws, stream) : hipSuccess;
            return finish(e != hipSuccess ? e : f);
        }
    }
    if (use_scratch) {
        if (plan.bytes > bsfp8::gemm_scratch_bytes()) return BSFP8_ESCRATCH;
        float* ws = nullptr;
        if (plan.S > 1 && bsfp8::gemm_scratch(&ws) != hipSuccess) return BSFP8_EHIP;
        return finish(bsfp8::launch_gemm(static_cast<const uint8_t*>(a), lda, a_s, static_cast<const uint8_t*>(b),
                                         ldb, bs, static_cast<uint16_t*>(c), ldc, M, N, K, fnuz, plan, ws, cus,
                                         stream));
    }
    float* ws = nullptr;
    if (plan.S > 1) {
        hipMemPool_t pool = nullptr;
        if (device_pool(&pool) != hipSuccess) return BSFP8_EHIP;
        if (hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(plan.bytes), pool, stream) !=
            hipSuccess)
            return BSFP8_EHIP;
    }
    const hipError_t e = bsfp8::launch_gemm(static_cast<const uint8_t*>(a), lda, a_s, static_cast<const uint8_t*>(b),
                                            ldb, bs, static_cast<uint16_t*>(c), ldc, M, N, K, fnuz, plan, ws,
                                            cus, stream);
    const hipError_t f = ws != nullptr ? hipFreeAsync(ws, stream) : hipSuccess;
    return finish(e != hipSuccess ? e : f);
}

// BSFP8_QUANT_LHS_STRIP (environment, read at each call): 1, 2, 4, 8 or 16 runs quantize_lhs in
// row strips of that many 16-byte pieces per thread wherever the alignment allows, 0 always in
// tiles, so tests and benchmarks can compare the variants. Unset or empty: automatic.
int env_lhs_strip() {
    const char* v = std::getenv("BSFP8_QUANT_LHS_STRIP");
    if (v == nullptr || *v == 0) return 0;
    const long n = std::strtol(v, nullptr, 10);
    return n == 1 || n == 2 || n == 4 || n == 8 || n == 16 ? static_cast<int>(n) : -1;
}

int quantize_lhs_impl(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq,
                      float* a_s, bool fnuz, void* stream) {
    if (M < 0 || K < 0) return BSFP8_EINVAL;
    if (M == 0 || K == 0) return BSFP8_OK;
    if (x == nullptr || q == nullptr || a_s == nullptr) return BSFP8_EINVAL;
    if (ldx < K || ldq < K) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_lhs(static_cast<const uint16_t*>(x), M, K, ldx,
                                             static_cast<uint8_t*>(q), ldq, a_s, fnuz, env_lhs_strip(),
                                             static_cast<hipStream_t>(stream)));
}

int quantize_rhs_impl(const void* x, int64_t K, int64_t N, int64_t ldx, void* qT, int64_t ldqT,
                      float* s, bool fnuz, void* stream) {
    if (K < 0 || N < 0) return BSFP8_EINVAL;
    if (K == 0 || N == 0) return BSFP8_OK;
    if (x == nullptr || qT == nullptr || s == nullptr) return BSFP8_EINVAL;
    if (ldx < N || ldqT < K) return BSFP8_EINVAL;
    if (cdiv(K, kGroupEdge) > kMaxGridY) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_rhs(static_cast<const uint16_t*>(x), K, N, ldx,
                                             static_cast<uint8_t*>(qT), ldqT, s, fnuz,
                                             static_cast<hipStream_t>(stream)));
}

int quantize_rhs_grouped_impl(const void* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets, int64_t E,
                              void* qT, int64_t ldqT, float* s, int64_t* padded, bool fnuz, void* stream) {
    if (T < 0 || N < 0 || E < 0) return BSFP8_EINVAL;
    if (offsets == nullptr || padded == nullptr) return BSFP8_EINVAL;
    const int64_t groups = cdiv(T, kGroupEdge) + E;  // bound on the padded groups
    if (groups > kMaxGridY || cdiv(N, 64) > 0x7FFFFFFFLL) return BSFP8_EINVAL;
    if (T > 0 && N > 0) {
        if (x == nullptr || qT == nullptr || s == nullptr) return BSFP8_EINVAL;
        if (ldx < N || ldqT < groups * kGroupEdge) return BSFP8_EINVAL;
    }
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_rhs_grouped(static_cast<const uint16_t*>(x), T, N, ldx, offsets, E,
                                                     static_cast<uint8_t*>(qT), ldqT, s, padded, fnuz,
                                                     static_cast<hipStream_t>(stream)));
}

int quantize_weight_impl(const void* w, int64_t N, int64_t K, int64_t ldw, void* q, int64_t ldq,
                         void* qT, int64_t ldqT, float* s, bool fnuz, void* stream) {
    if (N < 0 || K < 0) return BSFP8_EINVAL;
    if (N == 0 || K == 0) return BSFP8_OK;
    if (w == nullptr || q == nullptr || s == nullptr) return BSFP8_EINVAL;
    if (ldw < K || ldq < K || (qT != nullptr && ldqT < N)) return BSFP8_EINVAL;
    if (cdiv(N, kGroupEdge) > kMaxGridY) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_weight(static_cast<const uint16_t*>(w), N, K, ldw,
                                                static_cast<uint8_t*>(q), ldq,
                                                static_cast<uint8_t*>(qT), ldqT, s, fnuz,
                                                static_cast<hipStream_t>(stream)));
}

int quantize_dual_impl(const void* x, int64_t R, int64_t C, int64_t ldx, void* q, int64_t ldq,
                       float* a_s, void* qT, int64_t ldqT, float* s, bool fnuz, void* stream) {
    if (R < 0 || C < 0) return BSFP8_EINVAL;
    if (R == 0 || C == 0) return BSFP8_OK;
    if (x == nullptr || q == nullptr || a_s == nullptr || qT == nullptr || s == nullptr) return BSFP8_EINVAL;
    if (ldx < C || ldq < C || ldqT < R) return BSFP8_EINVAL;
    if (cdiv(R, kGroupEdge) > kMaxGridY || cdiv(C, kGroupEdge) > 0x7FFFFFFFLL) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_dual(static_cast<const uint16_t*>(x), R, C, ldx,
                                              static_cast<uint8_t*>(q), ldq, a_s,
                                              static_cast<uint8_t*>(qT), ldqT, s, fnuz,
                                              static_cast<hipStream_t>(stream)));
}

int quantize_step_impl(const void* x, int64_t M, int64_t K, int64_t ldx, void* qx, int64_t ldqx,
                       float* sx, const void* w, int64_t N, int64_t Kw, int64_t ldw, void* qw,
                       int64_t ldqw, void* qwT, int64_t ldqwT, float* sw, bool fnuz, void* stream) {
    if (M < 0 || K < 0 || N < 0 || Kw < 0) return BSFP8_EINVAL;
    const bool x_empty = M == 0 || K == 0, w_empty = N == 0 || Kw == 0;
    if (!x_empty && (x == nullptr || qx == nullptr || sx == nullptr || ldx < K || ldqx < K)) return BSFP8_EINVAL;
    if (!w_empty && (w == nullptr || qw == nullptr || sw == nullptr || ldw < Kw || ldqw < Kw ||
                     (qwT != nullptr && ldqwT < N)))
        return BSFP8_EINVAL;
    if (x_empty && w_empty) return BSFP8_OK;
    if (x_empty) return quantize_weight_impl(w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, fnuz, stream);
    if (w_empty) return quantize_lhs_impl(x, M, K, ldx, qx, ldqx, sx, fnuz, stream);
    if (cdiv(M, kGroupEdge) * cdiv(K, kGroupEdge) + cdiv(N, kGroupEdge) * cdiv(Kw, kGroupEdge) > 0x7FFFFFFFLL)
        return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_quantize_step(
        static_cast<const uint16_t*>(x), M, K, ldx, static_cast<uint8_t*>(qx), ldqx, sx,
        static_cast<const uint16_t*>(w), N, Kw, ldw, static_cast<uint8_t*>(qw), ldqw,
        static_cast<uint8_t*>(qwT), ldqwT, sw, fnuz, static_cast<hipStream_t>(stream)));
}

// Floats a strided 128x128 scale tensor spans (the largest index read, plus one).
int64_t bscale_extent(int64_t N, int64_t K, int64_t bs_nb, int64_t bs_kb) {
    return (cdiv(N, kGroupEdge) - 1) * bs_nb + (cdiv(K, kGroupEdge) - 1) * bs_kb + 1;
}

int gemm_128x128_impl(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                      const float* b_s, int64_t bs_stride_nb, int64_t bs_stride_kb, void* c,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, bool fnuz, void* stream,
                      bool use_scratch = false) {
    if (int rc = validate_gemm(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K)) return rc;
    if (M == 0 || N == 0) return BSFP8_OK;
    if (bs_stride_nb < 0 || bs_stride_kb < 0) return BSFP8_EINVAL;
    if (K > 0 && 4 * bscale_extent(N, K, bs_stride_nb, bs_stride_kb) > kMaxRange) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    bsfp8::BScale bs{b_s, bs_stride_nb, bs_stride_kb, 0};
    return run_gemm(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, fnuz, use_scratch, static_cast<hipStream_t>(stream));
}

int gemm_128x1_impl(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                    const float* b_s, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                    bool fnuz, void* stream, bool use_scratch = false) {
    if (int rc = validate_gemm(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K)) return rc;
    if (M == 0 || N == 0) return BSFP8_OK;
    if (4 * N * cdiv(K, kGroupEdge) > kMaxRange) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    bsfp8::BScale bs{b_s, 0, 0, 1};
    return run_gemm(a, lda, a_s, b, ldb, bs, c, ldc, M, N, K, fnuz, use_scratch, static_cast<hipStream_t>(stream));
}

int encode_impl(const float* x, void* q, int64_t n, bool fnuz, void* stream) {
    if (n < 0) return BSFP8_EINVAL;
    if (n == 0) return BSFP8_OK;
    if (x == nullptr || q == nullptr) return BSFP8_EINVAL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 3) != 0) return BSFP8_EALIGN;
    if ((n + 1023) / 1024 > 0x7FFFFFFFLL) return BSFP8_EINVAL;
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_encode(x, static_cast<uint8_t*>(q), n, fnuz,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* bsfp8_status_string(int status) {
    switch (status) {
        case BSFP8_OK: return "ok";
        case BSFP8_EINVAL: return "invalid argument";
        case BSFP8_EALIGN: return "operand rows not 16-byte aligned";
        case BSFP8_EDEVICE: return "current device is not gfx950";
        case BSFP8_EHIP: return "HIP call or kernel launch failed";
        case BSFP8_ESCRATCH: return "the K-split workspace exceeds the allocation-free scratch";
        default: return "unknown status";
    }
}

int quantize_lhs(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq,
                 float* a_s, void* stream) {
    return quantize_lhs_impl(x, M, K, ldx, q, ldq, a_s, false, stream);
}

int quantize_lhs_fnuz(const void* x, int64_t M, int64_t K, int64_t ldx, void* q, int64_t ldq,
                      float* a_s, void* stream) {
    return quantize_lhs_impl(x, M, K, ldx, q, ldq, a_s, true, stream);
}

int quantize_rhs(const void* x, int64_t K, int64_t N, int64_t ldx, void* qT, int64_t ldqT,
                 float* s, void* stream) {
    return quantize_rhs_impl(x, K, N, ldx, qT, ldqT, s, false, stream);
}

int quantize_rhs_fnuz(const void* x, int64_t K, int64_t N, int64_t ldx, void* qT, int64_t ldqT,
                      float* s, void* stream) {
    return quantize_rhs_impl(x, K, N, ldx, qT, ldqT, s, true, stream);
}

int quantize_weight_128x128(const void* w, int64_t N, int64_t K, int64_t ldw, void* q,
                            int64_t ldq, void* qT, int64_t ldqT, float* s, void* stream) {
    return quantize_weight_impl(w, N, K, ldw, q, ldq, qT, ldqT, s, false, stream);
}

int quantize_weight_128x128_fnuz(const void* w, int64_t N, int64_t K, int64_t ldw, void* q,
                                 int64_t ldq, void* qT, int64_t ldqT, float* s, void* stream) {
    return quantize_weight_impl(w, N, K, ldw, q, ldq, qT, ldqT, s, true, stream);
}

int gemm_1x128_128x128(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                       const float* b_s, int64_t bs_stride_nb, int64_t bs_stride_kb, void* c,
                       int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_128x128_impl(a, lda, a_s, b, ldb, b_s, bs_stride_nb, bs_stride_kb, c, ldc, M, N, K,
                             false, stream);
}

int gemm_1x128_128x128_noalloc(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                               const float* b_s, int64_t bs_stride_nb, int64_t bs_stride_kb, void* c,
                               int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
    return gemm_128x128_impl(a, lda, a_s, b, ldb, b_s, bs_stride_nb, bs_stride_kb, c, ldc, M, N, K,
                             false, stream, true);
}

int gemm_1x128_128x128_fnuz(const void* a, int64_t lda, const float* a_s, const void* b,
                            int64_t ldb, const float* b_s, int64_t bs_stride_nb,
                            int64_t bs_stride_kb, void* c, int64_t ldc, int64_t M, int64_t N,
                            int64_t K, void* stream) {
    return gemm_128x128_impl(a, lda, a_s, b, ldb, b_s, bs_stride_nb, bs_stride_kb, c, ldc, M, N, K,
                             true, stream);
}

int gemm_1x128_128x1(const void* a, int64_t lda, const float* a_s, const void* b, int64_t ldb,
                     const float* b_s, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                     void* stream) {
    return gemm_128x1_impl(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K, false, stream);
}

int gemm_1x128_128x1_fnuz(const void* a, int64_t lda, const float* a_s, const void* b,
                          int64_t ldb, const float* b_s, void* c, int64_t ldc, int64_t M,
                          int64_t N, int64_t K, void* stream) {
    return gemm_128x1_impl(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K, true, stream);
}

int quantize_lhs_and_rhs(const void* x, int64_t R, int64_t C, int64_t ldx, void* q, int64_t ldq,
                         float* a_s, void* qT, int64_t ldqT, float* s, void* stream) {
    return quantize_dual_impl(x, R, C, ldx, q, ldq, a_s, qT, ldqT, s, false, stream);
}

int quantize_lhs_and_rhs_fnuz(const void* x, int64_t R, int64_t C, int64_t ldx, void* q,
                              int64_t ldq, float* a_s, void* qT, int64_t ldqT, float* s,
                              void* stream) {
    return quantize_dual_impl(x, R, C, ldx, q, ldq, a_s, qT, ldqT, s, true, stream);
}

int quantize_rhs_grouped(const void* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets, int64_t E,
                         void* qT, int64_t ldqT, float* s, int64_t* padded_offsets, void* stream) {
    return quantize_rhs_grouped_impl(x, T, N, ldx, offsets, E, qT, ldqT, s, padded_offsets, false, stream);
}

int quantize_rhs_grouped_fnuz(const void* x, int64_t T, int64_t N, int64_t ldx, const int64_t* offsets,
                              int64_t E, void* qT, int64_t ldqT, float* s, int64_t* padded_offsets,
                              void* stream) {
    return quantize_rhs_grouped_impl(x, T, N, ldx, offsets, E, qT, ldqT, s, padded_offsets, true, stream);
}

int gemm_1x128_128x128_grouped(const void* a, int64_t lda, const float* a_s, const void* b,
                               int64_t ldb, int64_t b_stride, const float* b_s, int64_t bs_stride,
                               int64_t bs_stride_nb, int64_t bs_stride_kb, const int64_t* offsets,
                               int64_t E, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               void* stream) {
    if (E < 0 || K < 0) return BSFP8_EINVAL;
    if (E == 0 || M == 0 || N == 0) return M < 0 || N < 0 ? BSFP8_EINVAL : BSFP8_OK;
    if (K == 0 || K % kGroupEdge != 0) return BSFP8_EINVAL;
    if (int rc = validate_gemm(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K)) return rc;
    if (offsets == nullptr || b_stride < 0 || bs_stride < 0 || bs_stride_nb < 0 || bs_stride_kb < 0)
        return BSFP8_EINVAL;
    if (4 * bscale_extent(N, K, bs_stride_nb, bs_stride_kb) > kMaxRange) return BSFP8_EINVAL;
    if (b_stride % 16 != 0) return BSFP8_EALIGN;
    if (int rc = check_device()) return rc;
    bsfp8::BScale bs{b_s, bs_stride_nb, bs_stride_kb, 0};
    return finish(bsfp8::launch_gemm_grouped_rows(
        static_cast<const uint8_t*>(a), lda, a_s, static_cast<const uint8_t*>(b), ldb, b_stride, bs,
        bs_stride, offsets, E, static_cast<uint16_t*>(c), ldc, M, N, K,
        static_cast<hipStream_t>(stream)));
}

int gemm_1x128_128x1_grouped(const void* a, int64_t lda, const float* a_s, const void* b,
                             int64_t ldb, const float* b_s, const int64_t* offsets, int64_t E,
                             void* c, int64_t ldc, int64_t c_stride, int64_t M, int64_t N,
                             int64_t K, int32_t* status, void* stream) {
    if (E < 0 || K < 0) return BSFP8_EINVAL;
    if (E == 0 || M == 0 || N == 0) return M < 0 || N < 0 ? BSFP8_EINVAL : BSFP8_OK;
    if (K == 0 || K % kGroupEdge != 0 || E > 65535) return BSFP8_EINVAL;
    if (int rc = validate_gemm(a, lda, a_s, b, ldb, b_s, c, ldc, M, N, K)) return rc;
    if (4 * N * cdiv(K, kGroupEdge) > kMaxRange) return BSFP8_EINVAL;
    if (offsets == nullptr) return BSFP8_EINVAL;
    if (E > 1 && c_stride < (M - 1) * ldc + N) return BSFP8_EINVAL;  // expert outputs must not overlap
    if (int rc = check_device()) return rc;
    return finish(bsfp8::launch_gemm_grouped_k(
        static_cast<const uint8_t*>(a), lda, a_s, static_cast<const uint8_t*>(b), ldb, b_s, offsets,
        E, static_cast<uint16_t*>(c), ldc, c_stride, M, N, K, status, static_cast<hipStream_t>(stream)));
}

int quantize_lhs_and_weight(const void* x, int64_t M, int64_t K, int64_t ldx, void* qx, int64_t ldqx,
                            float* sx, const void* w, int64_t N, int64_t Kw, int64_t ldw, void* qw,
                            int64_t ldqw, void* qwT, int64_t ldqwT, float* sw, void* stream) {
    return quantize_step_impl(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, false,
                              stream);
}

int quantize_lhs_and_weight_fnuz(const void* x, int64_t M, int64_t K, int64_t ldx, void* qx,
                                 int64_t ldqx, float* sx, const void* w, int64_t N, int64_t Kw,
                                 int64_t ldw, void* qw, int64_t ldqw, void* qwT, int64_t ldqwT,
                                 float* sw, void* stream) {
    return quantize_step_impl(x, M, K, ldx, qx, ldqx, sx, w, N, Kw, ldw, qw, ldqw, qwT, ldqwT, sw, true,
                              stream);
}

int encode_e4m3_f32(const float* x, void* q, int64_t n, void* stream) {
    return encode_impl(x, q, n, false, stream);
}

int encode_e4m3fnuz_f32(const float* x, void* q, int64_t n, void* stream) {
    return encode_impl(x, q, n, true, stream);
}

}  // extern "C"
