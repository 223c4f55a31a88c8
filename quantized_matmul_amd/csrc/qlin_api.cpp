// qlin_api.cpp -- the C ABI of libqlin: argument validation and kernel
// dispatch. Every argument is checked on the host before anything is
// launched, so a rejected call has no device side effects (the pages ask for
// a clear error before the backend is touched: "Emily.QuantizedWeight",
// Microscaled modes section).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/qlin.h"
#include "qlin_common.h"

namespace qlin {

DeviceShape device_shape() {
    // one entry per device id; a racing first call on one device at worst
    // queries twice and stores the same values
    static std::atomic<int> cus[64], xcds[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceShape{256, 8};
    int c = cus[dev].load(std::memory_order_acquire);
    int x = xcds[dev].load(std::memory_order_acquire);
    if (c <= 0 || x <= 0) {
        c = 0;
        x = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
            c = 256;
        if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0) x = 1;
        xcds[dev].store(x, std::memory_order_release);
        cus[dev].store(c, std::memory_order_release);
    }
    return DeviceShape{c, x};
}

bool debug_lds_nan() {
    const char* e = getenv("QLIN_DEBUG_LDS_NAN");
    return e && e[0] == '1' && e[1] == 0;
}

// [in, out] layout with a caller's workspace (K split over workgroups)
size_t qmm_nt_split_workspace_bytes(const QmmArgs& q);
hipError_t launch_qmm_nt_split(const QmmArgs& q, void* workspace, hipStream_t st);
}  // namespace qlin

namespace {

thread_local std::string g_last_error;
// kernel path of the calling thread's last successful matmul-type call
thread_local const char* g_last_path = "";

// The generic kernel is the fp32 VALU fallback for shapes the fast kernels
// refuse; it can be 10-15x slower. QLIN_WARN_FALLBACK=1 prints one line to
// stderr each time it runs.
void note_path(const char* p) {
    g_last_path = p;
    if (!strcmp(p, "generic")) {
        const char* e = getenv("QLIN_WARN_FALLBACK");
        if (e && e[0] == '1' && e[1] == 0)
            fprintf(stderr, "libqlin: this shape runs on the generic fp32 VALU kernel (slow path)\n");
    }
}

qlin_status fail(qlin_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

// qqmm in mxfp8 takes the scaled fp8 MFMA kernel from this many rows of x
// (below it the weight stream bounds the time and the exact bf16 decode
// kernels serve).
constexpr int64_t kQqmmScaledMinRows = 32;

qlin_status ok() {
    g_last_error.clear();
    return QLIN_OK;
}

qlin_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(QLIN_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool is_float_dtype(int d) { return d == QLIN_F32 || d == QLIN_F16 || d == QLIN_BF16; }

// Parse the mode string and check (group_size, bits) against it and against
// the quantized axis length.
qlin_status check_mode(const char* mode, int group_size, int bits, int64_t qaxis, int* mode_out) {
    if (!mode) return fail(QLIN_ERR_INVALID_ARGUMENT, "mode is NULL");
    int m;
    if (!strcmp(mode, "affine")) m = qlin::AFFINE;
    else if (!strcmp(mode, "mxfp4")) m = qlin::MXFP4;
    else if (!strcmp(mode, "mxfp8")) m = qlin::MXFP8;
    else if (!strcmp(mode, "nvfp4")) m = qlin::NVFP4;
    else return fail(QLIN_ERR_INVALID_ARGUMENT, "unknown mode \"%s\" (affine, mxfp4, mxfp8, nvfp4)", mode);
    if (m == qlin::AFFINE) {
        if (bits != 2 && bits != 4 && bits != 8)
            return fail(QLIN_ERR_INVALID_ARGUMENT, "affine bits must be 2, 4 or 8 (got %d)", bits);
        if (group_size != 32 && group_size != 64 && group_size != 128)
            return fail(QLIN_ERR_INVALID_ARGUMENT, "affine group_size must be 32, 64 or 128 (got %d)",
                        group_size);
    } else {
        const int g = (m == qlin::NVFP4) ? 16 : 32, b = (m == qlin::MXFP8) ? 8 : 4;
        if (group_size != g || bits != b)
            return fail(QLIN_ERR_INVALID_ARGUMENT,
                        "mode %s requires group_size %d and bits %d (got %d and %d)", mode, g, b,
                        group_size, bits);
    }
    if (qaxis <= 0 || qaxis % group_size != 0)
        return fail(QLIN_ERR_INVALID_ARGUMENT,
                    "quantized axis length %lld must be a positive multiple of group_size %d",
                    (long long)qaxis, group_size);
    *mode_out = m;
    return QLIN_OK;
}

qlin_status check_scale_dtype(int mode, int scale_dtype, const void* biases) {
    if (mode == qlin::AFFINE) {
        if (!is_float_dtype(scale_dtype))
            return fail(QLIN_ERR_INVALID_ARGUMENT, "affine scales must be f32, f16 or bf16");
        if (!biases) return fail(QLIN_ERR_INVALID_ARGUMENT, "affine mode needs biases");
    } else {
        if (scale_dtype != QLIN_U8)
            return fail(QLIN_ERR_INVALID_ARGUMENT, "microscaled scales are uint8 bytes");
        if (biases) return fail(QLIN_ERR_INVALID_ARGUMENT, "microscaled modes take no biases");
    }
    return QLIN_OK;
}

// Kernel path override for tests of each code path ("generic", "decode",
// "tiled", "prefill", "prefill2", "split", "scaled"); unset means automatic
// choice.
int forced_path() {
    const char* e = getenv("QLIN_FORCE_PATH");
    if (!e || !*e) return 0;
    if (!strcmp(e, "generic")) return 1;
    if (!strcmp(e, "decode")) return 2;
    if (!strcmp(e, "tiled")) return 3;
    if (!strcmp(e, "prefill")) return 4;
    if (!strcmp(e, "split")) return 5;
    if (!strcmp(e, "scaled")) return 7;
    if (!strcmp(e, "prefill2")) return 8;
    return 0;
}

// QLIN_CHECK_INDICES=1: before any gather kernel, one small kernel looks for
// an index row whose expert is >= E or whose batch entry is >= B; the host
// waits for it and fails the call with that row. The indices are otherwise a
// precondition (the kernels then only keep their own accesses in range). The
// wait cannot happen under HIP graph capture, so the check refuses to run there.
bool index_check_enabled() {
    const char* e = getenv("QLIN_CHECK_INDICES");
    return e && e[0] == '1' && e[1] == 0;
}

qlin_status check_indices_if_asked(const uint32_t* rhs, const uint32_t* lhs, int64_t R, int64_t E,
                                   int64_t B, void* workspace, hipStream_t s) {
    if (!index_check_enabled()) return QLIN_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cs);
    if (e != hipSuccess) return device_status(e, "gather_qmm (index check)");
    if (cs != hipStreamCaptureStatusNone)
        return fail(QLIN_ERR_UNSUPPORTED,
                    "QLIN_CHECK_INDICES=1 waits for the device and cannot run under graph capture");
    uint32_t* res = qlin::index_check_result(workspace, R, E);
    if ((e = qlin::launch_check_indices(rhs, lhs, R, E, B, res, s)) != hipSuccess)
        return device_status(e, "gather_qmm (index check)");
    uint32_t h[3] = {0, 0, 0};
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return device_status(e, "gather_qmm (index check)");
    if ((e = hipMemcpy(h, res, sizeof h, hipMemcpyDeviceToHost)) != hipSuccess)
        return device_status(e, "gather_qmm (index check)");
    if (h[0] != 0xFFFFFFFFu) {
        if (h[1] >= (uint64_t)E)
            return fail(QLIN_ERR_INVALID_ARGUMENT, "rhs_indices[%u] = %u is not below E = %lld",
                        h[0], h[1], (long long)E);
        return fail(QLIN_ERR_INVALID_ARGUMENT, "%s[%u] = %u is not below B = %lld",
                    lhs ? "lhs_indices" : "index row", h[0], h[2], (long long)B);
    }
    return QLIN_OK;
}

qlin_status run_qmm(const qlin::QmmArgs& a, const uint32_t* perm, const uint32_t* offsets,
                    hipStream_t st, void* ws = nullptr, size_t ws_bytes = 0) {
    const int force = forced_path();
    if (a.R == 0 && (force == 0 || force == 2) && qlin::qmm_decode_supports(a)) {
        note_path("decode");
        return device_status(qlin::launch_qmm_decode(a, st), "quantized_matmul (decode kernel)");
    }
    if (a.R == 0 && ws && (force == 0 || force == 5)) {
        const size_t need = qlin::qmm_nt_split_workspace_bytes(a);
        if (need > 0 && ws_bytes >= need) {
            note_path("in_out_split");
            return device_status(qlin::launch_qmm_nt_split(a, ws, st),
                                 "quantized_matmul ([in,out] K-split kernel)");
        }
    }
    if (force == 5) return fail(QLIN_ERR_UNSUPPORTED, "K-split kernel does not take this shape or workspace");
    if (a.R == 0 && (force == 0 || force == 2) && qlin::qmm_nt_supports(a)) {
        note_path("in_out");
        return device_status(qlin::launch_qmm_nt(a, st), "quantized_matmul ([in,out] kernel)");
    }
    // [in,out] layout with 9..128 rows: the few-row kernel over blocks of 8
    // rows (each block streams W once; M16 at N = K = 8192 mxfp4 takes 2 x 35
    // us instead of 1.5 ms in the generic kernel)
    if (a.R == 0 && (force == 0 || force == 2) && !a.transpose && a.M > 8 && a.M <= 128 &&
        a.x_dtype == QLIN_BF16) {
        qlin::QmmArgs c = a;
        c.M = 8;
        if (qlin::qmm_nt_supports(c)) {
            note_path("in_out_row_blocks");
            for (int64_t m0 = 0; m0 < a.M; m0 += 8) {
                c.M = a.M - m0 < 8 ? a.M - m0 : 8;
                c.x = (const char*)a.x + m0 * a.K * 2;
                c.y = (char*)a.y + m0 * a.N * 2;
                const qlin_status r = device_status(qlin::launch_qmm_nt(c, st),
                                                    "quantized_matmul ([in,out] kernel, row blocks)");
                if (r != QLIN_OK) return r;
            }
            return QLIN_OK;
        }
    }
    if (force == 2) return fail(QLIN_ERR_UNSUPPORTED, "decode kernel does not take this shape");
    if (a.R == 0 && force == 8 && qlin::qmm_prefill2_supports(a)) {
        note_path("prefill2");
        return device_status(qlin::launch_qmm_prefill2(a, st),
                             "quantized_matmul (pipelined 4-bit prefill kernel)");
    }
    if (force == 8) return fail(QLIN_ERR_UNSUPPORTED, "pipelined 4-bit prefill kernel does not take this shape");
    if ((force == 0 || force == 4) && qlin::qmm_prefill_supports(a)) {
        note_path(a.R ? "gather_prefill" : "prefill");
        return device_status(qlin::launch_qmm_prefill(a, perm, offsets, st),
                             a.R ? "gather_qmm (many-row kernel)" : "quantized_matmul (prefill kernel)");
    }
    if (force == 4) return fail(QLIN_ERR_UNSUPPORTED, "prefill kernel does not take this shape");
    if ((force == 0 || force == 3) && qlin::qmm_tiled_supports(a)) {
        note_path("tiled");
        return device_status(qlin::launch_qmm_tiled(a, perm, offsets, st),
                             "quantized_matmul (tiled kernel)");
    }
    if (force == 3) return fail(QLIN_ERR_UNSUPPORTED, "tiled kernel does not take this shape");
    note_path("generic");
    return device_status(qlin::launch_qmm_generic(a, st), "quantized_matmul (generic kernel)");
}

}  // namespace

extern "C" {

const char* qlin_last_error(void) { return g_last_error.c_str(); }

const char* qlin_last_path(void) { return g_last_path; }

qlin_status qlin_quantize(const void* w, qlin_dtype w_dtype, int64_t rows, int64_t cols,
                          int group_size, int bits, const char* mode, uint32_t* wq, void* scales,
                          void* biases, void* stream) {
    int m;
    qlin_status st = check_mode(mode, group_size, bits, cols, &m);
    if (st) return st;
    if (!is_float_dtype(w_dtype)) return fail(QLIN_ERR_INVALID_ARGUMENT, "w must be f32, f16 or bf16");
    if (rows < 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "rows must be >= 0");
    if (m == qlin::AFFINE && !biases) return fail(QLIN_ERR_INVALID_ARGUMENT, "affine mode needs biases");
    if (m != qlin::AFFINE && biases)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "microscaled modes take no biases (pass NULL)");
    if (rows == 0) return ok();
    if (!w || !wq || !scales) return fail(QLIN_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    return device_status(qlin::launch_quantize(w, w_dtype, rows, cols, group_size, bits, m, wq,
                                               scales, biases, (hipStream_t)stream),
                         "quantize");
}

qlin_status qlin_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                            qlin_dtype scale_dtype, int64_t rows, int64_t cols, int group_size,
                            int bits, const char* mode, void* out, qlin_dtype out_dtype,
                            void* stream) {
    int m;
    qlin_status st = check_mode(mode, group_size, bits, cols, &m);
    if (st) return st;
    if ((st = check_scale_dtype(m, scale_dtype, biases))) return st;
    if (!is_float_dtype(out_dtype)) return fail(QLIN_ERR_INVALID_ARGUMENT, "out must be f32, f16 or bf16");
    if (rows < 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "rows must be >= 0");
    if (rows == 0) return ok();
    if (!wq || !scales || !out) return fail(QLIN_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    return device_status(qlin::launch_dequantize(wq, scales, biases, scale_dtype, rows, cols,
                                                 group_size, bits, m, out, out_dtype,
                                                 (hipStream_t)stream),
                         "dequantize");
}

}  // extern "C"

namespace {

// Shared by quantized_matmul and quantized_dense: checks, then the kernel
// that takes the shape, with the dense layer's bias in its output stage.
qlin_status qmm_entry(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                      const void* scales, const void* biases, qlin_dtype scale_dtype, int64_t N,
                      int transpose, int group_size, int bits, const char* mode,
                      const qlin::OutBias& ob, void* y, void* stream, void* ws = nullptr,
                      size_t ws_bytes = 0) {
    int m;
    if (N <= 0 || K <= 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "N and K must be positive");
    qlin_status st = check_mode(mode, group_size, bits, transpose ? K : N, &m);
    if (st) return st;
    if ((st = check_scale_dtype(m, scale_dtype, biases))) return st;
    if (!is_float_dtype(x_dtype)) return fail(QLIN_ERR_INVALID_ARGUMENT, "x must be f32, f16 or bf16");
    if (m == qlin::AFFINE && scale_dtype != x_dtype)
        return fail(QLIN_ERR_INVALID_ARGUMENT,
                    "affine output follows the scales dtype: x and scales must share a dtype");
    if (M < 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "M must be >= 0");
    if (M == 0) return ok();
    if (!x || !wq || !scales || !y) return fail(QLIN_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    if (M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31))
        return fail(QLIN_ERR_UNSUPPORTED, "dimensions above 2^31 are not supported");
    if (ws && ((uintptr_t)ws & 15) != 0)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    qlin::QmmArgs a{};
    a.x = x;
    a.wq = wq;
    a.scales = scales;
    a.biases = biases;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.x_dtype = x_dtype;
    a.scale_dtype = scale_dtype;
    a.transpose = transpose ? 1 : 0;
    a.group_size = group_size;
    a.bits = bits;
    a.mode = m;
    a.ob = ob;
    return run_qmm(a, nullptr, nullptr, (hipStream_t)stream, ws, ws ? ws_bytes : 0);
}

}  // namespace

extern "C" {

qlin_status qlin_quantized_matmul(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                  const uint32_t* wq, const void* scales, const void* biases,
                                  qlin_dtype scale_dtype, int64_t N, int transpose, int group_size,
                                  int bits, const char* mode, void* y, void* stream) {
    const qlin::OutBias none{nullptr, 0.f, qlin::OB_NONE, QLIN_F32};
    return qmm_entry(x, x_dtype, M, K, wq, scales, biases, scale_dtype, N, transpose, group_size,
                     bits, mode, none, y, stream);
}

size_t qlin_quantized_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N, int transpose,
                                             int group_size, int bits, const char* mode) {
    int m;
    if (M < 1 || N <= 0 || K <= 0) return 0;
    if (check_mode(mode, group_size, bits, transpose ? K : N, &m) != QLIN_OK) return 0;
    if (M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31)) return 0;
    qlin::QmmArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.x_dtype = QLIN_BF16;
    a.scale_dtype = m == qlin::AFFINE ? QLIN_BF16 : QLIN_U8;
    a.transpose = transpose ? 1 : 0;
    a.group_size = group_size;
    a.bits = bits;
    a.mode = m;
    return qlin::qmm_nt_split_workspace_bytes(a);
}

qlin_status qlin_quantized_matmul_ws(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                     const uint32_t* wq, const void* scales, const void* biases,
                                     qlin_dtype scale_dtype, int64_t N, int transpose,
                                     int group_size, int bits, const char* mode, void* workspace,
                                     size_t workspace_bytes, void* y, void* stream) {
    const qlin::OutBias none{nullptr, 0.f, qlin::OB_NONE, QLIN_F32};
    return qmm_entry(x, x_dtype, M, K, wq, scales, biases, scale_dtype, N, transpose, group_size,
                     bits, mode, none, y, stream, workspace, workspace_bytes);
}

qlin_status qlin_quantized_dense(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                 const uint32_t* wq, const void* scales, const void* biases,
                                 qlin_dtype scale_dtype, int64_t N, int transpose, int group_size,
                                 int bits, const char* mode, const void* bias, qlin_dtype bias_dtype,
                                 double bias_value, void* y, void* stream) {
    qlin::OutBias ob{nullptr, 0.f, qlin::OB_NONE, QLIN_F32};
    if (bias) {
        if (!is_float_dtype(bias_dtype))
            return fail(QLIN_ERR_INVALID_ARGUMENT, "bias must be f32, f16 or bf16");
        const uintptr_t align = bias_dtype == QLIN_F32 ? 4 : 2;
        if ((uintptr_t)bias % align)
            return fail(QLIN_ERR_INVALID_ARGUMENT, "bias is not aligned to its element size");
        ob = {bias, 0.f, qlin::OB_COLUMN, (int)bias_dtype};
    } else {
        // the number is taken in fp32, like the accumulation it is added to
        if (!std::isfinite((float)bias_value))
            return fail(QLIN_ERR_INVALID_ARGUMENT, "bias value must be finite in fp32");
        if (bias_value != 0.0) ob = {nullptr, (float)bias_value, qlin::OB_SCALAR, QLIN_F32};
    }
    return qmm_entry(x, x_dtype, M, K, wq, scales, biases, scale_dtype, N, transpose, group_size,
                     bits, mode, ob, y, stream);
}

size_t qlin_qqmm_workspace_bytes(int64_t M, int64_t K) {
    if (M < 0) M = 0;
    if (K < 0) K = 0;
    return (size_t)M * (size_t)K * 2u;   // the decoded bf16 x
}

qlin_status qlin_qqmm(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                      const void* scales, int64_t N, int transpose, int group_size, int bits,
                      const char* mode, void* workspace, size_t workspace_bytes, void* y,
                      void* stream) {
    int m;
    if (N <= 0 || K <= 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "N and K must be positive");
    qlin_status st = check_mode(mode, group_size, bits, transpose ? K : N, &m);
    if (st) return st;
    if (m != qlin::NVFP4 && m != qlin::MXFP8)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "qqmm takes the nvfp4 and mxfp8 modes");
    if (K % group_size != 0)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "x is quantized along K: K must be a multiple of group_size");
    if (x_dtype != QLIN_BF16) return fail(QLIN_ERR_UNSUPPORTED, "qqmm takes bf16 x");
    if (M < 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "M must be >= 0");
    if (M == 0) return ok();
    if (!x || !wq || !scales || !y) return fail(QLIN_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    const size_t need = qlin_qqmm_workspace_bytes(M, K);
    if (!workspace || workspace_bytes < need)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed (got %zu)", need,
                    workspace_bytes);
    if (((uintptr_t)workspace & 15) != 0)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31))
        return fail(QLIN_ERR_UNSUPPORTED, "dimensions above 2^31 are not supported");
    hipStream_t s = (hipStream_t)stream;
    // mxfp8 with enough rows: x's codes and scales are the scaled fp8 MFMA's
    // operands as they are (workspace: M*K code bytes, then M*K/32 scale
    // bytes), so the product runs at the fp8 rate with no decode at all
    const int force = forced_path();
    if (m == qlin::MXFP8 && transpose && (force == 0 || force == 7) && M >= kQqmmScaledMinRows &&
        qlin::qqmm_mx8_supports(M, N, K, wq, scales)) {
        uint8_t* xq = (uint8_t*)workspace;
        uint8_t* xs = xq + M * K;
        hipError_t e = qlin::launch_quantize(x, QLIN_BF16, M, K, group_size, bits, m, (uint32_t*)xq, xs,
                                             nullptr, s);
        if (e != hipSuccess) return device_status(e, "qqmm (activation quantization)");
        note_path("qqmm_scaled_mfma");
        return device_status(qlin::launch_qqmm_mx8(xq, xs, (const uint8_t*)wq, (const uint8_t*)scales,
                                                   (uint16_t*)y, M, N, K, s),
                             "qqmm (scaled fp8 MFMA kernel)");
    }
    if (force == 7) return fail(QLIN_ERR_UNSUPPORTED, "scaled-MFMA qqmm does not take this shape");
    hipError_t e = qlin::launch_qdq_micro(x, M, K, group_size, m, workspace, s);
    if (e != hipSuccess) return device_status(e, "qqmm (activation quantization)");
    qlin::QmmArgs a{};
    a.x = workspace;
    a.wq = wq;
    a.scales = scales;
    a.biases = nullptr;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.x_dtype = QLIN_BF16;
    a.scale_dtype = QLIN_U8;
    a.transpose = transpose ? 1 : 0;
    a.group_size = group_size;
    a.bits = bits;
    a.mode = m;
    return run_qmm(a, nullptr, nullptr, s);
}

size_t qlin_gather_qmm_workspace_bytes(int64_t R, int64_t E) {
    if (R < 0) R = 0;
    if (E < 0) E = 0;
    return qlin::bucket_workspace_bytes(R, E);
}

qlin_status qlin_gather_qmm(const void* x, qlin_dtype x_dtype, int64_t B, int64_t M, int64_t K,
                            const uint32_t* wq, const void* scales, const void* biases,
                            qlin_dtype scale_dtype, int64_t E, int64_t N,
                            const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t R,
                            int transpose, int group_size, int bits, const char* mode,
                            int sorted_indices, void* workspace, size_t workspace_bytes, void* y,
                            void* stream) {
    int m;
    if (N <= 0 || K <= 0 || E <= 0)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "N, K and E must be positive");
    qlin_status st = check_mode(mode, group_size, bits, transpose ? K : N, &m);
    if (st) return st;
    if ((st = check_scale_dtype(m, scale_dtype, biases))) return st;
    if (!is_float_dtype(x_dtype)) return fail(QLIN_ERR_INVALID_ARGUMENT, "x must be f32, f16 or bf16");
    if (m == qlin::AFFINE && scale_dtype != x_dtype)
        return fail(QLIN_ERR_INVALID_ARGUMENT,
                    "affine output follows the scales dtype: x and scales must share a dtype");
    if (R < 0 || M < 0 || B < 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "negative size");
    if (!lhs_indices && B != R)
        return fail(QLIN_ERR_INVALID_ARGUMENT,
                    "without lhs_indices, x must have one batch entry per index row (B == R)");
    if (R == 0 || M == 0) return ok();
    if (B == 0) return fail(QLIN_ERR_INVALID_ARGUMENT, "x has no batch entries");
    if (!x || !wq || !scales || !y || !rhs_indices)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "NULL tensor pointer");
    const size_t need = qlin::bucket_workspace_bytes(R, E);
    if (!workspace || workspace_bytes < need)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "workspace of %zu bytes needed (got %zu)", need,
                    workspace_bytes);
    if (R * M > (1LL << 31) || N > (1LL << 31) || K > (1LL << 31) || E > (1LL << 31))
        return fail(QLIN_ERR_UNSUPPORTED, "dimensions above 2^31 are not supported");
    qlin::QmmArgs a{};
    a.x = x;
    a.wq = wq;
    a.scales = scales;
    a.biases = biases;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.x_dtype = x_dtype;
    a.scale_dtype = scale_dtype;
    a.transpose = transpose ? 1 : 0;
    a.group_size = group_size;
    a.bits = bits;
    a.mode = m;
    a.batch_x = B;
    a.R = R;
    a.E = E;
    a.lhs = lhs_indices;
    a.rhs = rhs_indices;
    hipStream_t s = (hipStream_t)stream;
    if ((st = check_indices_if_asked(rhs_indices, lhs_indices, R, E, B, workspace, s))) return st;
    uint32_t *perm = nullptr, *offsets = nullptr;
    // the MFMA paths read rows bucketed by expert, in tiles of their own size;
    // few rows per expert (decode) take the small-M kernel's gather form
    const int force = forced_path();
    int tile_rows = 0, decode_rows = 0;
    if ((force == 0 || force == 2) && (decode_rows = qlin::qmm_decode_gather_tile_rows(a)) != 0)
        tile_rows = decode_rows;   // -1: no bucketing
    else if (force == 2)
        return fail(QLIN_ERR_UNSUPPORTED, "decode kernel does not take this gather shape");
    else if ((force == 0 || force == 4) && qlin::qmm_prefill_supports(a))
        tile_rows = qlin::prefill_gather_tile_rows(a.R * a.M, a.E);
    else if ((force == 0 || force == 3) && qlin::qmm_tiled_supports(a))
        tile_rows = qlin::kTiledGatherRows;
    if (tile_rows > 0) {
        hipError_t e = qlin::launch_bucket(rhs_indices, R, E, M, sorted_indices, tile_rows,
                                           workspace, &perm, &offsets, s);
        if (e != hipSuccess) return device_status(e, "gather_qmm (expert bucketing)");
    }
    if (decode_rows != 0) {
        note_path("gather_decode");
        return device_status(qlin::launch_qmm_decode_gather(a, perm, offsets, decode_rows, s),
                             "gather_qmm (decode kernel)");
    }
    return run_qmm(a, perm, offsets, s);
}

}  // extern "C"

// ------------------------------------------------------------------------
// gather_qmm without a caller's workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). The bucketing scratch (row permutation,
// expert offsets, row-tile prefix, index-check result) lives in a
// file-scope device array of fixed size; every GPU holds its own copy until
// the process ends. Calls on one GPU share that array: calls that overlap
// in time on one GPU (different streams, or threads) race on it.

namespace {

constexpr int64_t kNoAllocMaxRows = 65536;      // index rows R
constexpr int64_t kNoAllocMaxExperts = 4096;    // experts E
constexpr size_t kScratchBytes =                 // bucket_workspace_bytes(R max, E max)
    (size_t)(2 * (kNoAllocMaxExperts + 1) + kNoAllocMaxRows) * sizeof(uint32_t) + 256;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array, looked up once per device
// with that device current (the array's host-side name is not a device
// address).
qlin_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return device_status(e, "gather_qmm_noalloc (current device)");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QLIN_ERR_UNSUPPORTED, "device ordinal %d above the %d this library tracks", dev,
                    kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return device_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                     "gather_qmm_noalloc (scratch address)");
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QLIN_OK;
}

}  // namespace

extern "C" {

size_t qlin_gather_qmm_noalloc_max_rows(void) { return (size_t)kNoAllocMaxRows; }
size_t qlin_gather_qmm_noalloc_max_experts(void) { return (size_t)kNoAllocMaxExperts; }

qlin_status qlin_gather_qmm_noalloc(const void* x, qlin_dtype x_dtype, int64_t B, int64_t M,
                                    int64_t K, const uint32_t* wq, const void* scales,
                                    const void* biases, qlin_dtype scale_dtype, int64_t E,
                                    int64_t N, const uint32_t* lhs_indices,
                                    const uint32_t* rhs_indices, int64_t R, int transpose,
                                    int group_size, int bits, const char* mode, int sorted_indices,
                                    void* y, void* stream) {
    if (R > kNoAllocMaxRows || E > kNoAllocMaxExperts)
        return fail(QLIN_ERR_INVALID_ARGUMENT,
                    "gather_qmm_noalloc takes at most %lld index rows and %lld experts "
                    "(got %lld and %lld); use qlin_gather_qmm with a workspace",
                    (long long)kNoAllocMaxRows, (long long)kNoAllocMaxExperts, (long long)R,
                    (long long)E);
    if (R < 0 || E <= 0 || qlin::bucket_workspace_bytes(R, E) > kScratchBytes)
        return fail(QLIN_ERR_INVALID_ARGUMENT, "negative size or no experts");
    void* ws = nullptr;   // an empty problem returns before the workspace is looked at
    if (R > 0 && M > 0) {
        qlin_status st = scratch_for_current_device(&ws);
        if (st) return st;
    }
    return qlin_gather_qmm(x, x_dtype, B, M, K, wq, scales, biases, scale_dtype, E, N, lhs_indices,
                           rhs_indices, R, transpose, group_size, bits, mode, sorted_indices, ws,
                           kScratchBytes, y, stream);
}

}  // extern "C"
