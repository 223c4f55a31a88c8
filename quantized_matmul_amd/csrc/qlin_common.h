// qlin_common.h -- device helpers and internal launcher declarations shared by
// the HIP translation units of libqlin (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlin.h"

namespace qlin {

// Compute units and XCDs (accelerator dies, each with its own L2) of the
// current device, queried once per device. Workgroups are dealt to the XCDs
// round-robin, so kernels that share data between neighbouring tiles
// renumber their blocks so that each XCD walks a contiguous run.
struct DeviceShape {
    int cus;
    int xcds;
};
DeviceShape device_shape();

// QLIN_DEBUG_LDS_NAN=1: the LDS-tiled kernels (many-row, pipelined 4-bit,
// scaled fp8) fill their whole LDS with NaN bytes before each tile, so a
// read of LDS that no load or store of the tile wrote -- a missing wait or
// barrier, a wrong index -- turns the output into NaN. Read at each launch.
bool debug_lds_nan();

// Renumbers block b of nblk so that XCD x (= b % xcds) takes the contiguous
// run [x * nblk / xcds, (x + 1) * nblk / xcds); a bijection when xcds divides
// nblk, the identity otherwise.
__device__ __forceinline__ int xcd_block(int b, int nblk, int xcds) {
    if (xcds <= 1 || nblk % xcds != 0) return b;
    return (b % xcds) * (nblk / xcds) + b / xcds;
}

enum Mode : int { AFFINE = 0, MXFP4 = 1, MXFP8 = 2, NVFP4 = 3 };

// ---------------------------------------------------------------- dtype I/O

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;  // exact widening
}

// Nearest-even fp32 -> bf16 bit pattern (inputs are finite or inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32 under the default round-to-nearest-even mode
    return __builtin_bit_cast(uint16_t, h);
}

// Load element i of a float tensor stored as dtype DT.
template <int DT>
__device__ __forceinline__ float load_f(const void* p, int64_t i) {
    if constexpr (DT == QLIN_F32) return ((const float*)p)[i];
    else if constexpr (DT == QLIN_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    else return f16_bits_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_f(void* p, int64_t i, float v) {
    if constexpr (DT == QLIN_F32) ((float*)p)[i] = v;
    else if constexpr (DT == QLIN_BF16) ((uint16_t*)p)[i] = (uint16_t)f32_to_bf16_rne(v);
    else ((uint16_t*)p)[i] = (uint16_t)f32_to_f16_rne(v);
}

// Bias of the dense layer ("Emily.Quantization.Layers", quantized_dense: the
// layer adds a bias, a tensor or a number, to x times W): none, one number for
// every output, or one value per output column (a vector of N elements).
// Added in fp32 to the accumulated output before its single rounding.
enum OutBiasKind : int { OB_NONE = 0, OB_SCALAR = 1, OB_COLUMN = 2 };
struct OutBias {
    const void* p;   // [N] (OB_COLUMN), dtype below
    float value;     // OB_SCALAR
    int kind;
    int dtype;       // QLIN_F32, QLIN_BF16 or QLIN_F16
};

__device__ __forceinline__ float out_bias_at(const OutBias& b, int64_t n) {
    if (b.kind != OB_COLUMN) return b.value;
    if (b.dtype == QLIN_F32) return ((const float*)b.p)[n];
    const uint32_t h = ((const uint16_t*)b.p)[n];
    return b.dtype == QLIN_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// v plus the bias of output column n (v unchanged without a bias).
__device__ __forceinline__ float add_out_bias(const OutBias& b, int64_t n, float v) {
    return b.kind == OB_NONE ? v : v + out_bias_at(b, n);
}

// ------------------------------------------------- small formats (decoding)

// E8M0 scale byte: 2^(b-127). b = 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// E4M3 (OCP "FN" variant): bias 7, 3 mantissa bits, no inf. Finite codes only.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = e ? __builtin_ldexpf((float)(8u + m), (int)e - 10) : __builtin_ldexpf((float)m, -9);
    return (c & 0x80u) ? -mag : mag;
}

// E2M1: bias 1, 1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = e ? __builtin_ldexpf((float)(2u + m), (int)e - 2) : 0.5f * (float)m;
    return (c & 8u) ? -mag : mag;
}

// Byte Q of v holds two E2M1 codes (low nibble first); returns them times
// `scale` as packed bf16 (exact). The gfx950 scaled-convert instructions
// apply only the exponent of their scale operand, so arbitrary (E4M3)
// scales are applied by an fp32 multiply after a unit-scale decode.
template <int Q>
__device__ __forceinline__ uint32_t e2m1_pair_times(uint32_t v, float scale) {
    const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, Q);
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    bf16x2_t r = {(__bf16)(f[0] * scale), (__bf16)(f[1] * scale)};
    return __builtin_bit_cast(uint32_t, r);
}

// ----------------------------------------------------------- launchers

struct QmmArgs {
    const void* x;       // [rows of A, K]
    const uint32_t* wq;  // packed weight (expert 0)
    const void* scales;
    const void* biases;
    void* y;
    int64_t M, N, K;
    int x_dtype, scale_dtype;
    int transpose, group_size, bits, mode;
    // gather form (all zero / null for a plain matmul)
    int64_t batch_x;             // B
    int64_t R;                   // rows of the index arrays
    int64_t E;
    const uint32_t* lhs;         // [R] or null
    const uint32_t* rhs;         // [R] or null
    OutBias ob;                  // dense-layer bias (plain matmul only)
};

hipError_t launch_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int g,
                           int bits, int mode, uint32_t* wq, void* scales, void* biases,
                           hipStream_t s);
hipError_t launch_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                             int sdtype, int64_t rows, int64_t cols, int g, int bits, int mode,
                             void* out, int out_dtype, hipStream_t s);
// qqmm's activation step: bf16 x [rows, cols] quantized with a microscaled
// mode (MXFP8 or NVFP4, group g along cols) and decoded back into bf16 xhat.
hipError_t launch_qdq_micro(const void* x, int64_t rows, int64_t cols, int g, int mode,
                           void* xhat, hipStream_t s);
// fp32 VALU path: any dtype, layout and mode; gather form if a.R > 0.
hipError_t launch_qmm_generic(const QmmArgs& a, hipStream_t s);
// MFMA small-M path (M <= 16, transpose, bf16 x). Returns hipErrorNotSupported
// for shapes it does not take.
hipError_t launch_qmm_decode(const QmmArgs& a, hipStream_t s);
// MFMA LDS-tiled path (transpose, bf16 x), plain or gathered rows.
hipError_t launch_qmm_tiled(const QmmArgs& a, const uint32_t* row_perm,
                            const uint32_t* expert_offsets, hipStream_t s);
bool qmm_tiled_supports(const QmmArgs& a);
// MFMA path for many rows (transpose, bf16 x), plain or expert-gathered:
// the weight tile is dequantized once into LDS per tile of activation rows.
// The gather form needs the bucketing below, run with tiles of
// prefill_gather_tile_rows rows: 128 rows of one expert once the experts
// average 48 rows or more (each expert's weight tile is then dequantized
// once: 512 tokens x top-8 over 64 experts 85 -> 77 us), else 64.
inline int prefill_gather_tile_rows(int64_t rows, int64_t experts) {
    return rows >= 48 * experts ? 128 : 64;
}
constexpr int kTiledGatherRows = 64;   // row tile of the LDS-tiled gather kernel
hipError_t launch_qmm_prefill(const QmmArgs& a, const uint32_t* row_perm,
                              const uint32_t* expert_offsets, hipStream_t s);
bool qmm_prefill_supports(const QmmArgs& a);
// Software-pipelined MFMA path for many rows of 4-bit affine weights
// (transpose, bf16 x, K a multiple of 256): the weight is dequantized in
// registers straight into the MFMA operand. Slower than the LDS-tiled
// many-row kernel on every measured shape, so it runs only when forced
// (QLIN_FORCE_PATH=prefill2).
hipError_t launch_qmm_prefill2(const QmmArgs& a, hipStream_t s);
bool qmm_prefill2_supports(const QmmArgs& a);
// VALU path for the [in, out] layout (transpose = false), M <= 8, bf16 x.
hipError_t launch_qmm_nt(const QmmArgs& a, hipStream_t s);
bool qmm_nt_supports(const QmmArgs& a);
bool qmm_decode_supports(const QmmArgs& a);
// qqmm in mxfp8 on the scaled fp8 MFMA: x's E4M3 codes [M, K] and E8M0
// scales [M, K/32] against W's, y bf16 [M, N] (transpose layout).
bool qqmm_mx8_supports(int64_t M, int64_t N, int64_t K, const void* wq, const void* ws);
hipError_t launch_qqmm_mx8(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                           uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t st);

// Gather form of the small-M kernel (transpose, bf16 x, few rows per
// expert): rows bucketed by expert into tiles of the returned height, each
// tile streaming its expert's weight once; -1: far fewer rows than experts,
// each index row is its own tile and no bucketing is needed; 0: not taken.
int qmm_decode_gather_tile_rows(const QmmArgs& a);
hipError_t launch_qmm_decode_gather(const QmmArgs& a, const uint32_t* row_perm,
                                    const uint32_t* expert_offsets, int tile_rows, hipStream_t s);
// MoE bucketing: counts rows per expert, scans, and writes a permutation of
// the rows grouped by expert (any order within an expert; skipped when the
// rows are pre-sorted). rows_per_tile sets the row-tile prefix written after
// the offsets.
hipError_t launch_bucket(const uint32_t* rhs, int64_t R, int64_t E, int64_t M, int sorted,
                         int rows_per_tile, void* workspace, uint32_t** row_perm,
                         uint32_t** expert_offsets, hipStream_t s);
size_t bucket_workspace_bytes(int64_t R, int64_t E);
// Opt-in index range check: one small kernel writes, into `result` (3
// words of device memory), the first index row r with rhs[r] >= E or
// lhs[r] >= B (r >= B without lhs), or 0xFFFFFFFF, then rhs[r] and lhs[r].
hipError_t launch_check_indices(const uint32_t* rhs, const uint32_t* lhs, int64_t R, int64_t E,
                                int64_t B, uint32_t* result, hipStream_t s);
// Where the check's result lives in a gather workspace of
// bucket_workspace_bytes(R, E) bytes (16-byte aligned, past the buckets).
uint32_t* index_check_result(void* workspace, int64_t R, int64_t E);

}  // namespace qlin
