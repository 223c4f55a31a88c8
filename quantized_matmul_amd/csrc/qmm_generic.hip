// qmm_generic.hip -- fp32 VALU quantized matmul for every dtype, layout and
// mode, plain or gathered (gfx950).
//
// Computes y = x . dequant(W)^T (transpose) or x . dequant(W) without a
// dense W ("EMLX.Quantization", quantized_matmul; "Emily.Quantization.Layers",
// quantized_dense for the two layouts) and its expert-gathered form
// ("EMLX.Quantization", gather_quantized_matmul). Each weight is dequantized
// in registers with one fp32 FMA (scale*q + bias) and products accumulate in
// fp32. This path carries fp32/f16 activations and the [in, out] layout;
// bf16 activations with the [out, in] layout go to the MFMA kernels.

#include "qlin_common.h"

namespace qlin {
namespace {

// Dequantize the PER codes of one packed word with the group's scale/bias.
template <int MODE, int BITS, int SDT>
struct Deq {
    static constexpr int PER = 32 / BITS;
    float s, z;
    __device__ __forceinline__ void load(const void* scales, const void* biases, int64_t gidx) {
        if constexpr (MODE == AFFINE) {
            s = load_f<SDT>(scales, gidx);
            z = load_f<SDT>(biases, gidx);
        } else if constexpr (MODE == NVFP4) {
            s = e4m3_to_f32(((const uint8_t*)scales)[gidx]);
            z = 0.0f;
        } else {
            s = e8m0_to_f32(((const uint8_t*)scales)[gidx]);
            z = 0.0f;
        }
    }
    __device__ __forceinline__ float at(uint32_t word, int e) const {
        uint32_t q = (word >> (e * BITS)) & ((1u << BITS) - 1u);
        if constexpr (MODE == AFFINE) return __builtin_fmaf(s, (float)q, z);
        else if constexpr (MODE == MXFP8) return e4m3_to_f32(q) * s;
        else return e2m1_to_f32(q) * s;
    }
};

// Map logical output row rho in [0, R*M) (or [0, M)) to (x row, expert).
__device__ __forceinline__ void row_map(const QmmArgs& a, int64_t rho, int64_t& xrow,
                                        int64_t& expert) {
    if (a.R == 0) {
        xrow = rho;
        expert = 0;
        return;
    }
    int64_t r = rho / a.M, m = rho - r * a.M;
    int64_t b = a.lhs ? (int64_t)a.lhs[r] : r;
    expert = a.rhs[r];
    // indices are a precondition; out-of-range ones read row 0 / expert 0
    // (that output row is then meaningless) instead of leaving the buffers
    if (b >= a.batch_x) b = 0;
    if (expert >= a.E) expert = 0;
    xrow = b * a.M + m;
}

constexpr int ROWS_PER_WAVE = 4;

// transpose=true: one wave per (column n, ROWS_PER_WAVE consecutive rows);
// lanes stride over the packed words of W row n; wave-wide sum at the end.
template <int XDT, int SDT, int MODE, int BITS>
__global__ void __launch_bounds__(256) qmm_generic_t_kernel(QmmArgs a, int64_t total_rows) {
    using D = Deq<MODE, BITS, SDT>;
    constexpr int PER = D::PER;
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n = wave % a.N;
    const int64_t rho0 = (wave / a.N) * ROWS_PER_WAVE;
    if (rho0 >= total_rows) return;
    const int64_t words = a.K / PER, groups = a.K / a.group_size;
    const int64_t wsize = a.N * words, ssize = a.N * groups;

    float acc[ROWS_PER_WAVE];
    int64_t xrow[ROWS_PER_WAVE], ex[ROWS_PER_WAVE];
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        acc[i] = 0.0f;
        int64_t rho = rho0 + i < total_rows ? rho0 + i : total_rows - 1;
        row_map(a, rho, xrow[i], ex[i]);
    }
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        const uint32_t* wrow = a.wq + ex[i] * wsize + n * words;
        for (int64_t c = lane; c < words; c += 64) {
            D d;
            int64_t gidx = ex[i] * ssize + n * groups + (c * PER) / a.group_size;
            d.load(a.scales, a.biases, gidx);
            uint32_t word = wrow[c];
#pragma unroll
            for (int e = 0; e < PER; ++e)
                acc[i] = __builtin_fmaf(load_f<XDT>(a.x, xrow[i] * a.K + c * PER + e), d.at(word, e), acc[i]);
        }
    }
    for (int i = 0; i < ROWS_PER_WAVE; ++i) {
        float v = acc[i];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[i] = v;
    }
    if (lane == 0) {
        for (int i = 0; i < ROWS_PER_WAVE; ++i)
            if (rho0 + i < total_rows) store_f<XDT>(a.y, (rho0 + i) * a.N + n, add_out_bias(a.ob, n, acc[i]));
    }
}

// transpose=false: W is [K, N] packed along N. A block owns 64 word columns
// (64*PER outputs) of one row; its 4 waves split K and meet in LDS.
template <int XDT, int SDT, int MODE, int BITS>
__global__ void __launch_bounds__(256) qmm_generic_n_kernel(QmmArgs a, int64_t total_rows) {
    using D = Deq<MODE, BITS, SDT>;
    constexpr int PER = D::PER;
    __shared__ float red[4][64][PER];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t wcols = a.N / PER, groups = a.N / a.group_size;
    const int64_t cblocks = (wcols + 63) / 64;
    const int64_t rho = blockIdx.x / cblocks;
    const int64_t c = (blockIdx.x % cblocks) * 64 + lane;
    if (rho >= total_rows) return;
    int64_t xrow, ex;
    row_map(a, rho, xrow, ex);
    const int64_t wsize = a.K * wcols, ssize = a.K * groups;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    if (c < wcols) {
        const int64_t k_per = (a.K + 3) / 4;
        const int64_t k0 = wv * k_per, k1 = (k0 + k_per < a.K) ? k0 + k_per : a.K;
        for (int64_t k = k0; k < k1; ++k) {
            D d;
            d.load(a.scales, a.biases, ex * ssize + k * groups + (c * PER) / a.group_size);
            uint32_t word = a.wq[ex * wsize + k * wcols + c];
            float xv = load_f<XDT>(a.x, xrow * a.K + k);
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = __builtin_fmaf(xv, d.at(word, e), acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) red[wv][lane][e] = acc[e];
    __syncthreads();
    if (wv == 0 && c < wcols) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float v = red[0][lane][e] + red[1][lane][e] + red[2][lane][e] + red[3][lane][e];
            store_f<XDT>(a.y, rho * a.N + c * PER + e, add_out_bias(a.ob, c * PER + e, v));
        }
    }
}

template <int XDT, int SDT, int MODE, int BITS>
hipError_t launch_one(const QmmArgs& a, hipStream_t st) {
    const int64_t total_rows = a.R ? a.R * a.M : a.M;
    if (a.transpose) {
        const int64_t waves = a.N * ((total_rows + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE);
        const int64_t blocks = (waves + 3) / 4;
        qmm_generic_t_kernel<XDT, SDT, MODE, BITS><<<(unsigned)blocks, 256, 0, st>>>(a, total_rows);
    } else {
        const int64_t cblocks = (a.N / (32 / BITS) + 63) / 64;
        qmm_generic_n_kernel<XDT, SDT, MODE, BITS><<<(unsigned)(total_rows * cblocks), 256, 0, st>>>(a, total_rows);
    }
    return hipGetLastError();
}

template <int XDT, int SDT>
hipError_t by_mode(const QmmArgs& a, hipStream_t st) {
    switch (a.mode) {
    case AFFINE:
        if (a.bits == 2) return launch_one<XDT, SDT, AFFINE, 2>(a, st);
        if (a.bits == 4) return launch_one<XDT, SDT, AFFINE, 4>(a, st);
        return launch_one<XDT, SDT, AFFINE, 8>(a, st);
    case MXFP4: return launch_one<XDT, SDT, MXFP4, 4>(a, st);
    case MXFP8: return launch_one<XDT, SDT, MXFP8, 8>(a, st);
    default: return launch_one<XDT, SDT, NVFP4, 4>(a, st);
    }
}

template <int XDT>
hipError_t by_sdtype(const QmmArgs& a, hipStream_t st) {
    if (a.mode != AFFINE) return by_mode<XDT, QLIN_F32>(a, st);  // scale dtype unused
    // affine requires scale dtype == x dtype (checked by the API layer)
    return by_mode<XDT, XDT>(a, st);
}

}  // namespace

hipError_t launch_qmm_generic(const QmmArgs& a, hipStream_t st) {
    switch (a.x_dtype) {
    case QLIN_F32: return by_sdtype<QLIN_F32>(a, st);
    case QLIN_BF16: return by_sdtype<QLIN_BF16>(a, st);
    default: return by_sdtype<QLIN_F16>(a, st);
    }
}

}  // namespace qlin
