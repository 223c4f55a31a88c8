// quant.hip -- group-wise quantize and dequantize kernels (gfx950).
//
// Quantize follows the affine rule "w ~ scale*q + bias" of the mlx-rs
// quantization.rs quantize/quantized_matmul doc comments, with one scale and
// bias per group of group_size elements along a row, and the microscaled
// modes of the "Emily.QuantizedWeight" Microscaled modes table. Codes are
// packed 32/bits per uint32, lowest element in the lowest bits
// ("Emily.QuantizedWeight", Layout).
//
// Every rounding step is explicit so that codes, scales and biases are
// bit-for-bit reproducible: fp32 subtraction, correctly rounded fp32
// division (__fdiv_rn), nearest-even (rintf), directed rounding into the
// storage dtype done on bit patterns. This file is compiled with
// -ffp-contract=off.
//
// Both kernels are HBM-streaming: one thread owns one group (quantize) or
// one packed word (dequantize).

#include "qlin_common.h"

namespace qlin {
namespace {

// ------------------------------------------------- directed rounding (bits)

// bf16: truncation drops the low 16 bits (toward zero); one bf16 step away
// from zero is +1 on the 16-bit pattern for either sign.
__device__ __forceinline__ float bf16_round_down(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t t = u & 0xFFFF0000u;
    if ((u & 0xFFFFu) && (u >> 31)) t += 0x10000u;  // negative: away from zero is down
    return __uint_as_float(t);
}
__device__ __forceinline__ float bf16_round_up(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t t = u & 0xFFFF0000u;
    if ((u & 0xFFFFu) && !(u >> 31)) t += 0x10000u;  // positive: away from zero is up
    return __uint_as_float(t);
}

// f16: nearest-even conversion, then one step if it landed on the wrong side.
__device__ __forceinline__ uint32_t f16_step(uint32_t h, bool up) {
    bool neg = h & 0x8000u;
    if ((h & 0x7FFFu) == 0) return up ? 0x0001u : 0x8001u;  // +-0
    return (up != neg) ? h + 1u : h - 1u;                   // away from / toward zero
}
__device__ __forceinline__ float f16_round_dir(float v, bool up) {
    uint32_t h = f32_to_f16_rne(v);
    float hv = f16_bits_to_f32(h);
    if (up ? (hv < v) : (hv > v)) h = f16_step(h, up);
    return f16_bits_to_f32(h);
}

template <int DT>
__device__ __forceinline__ float round_down_to(float v) {
    if constexpr (DT == QLIN_F32) return v;
    else if constexpr (DT == QLIN_BF16) return bf16_round_down(v);
    else return f16_round_dir(v, false);
}
template <int DT>
__device__ __forceinline__ float round_up_to(float v) {
    if constexpr (DT == QLIN_F32) return v;
    else if constexpr (DT == QLIN_BF16) return bf16_round_up(v);
    else return f16_round_dir(v, true);
}

// ------------------------------------------------- small formats (encoding)

// E2M1 nearest-even, saturating at 6, sign kept. The magnitude code is the
// number of rounding boundaries at or below |v|; at a tie the boundary
// counts toward the even code (0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2,
// 2.5->2, 3.5->4, 5->4).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    float a = fabsf(v);
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                 (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// E4M3 (FN) nearest-even, saturating at 448, sign kept.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    float a = fabsf(v);
    uint32_t mag;
    if (a >= 448.0f) {
        mag = 0x7Eu;
    } else if (a < 0.015625f) {  // below 2^-6: subnormal grid of spacing 2^-9
        mag = (uint32_t)rintf(__builtin_ldexpf(a, 9));
    } else {
        int E = (int)(__float_as_uint(a) >> 23) - 127;   // a is a normal fp32 here
        float t = __builtin_ldexpf(a, 3 - E);             // [8, 16), exact
        mag = (uint32_t)((E + 7) << 3) + ((uint32_t)rintf(t) - 8u);
    }
    return mag | ((__float_as_uint(v) >> 24) & 0x80u);
}

// floor(log2 a) of a positive finite fp32 (normal or subnormal).
__device__ __forceinline__ int floor_log2(float a) {
    uint32_t u = __float_as_uint(a);
    uint32_t e = u >> 23;
    if (e) return (int)e - 127;
    return (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;
}

// ---------------------------------------------------------------- kernels

template <int DT, int BITS>
__global__ void __launch_bounds__(256) quantize_affine_kernel(
    const void* __restrict__ w, int64_t rows, int64_t cols, int g, uint32_t* __restrict__ wq,
    void* __restrict__ scales, void* __restrict__ biases) {
    const int64_t groups_per_row = cols / g;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * groups_per_row) return;
    const int64_t base = gid * g;  // groups are contiguous in row-major order
    const int n = (1 << BITS) - 1;

    // plain comparisons (not fminf/fmaxf) so that the first of +0/-0 is kept
    float lo = load_f<DT>(w, base), hi = lo;
    for (int i = 1; i < g; ++i) {
        float v = load_f<DT>(w, base + i);
        lo = (v < lo) ? v : lo;
        hi = (v > hi) ? v : hi;
    }
    const float z = round_down_to<DT>(lo);
    const float range = hi - z;
    const float s32 = __fdiv_rn(range, (float)n);
    const float s = round_up_to<DT>(s32);

    constexpr int PER = 32 / BITS;
    uint32_t* out = wq + base / PER;
    for (int i0 = 0; i0 < g; i0 += PER) {
        uint32_t word = 0;
        for (int e = 0; e < PER; ++e) {
            uint32_t q = 0;
            if (s != 0.0f) {
                float d = load_f<DT>(w, base + i0 + e) - z;
                float t = rintf(__fdiv_rn(d, s));
                t = fminf(fmaxf(t, 0.0f), (float)n);
                q = (uint32_t)t;
            }
            word |= q << (e * BITS);
        }
        out[i0 / PER] = word;
    }
    store_f<DT>(scales, gid, s);
    store_f<DT>(biases, gid, z);
}

template <int DT, int MODE>
__global__ void __launch_bounds__(256) quantize_micro_kernel(
    const void* __restrict__ w, int64_t rows, int64_t cols, int g, uint32_t* __restrict__ wq,
    uint8_t* __restrict__ scales) {
    constexpr int BITS = (MODE == MXFP8) ? 8 : 4;
    constexpr int PER = 32 / BITS;
    const int64_t groups_per_row = cols / g;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= rows * groups_per_row) return;
    const int64_t base = gid * g;

    float amax = 0.0f;
    for (int i = 0; i < g; ++i) amax = fmaxf(amax, fabsf(load_f<DT>(w, base + i)));

    uint32_t sbyte;
    float sc = 0.0f;  // nvfp4 element divisor
    int e = 0;        // mx shared exponent
    if constexpr (MODE == NVFP4) {
        sbyte = e4m3_encode(__fdiv_rn(amax, 6.0f));
        sc = e4m3_to_f32(sbyte);
    } else {
        constexpr int EMAX_ELEM = (MODE == MXFP8) ? 8 : 2;
        e = (amax == 0.0f) ? -127 : floor_log2(amax) - EMAX_ELEM;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        sbyte = (uint32_t)(e + 127);
    }

    uint32_t* out = wq + base / PER;
    for (int i0 = 0; i0 < g; i0 += PER) {
        uint32_t word = 0;
        for (int k = 0; k < PER; ++k) {
            float v = load_f<DT>(w, base + i0 + k);
            uint32_t c;
            if constexpr (MODE == NVFP4) {
                c = (sc == 0.0f) ? ((__float_as_uint(v) >> 28) & 8u) : e2m1_encode(__fdiv_rn(v, sc));
            } else if constexpr (MODE == MXFP8) {
                c = e4m3_encode(__builtin_ldexpf(v, -e));
            } else {
                c = e2m1_encode(__builtin_ldexpf(v, -e));
            }
            word |= c << (k * BITS);
        }
        out[i0 / PER] = word;
    }
    scales[gid] = (uint8_t)sbyte;
}

// One thread per packed word; out row-major [rows, cols].
template <int SDT, int ODT, int BITS, int MODE>
__global__ void __launch_bounds__(256) dequantize_kernel(
    const uint32_t* __restrict__ wq, const void* __restrict__ scales,
    const void* __restrict__ biases, int64_t rows, int64_t cols, int g, void* __restrict__ out) {
    constexpr int PER = 32 / BITS;
    const int64_t words = rows * (cols / PER);
    const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (wid >= words) return;
    const int64_t k0 = wid * PER;           // flat element index of the word's first code
    const int64_t gidx = k0 / g;            // flat group index (groups never straddle words)
    const uint32_t word = wq[wid];
    float s, z = 0.0f;
    if constexpr (MODE == AFFINE) {
        s = load_f<SDT>(scales, gidx);
        z = load_f<SDT>(biases, gidx);
    } else if constexpr (MODE == NVFP4) {
        s = e4m3_to_f32(((const uint8_t*)scales)[gidx]);
    } else {
        s = e8m0_to_f32(((const uint8_t*)scales)[gidx]);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        uint32_t q = (word >> (e * BITS)) & ((1u << BITS) - 1u);
        float v;
        if constexpr (MODE == AFFINE) v = __builtin_fmaf(s, (float)q, z);
        else if constexpr (MODE == MXFP8) v = e4m3_to_f32(q) * s;
        else v = e2m1_to_f32(q) * s;
        store_f<ODT>(out, k0 + e, v);
    }
}

template <typename F>
hipError_t dispatch_dtype(int dt, F&& f) {
    switch (dt) {
    case QLIN_F32: return f(std::integral_constant<int, QLIN_F32>{});
    case QLIN_BF16: return f(std::integral_constant<int, QLIN_BF16>{});
    case QLIN_F16: return f(std::integral_constant<int, QLIN_F16>{});
    default: return hipErrorInvalidValue;
    }
}

inline unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int g,
                           int bits, int mode, uint32_t* wq, void* scales, void* biases,
                           hipStream_t st) {
    const int64_t groups = rows * (cols / g);
    const unsigned nb = nblocks(groups);
    return dispatch_dtype(w_dtype, [&](auto dt) -> hipError_t {
        constexpr int DT = decltype(dt)::value;
        if (mode == AFFINE) {
            if (bits == 2) quantize_affine_kernel<DT, 2><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, scales, biases);
            else if (bits == 4) quantize_affine_kernel<DT, 4><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, scales, biases);
            else quantize_affine_kernel<DT, 8><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, scales, biases);
        } else if (mode == MXFP4) {
            quantize_micro_kernel<DT, MXFP4><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, (uint8_t*)scales);
        } else if (mode == MXFP8) {
            quantize_micro_kernel<DT, MXFP8><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, (uint8_t*)scales);
        } else {
            quantize_micro_kernel<DT, NVFP4><<<nb, 256, 0, st>>>(w, rows, cols, g, wq, (uint8_t*)scales);
        }
        return hipGetLastError();
    });
}

hipError_t launch_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                             int sdtype, int64_t rows, int64_t cols, int g, int bits, int mode,
                             void* out, int out_dtype, hipStream_t st) {
    const int64_t words = rows * (cols * bits / 32);
    const unsigned nb = nblocks(words);
    return dispatch_dtype(out_dtype, [&](auto odt) -> hipError_t {
        constexpr int ODT = decltype(odt)::value;
        if (mode != AFFINE) {
            if (mode == MXFP4) dequantize_kernel<QLIN_F32, ODT, 4, MXFP4><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            else if (mode == NVFP4) dequantize_kernel<QLIN_F32, ODT, 4, NVFP4><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            else dequantize_kernel<QLIN_F32, ODT, 8, MXFP8><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            return hipGetLastError();
        }
        return dispatch_dtype(sdtype, [&](auto sdt) -> hipError_t {
            constexpr int SDT = decltype(sdt)::value;
            if (bits == 2) dequantize_kernel<SDT, ODT, 2, AFFINE><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            else if (bits == 4) dequantize_kernel<SDT, ODT, 4, AFFINE><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            else dequantize_kernel<SDT, ODT, 8, AFFINE><<<nb, 256, 0, st>>>(wq, scales, biases, rows, cols, g, out);
            return hipGetLastError();
        });
    });
}

}  // namespace qlin
