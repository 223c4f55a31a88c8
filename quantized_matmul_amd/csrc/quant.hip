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
// All kernels are HBM-streaming: one thread owns one packed word and the
// elements it encodes (the lanes of a group cooperate on its scale).

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
//
// Quantize: lane l of the grid owns packed word l, i.e. the PER = 32/bits
// consecutive elements it encodes, so a wave reads 64*PER contiguous
// elements (16-byte vector loads when w is 16-byte aligned) and writes 64
// contiguous words. A group is g/PER adjacent lanes of one wave (the flat
// element count is a multiple of g and a group never straddles a row, so
// groups are whole and wave-aligned); its min/max (or amax) is combined
// across those lanes with xor shuffles. Rounding is unchanged: every code
// still takes one correctly rounded fp32 division and rint.

// PER elements of dtype DT starting at element i (i a multiple of PER).
template <int DT, int PER, bool VEC>
__device__ __forceinline__ void load_chunk(const void* w, int64_t i, float (&v)[PER]) {
    if constexpr (!VEC) {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[e] = load_f<DT>(w, i + e);
    } else if constexpr (DT == QLIN_F32) {
        const float4* p = (const float4*)((const float*)w + i);
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) {
            const float4 t = p[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    } else {
        constexpr int NW = PER / 2;    // dwords of 16-bit elements
        uint32_t d[NW];
        if constexpr (NW % 4 == 0) {
            const uint4* p = (const uint4*)((const uint16_t*)w + i);
#pragma unroll
            for (int q = 0; q < NW / 4; ++q) {
                const uint4 t = p[q];
                d[4 * q] = t.x; d[4 * q + 1] = t.y; d[4 * q + 2] = t.z; d[4 * q + 3] = t.w;
            }
        } else {   // NW == 2
            const uint2 t = *(const uint2*)((const uint16_t*)w + i);
            d[0] = t.x; d[1] = t.y;
        }
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            if constexpr (DT == QLIN_BF16) {
                v[2 * q] = bf16_bits_to_f32(d[q] & 0xFFFFu);
                v[2 * q + 1] = bf16_bits_to_f32(d[q] >> 16);
            } else {
                v[2 * q] = f16_bits_to_f32(d[q] & 0xFFFFu);
                v[2 * q + 1] = f16_bits_to_f32(d[q] >> 16);
            }
        }
    }
}

// The IEEE fp32 quotient d / s from r = 1/s correctly rounded in fp64:
// (float)(d * r) rounds the fp64 product once more, to fp32. The product is
// within 2^-52 (relative) of d / s, and a quotient of two 24-bit
// significands that is not itself an fp32 value lies at least 2^-48 from
// every fp32 rounding boundary in the normal range (a midpoint has 25
// significant bits, and d - s * midpoint is a nonzero multiple of a unit
// 2^-47 of d), so both roundings land on the same fp32 value. Quotients in
// the subnormal range may differ in their last bit; every caller maps such
// a value to code 0 (affine) or to a signed zero (E2M1), as it does the
// exact quotient. One fp64 reciprocal per word replaces a division per
// element, which bound the quantize kernels on VALU issue.
__device__ __forceinline__ float div_by_recip(float d, double r) { return (float)((double)d * r); }

// Min (MIN) or max of v over the LPG adjacent lanes of a group, LPG a power
// of two <= 64. Each stage merges two neighbouring blocks of lanes with the
// lower block's value as the first operand, so among equal values (+0 and
// -0) every lane ends with the first one in element order, as a sequential
// scan with plain comparisons keeps it.
template <int LPG, bool MIN>
__device__ __forceinline__ float group_minmax(float v) {
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) {
        const float p = __shfl_xor(v, off, 64);
        const bool low = (threadIdx.x & off) == 0;
        const float a = low ? v : p, b = low ? p : v;   // a: lower block, b: upper block
        v = MIN ? ((b < a) ? b : a) : ((b > a) ? b : a);
    }
    return v;
}

// Max of non-negative v over the LPG adjacent lanes of a group.
template <int LPG>
__device__ __forceinline__ float group_amax(float v) {
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// One packed word of codes from its PER elements v; the LPG lanes of a
// group hold its consecutive words (whole groups are live or not).
template <int DT, int BITS, int LPG>
__device__ __forceinline__ void quantize_affine_word(const float (&v)[32 / BITS], int64_t wid, bool live,
                                                     uint32_t* __restrict__ wq, void* __restrict__ scales,
                                                     void* __restrict__ biases) {
    constexpr int PER = 32 / BITS;
    const int n = (1 << BITS) - 1;
    // group min and max; plain comparisons (not fminf/fmaxf) keep the first
    // of +0/-0 within a lane, and the lanes are combined in element order
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int e = 1; e < PER; ++e) {
        lo = (v[e] < lo) ? v[e] : lo;
        hi = (v[e] > hi) ? v[e] : hi;
    }
    lo = group_minmax<LPG, true>(lo);
    hi = group_minmax<LPG, false>(hi);
    const float z = round_down_to<DT>(lo);
    const float s = round_up_to<DT>(__fdiv_rn(hi - z, (float)n));

    uint32_t word = 0;
    if (s != 0.0f) {
        const double r = 1.0 / (double)s;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float t = rintf(div_by_recip(v[e] - z, r));
            t = fminf(fmaxf(t, 0.0f), (float)n);
            word |= (uint32_t)t << (e * BITS);
        }
    }
    if (live) {
        wq[wid] = word;
        if ((threadIdx.x & (LPG - 1)) == 0) {
            const int64_t gid = wid / LPG;
            store_f<DT>(scales, gid, s);
            store_f<DT>(biases, gid, z);
        }
    }
}

// WPT words per thread, thread t of a block taking words base + t + 256 j:
// every wave-wide load and store stays contiguous and a group's LPG lanes
// stay consecutive; all WPT words' elements are loaded before any is coded.
template <int DT, int BITS, bool VEC, int LPG, int WPT>
__global__ void __launch_bounds__(256) quantize_affine_kernel(
    const void* __restrict__ w, int64_t words, int g, uint32_t* __restrict__ wq,
    void* __restrict__ scales, void* __restrict__ biases) {
    constexpr int PER = 32 / BITS;
    const int64_t base = (int64_t)blockIdx.x * (256 * WPT) + threadIdx.x;
    float v[WPT][PER];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int64_t wid = base + 256 * j;
        load_chunk<DT, PER, VEC>(w, (wid < words ? wid : 0) * PER, v[j]);
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int64_t wid = base + 256 * j;
        quantize_affine_word<DT, BITS, LPG>(v[j], wid, wid < words, wq, scales, biases);
    }
}

// Block scale of a microscaled group from its amax ("Emily.QuantizedWeight",
// Microscaled modes; OCP MX shared exponent for mx*, E4M3(amax/6) for
// nvfp4): the scale byte, and the divisor (nvfp4) or exponent (mx*) the
// elements are encoded with.
template <int MODE>
struct MicroScale {
    uint32_t sbyte;
    float sc;   // nvfp4 element divisor
    double rsc; // its fp64 reciprocal (0 when sc is 0)
    int e;      // mx shared exponent
};
template <int MODE>
__device__ __forceinline__ MicroScale<MODE> micro_scale(float amax) {
    MicroScale<MODE> m{0u, 0.0f, 0.0, 0};
    if constexpr (MODE == NVFP4) {
        m.sbyte = e4m3_encode(__fdiv_rn(amax, 6.0f));
        m.sc = e4m3_to_f32(m.sbyte);
        m.rsc = m.sc == 0.0f ? 0.0 : 1.0 / (double)m.sc;
    } else {
        constexpr int EMAX_ELEM = (MODE == MXFP8) ? 8 : 2;
        int e = (amax == 0.0f) ? -127 : floor_log2(amax) - EMAX_ELEM;
        e = e < -127 ? -127 : (e > 127 ? 127 : e);
        m.e = e;
        m.sbyte = (uint32_t)(e + 127);
    }
    return m;
}

// Element code of v under the group's scale.
template <int MODE>
__device__ __forceinline__ uint32_t micro_encode(float v, const MicroScale<MODE>& m) {
    if constexpr (MODE == NVFP4)
        return (m.sc == 0.0f) ? ((__float_as_uint(v) >> 28) & 8u) : e2m1_encode(div_by_recip(v, m.rsc));
    else if constexpr (MODE == MXFP8)
        return e4m3_encode(__builtin_ldexpf(v, -m.e));
    else
        return e2m1_encode(__builtin_ldexpf(v, -m.e));
}

template <int MODE, int LPG>
__device__ __forceinline__ void quantize_micro_word(const float (&v)[MODE == MXFP8 ? 4 : 8], int64_t wid,
                                                    bool live, uint32_t* __restrict__ wq,
                                                    uint8_t* __restrict__ scales) {
    constexpr int BITS = (MODE == MXFP8) ? 8 : 4;
    constexpr int PER = 32 / BITS;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const MicroScale<MODE> m = micro_scale<MODE>(group_amax<LPG>(amax));
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) word |= micro_encode<MODE>(v[k], m) << (k * BITS);
    if (live) {
        wq[wid] = word;
        if ((threadIdx.x & (LPG - 1)) == 0) scales[wid / LPG] = (uint8_t)m.sbyte;
    }
}

template <int DT, int MODE, bool VEC, int LPG, int WPT>
__global__ void __launch_bounds__(256) quantize_micro_kernel(
    const void* __restrict__ w, int64_t words, int g, uint32_t* __restrict__ wq,
    uint8_t* __restrict__ scales) {
    constexpr int BITS = (MODE == MXFP8) ? 8 : 4;
    constexpr int PER = 32 / BITS;
    const int64_t base = (int64_t)blockIdx.x * (256 * WPT) + threadIdx.x;
    float v[WPT][PER];
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int64_t wid = base + 256 * j;
        load_chunk<DT, PER, VEC>(w, (wid < words ? wid : 0) * PER, v[j]);
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int64_t wid = base + 256 * j;
        quantize_micro_word<MODE, LPG>(v[j], wid, wid < words, wq, scales);
    }
}

// qqmm's activation step (mlx-rs qqmm: x is quantized on the fly): bf16 x
// quantized along its rows with a microscaled mode and decoded straight
// back, xhat = decode(code) * decode(scale byte). Every such value is exact
// in bf16 (at most 6 significant bits), so the matmul kernels then take
// xhat as an ordinary bf16 activation. Lanes and groups as in quantize.
template <int MODE, bool VEC, int LPG>
__global__ void __launch_bounds__(256) qdq_micro_kernel(const void* __restrict__ x, int64_t words,
                                                        uint16_t* __restrict__ xhat) {
    constexpr int BITS = (MODE == MXFP8) ? 8 : 4;
    constexpr int PER = 32 / BITS;
    const int64_t wid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = wid < words;
    float v[PER];
    load_chunk<QLIN_BF16, PER, VEC>(x, (live ? wid : 0) * PER, v);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < PER; ++e) amax = fmaxf(amax, fabsf(v[e]));
    const MicroScale<MODE> m = micro_scale<MODE>(group_amax<LPG>(amax));
    const float s = MODE == NVFP4 ? e4m3_to_f32(m.sbyte) : e8m0_to_f32(m.sbyte);
    uint32_t d[PER / 2];
#pragma unroll
    for (int k = 0; k < PER; k += 2) {
        const uint32_t c0 = micro_encode<MODE>(v[k], m), c1 = micro_encode<MODE>(v[k + 1], m);
        const float f0 = (MODE == MXFP8 ? e4m3_to_f32(c0) : e2m1_to_f32(c0)) * s;
        const float f1 = (MODE == MXFP8 ? e4m3_to_f32(c1) : e2m1_to_f32(c1)) * s;
        d[k / 2] = f32_to_bf16_rne(f0) | (f32_to_bf16_rne(f1) << 16);
    }
    if (!live) return;
    if constexpr (VEC) {
        if constexpr (PER == 8) {
            *(uint4*)(xhat + wid * PER) = uint4{d[0], d[1], d[2], d[3]};
        } else {
            *(uint2*)(xhat + wid * PER) = uint2{d[0], d[1]};
        }
    } else {
#pragma unroll
        for (int k = 0; k < PER / 2; ++k) {
            xhat[wid * PER + 2 * k] = (uint16_t)(d[k] & 0xFFFFu);
            xhat[wid * PER + 2 * k + 1] = (uint16_t)(d[k] >> 16);
        }
    }
}

// One packed word; out row-major [rows, cols]. VEC: the word's PER outputs
// go out as 16-byte (or 8-byte) vector stores.
template <int SDT, int ODT, int BITS, int MODE, bool VEC>
__device__ __forceinline__ void dequantize_word(const uint32_t word, int64_t wid,
    const void* __restrict__ scales, const void* __restrict__ biases, int g, void* __restrict__ out);

// WPT packed words per thread, thread t of a block taking words
// base + t + 256 j, so every wave-wide load and store stays contiguous. Four
// words per thread measured faster for 4- and 8-bit codes (W [14336, 4096]
// int4 g64 to bf16, inputs cycled past the Infinity Cache: 39.5 -> 35.7 us;
// int8 54.2 -> 41.7 us; mxfp4 [8192, 8192] 50.1 -> 47.8 us); 2-bit codes
// (16 outputs a word) keep one (38.2 against 41.6 us); loading the four words
// as one 16-byte vector per lane, stores then 64 bytes apart, ran twice as long.
template <int SDT, int ODT, int BITS, int MODE, bool VEC, int WPT>
__global__ void __launch_bounds__(256) dequantize_kernel(
    const uint32_t* __restrict__ wq, const void* __restrict__ scales,
    const void* __restrict__ biases, int64_t words, int g, void* __restrict__ out) {
    const int64_t base = (int64_t)blockIdx.x * (256 * WPT) + threadIdx.x;
    uint32_t wv[WPT];
#pragma unroll
    for (int j = 0; j < WPT; ++j) wv[j] = base + 256 * j < words ? wq[base + 256 * j] : 0u;
#pragma unroll
    for (int j = 0; j < WPT; ++j)
        if (base + 256 * j < words)
            dequantize_word<SDT, ODT, BITS, MODE, VEC>(wv[j], base + 256 * j, scales, biases, g, out);
}

template <int SDT, int ODT, int BITS, int MODE, bool VEC>
__device__ __forceinline__ void dequantize_word(const uint32_t word, int64_t wid,
    const void* __restrict__ scales, const void* __restrict__ biases, int g, void* __restrict__ out) {
    constexpr int PER = 32 / BITS;
    const int64_t k0 = wid * PER;           // flat element index of the word's first code
    const int64_t gidx = k0 / g;            // flat group index (groups never straddle words)
    float s, z = 0.0f;
    if constexpr (MODE == AFFINE) {
        s = load_f<SDT>(scales, gidx);
        z = load_f<SDT>(biases, gidx);
    } else if constexpr (MODE == NVFP4) {
        s = e4m3_to_f32(((const uint8_t*)scales)[gidx]);
    } else {
        s = e8m0_to_f32(((const uint8_t*)scales)[gidx]);
    }
    float v[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        uint32_t q = (word >> (e * BITS)) & ((1u << BITS) - 1u);
        if constexpr (MODE == AFFINE) v[e] = __builtin_fmaf(s, (float)q, z);
        else if constexpr (MODE == MXFP8) v[e] = e4m3_to_f32(q) * s;
        else v[e] = e2m1_to_f32(q) * s;
    }
    if constexpr (!VEC) {
#pragma unroll
        for (int e = 0; e < PER; ++e) store_f<ODT>(out, k0 + e, v[e]);
    } else if constexpr (ODT == QLIN_F32) {
        float4* p = (float4*)((float*)out + k0);
#pragma unroll
        for (int q = 0; q < PER / 4; ++q) p[q] = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    } else {
        uint32_t d[PER / 2];
#pragma unroll
        for (int q = 0; q < PER / 2; ++q) {
            const uint32_t a = ODT == QLIN_BF16 ? f32_to_bf16_rne(v[2 * q]) : f32_to_f16_rne(v[2 * q]);
            const uint32_t b = ODT == QLIN_BF16 ? f32_to_bf16_rne(v[2 * q + 1]) : f32_to_f16_rne(v[2 * q + 1]);
            d[q] = a | (b << 16);
        }
        if constexpr (PER / 2 % 4 == 0) {
            uint4* p = (uint4*)((uint16_t*)out + k0);
#pragma unroll
            for (int q = 0; q < PER / 8; ++q) p[q] = uint4{d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]};
        } else {   // PER == 4
            *(uint2*)((uint16_t*)out + k0) = uint2{d[0], d[1]};
        }
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

// lanes per group: g / PER, a power of two from 1 to 32
template <class F>
hipError_t dispatch_lpg(int lpg, F&& f) {
    switch (lpg) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int g,
                           int bits, int mode, uint32_t* wq, void* scales, void* biases,
                           hipStream_t st) {
    const int64_t words = rows * (cols * bits / 32);
    // Words per thread, from rotating-buffer timings over 5 weight copies
    // (14336x4096 affine, 8192x8192 micro; us per call, 1 -> 4 words):
    // affine 8-bit 57.3 -> 54.3, MXFP8 61.0 -> 48.9, MXFP4 45.0 -> 43.0 gain;
    // affine 4-bit 40.1 -> 44.0 and 2-bit 34 -> 41 lose, NVFP4 is flat.
    // Both choices write identical bytes.
    const unsigned nb = nblocks(words), nb4 = nblocks((words + 3) / 4);
    const int per = 32 / bits;
    const bool vec = ((uintptr_t)w & 15) == 0;
    return dispatch_dtype(w_dtype, [&](auto dt) -> hipError_t {
        constexpr int DT = decltype(dt)::value;
        return dispatch_lpg(g / per, [&](auto lpgc) -> hipError_t {
            constexpr int LPG = decltype(lpgc)::value;
            auto go = [&](auto kv) -> hipError_t {
                constexpr bool V = decltype(kv)::value;
                if (mode == AFFINE) {
                    if (bits == 2) quantize_affine_kernel<DT, 2, V, LPG, 1><<<nb, 256, 0, st>>>(w, words, g, wq, scales, biases);
                    else if (bits == 4) quantize_affine_kernel<DT, 4, V, LPG, 1><<<nb, 256, 0, st>>>(w, words, g, wq, scales, biases);
                    else quantize_affine_kernel<DT, 8, V, LPG, 4><<<nb4, 256, 0, st>>>(w, words, g, wq, scales, biases);
                } else if (mode == MXFP4) {
                    quantize_micro_kernel<DT, MXFP4, V, LPG, 4><<<nb4, 256, 0, st>>>(w, words, g, wq, (uint8_t*)scales);
                } else if (mode == MXFP8) {
                    quantize_micro_kernel<DT, MXFP8, V, LPG, 4><<<nb4, 256, 0, st>>>(w, words, g, wq, (uint8_t*)scales);
                } else {
                    quantize_micro_kernel<DT, NVFP4, V, LPG, 1><<<nb, 256, 0, st>>>(w, words, g, wq, (uint8_t*)scales);
                }
                return hipGetLastError();
            };
            return vec ? go(std::true_type{}) : go(std::false_type{});
        });
    });
}

hipError_t launch_qdq_micro(const void* x, int64_t rows, int64_t cols, int g, int mode,
                           void* xhat, hipStream_t st) {
    const int bits = mode == MXFP8 ? 8 : 4;
    const int64_t words = rows * (cols * bits / 32);
    const unsigned nb = nblocks(words);
    const bool vec = (((uintptr_t)x | (uintptr_t)xhat) & 15) == 0;
    return dispatch_lpg(g / (32 / bits), [&](auto lpgc) -> hipError_t {
        constexpr int LPG = decltype(lpgc)::value;
        auto go = [&](auto kv) -> hipError_t {
            constexpr bool V = decltype(kv)::value;
            if (mode == MXFP8) qdq_micro_kernel<MXFP8, V, LPG><<<nb, 256, 0, st>>>(x, words, (uint16_t*)xhat);
            else if (mode == NVFP4) qdq_micro_kernel<NVFP4, V, LPG><<<nb, 256, 0, st>>>(x, words, (uint16_t*)xhat);
            else return hipErrorInvalidValue;
            return hipGetLastError();
        };
        return vec ? go(std::true_type{}) : go(std::false_type{});
    });
}

hipError_t launch_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                             int sdtype, int64_t rows, int64_t cols, int g, int bits, int mode,
                             void* out, int out_dtype, hipStream_t st) {
    const int64_t words = rows * (cols * bits / 32);
    const unsigned nb = nblocks(words), nb4 = nblocks((words + 3) / 4);
    const bool vec = ((uintptr_t)out & 15) == 0;
    return dispatch_dtype(out_dtype, [&](auto odt) -> hipError_t {
        constexpr int ODT = decltype(odt)::value;
        auto go = [&](auto kv) -> hipError_t {
            constexpr bool V = decltype(kv)::value;
            if (mode != AFFINE) {
                if (mode == MXFP4) dequantize_kernel<QLIN_F32, ODT, 4, MXFP4, V, 4><<<nb4, 256, 0, st>>>(wq, scales, biases, words, g, out);
                else if (mode == NVFP4) dequantize_kernel<QLIN_F32, ODT, 4, NVFP4, V, 4><<<nb4, 256, 0, st>>>(wq, scales, biases, words, g, out);
                else dequantize_kernel<QLIN_F32, ODT, 8, MXFP8, V, 4><<<nb4, 256, 0, st>>>(wq, scales, biases, words, g, out);
                return hipGetLastError();
            }
            return dispatch_dtype(sdtype, [&](auto sdt) -> hipError_t {
                constexpr int SDT = decltype(sdt)::value;
                if (bits == 2) dequantize_kernel<SDT, ODT, 2, AFFINE, V, 1><<<nb, 256, 0, st>>>(wq, scales, biases, words, g, out);
                else if (bits == 4) dequantize_kernel<SDT, ODT, 4, AFFINE, V, 4><<<nb4, 256, 0, st>>>(wq, scales, biases, words, g, out);
                else dequantize_kernel<SDT, ODT, 8, AFFINE, V, 4><<<nb4, 256, 0, st>>>(wq, scales, biases, words, g, out);
                return hipGetLastError();
            });
        };
        return vec ? go(std::true_type{}) : go(std::false_type{});
    });
}

}  // namespace qlin
