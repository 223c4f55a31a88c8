// qmm_nt.hip -- quantized matmul for the [in, out] weight layout
// (transpose = false) with few activation rows (gfx950).
//
// y[m, n] = sum_k x[m, k] * (s[k, g(n)] * q[k, n] + z[k, g(n)]) with W stored
// [K, N] and packed along N ("Emily.Quantization.Layers", quantized_dense:
// transpose false is the [in, out] layout that computes x @ W; mlx-rs
// test_quantized_matmul exercises it). The contraction runs down the rows of
// W, so each lane owns packed words of one column range and walks K:
//   * per row k the group scale is folded into x (a = x[m,k] * s, one multiply
//     per row and group) and the bias term x[m,k] * z is summed once per row;
//   * codes become fp32 and accumulate with one FMA each (fp32 throughout);
//   * a wave load covers 8 rows x 8 packed words, so a workgroup spans few
//     columns and the grid has enough workgroups; its 16 waves split K and
//     meet once in LDS; the weight words stream through a 16-deep prefetch
//     ring;
//   * x for all of K is staged in LDS up front; each row's scale and bias
//     ride in the prefetch ring with its packed word (staging them up front
//     serialised thousands of scattered 2-byte loads before the weight
//     stream started: 27 -> 25 us at M1, 63 -> 53 us at M8).

#include "qlin_common.h"

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct NtArgs {
    const uint16_t* x;   // bf16 [M, K]
    const uint32_t* wq;  // [K, N/PER]
    const void* scales;  // [K, N/G] bf16 or u8
    const uint16_t* biases;
    uint16_t* y;         // bf16 [M, N]
    int M, N, K;
    OutBias ob;          // dense-layer bias
};

// Lane (rr, cl) = (lane / WPB, lane % WPB) handles packed word c0 + cl of
// row k = RPS * step + rr: one wave load covers RPS = 64 / WPB rows x WPB
// words. The NW waves of a workgroup split K. Each lane keeps RING2 steps
// (word, scale, bias) in flight: 16 for up to 2 activation rows of affine
// codes (32 for one row), fewer otherwise (the accumulators and decoding
// take the registers). MR = activation rows rounded up (<= 8).
template <int MODE, int BITS, int G, int MR, int WPB, int NW>
__global__ void __launch_bounds__(64 * NW) qmm_nt_kernel(NtArgs a) {
    // steps in flight per lane (microscaled decoding needs more registers):
    // the kernel is bound by the bytes each lane keeps in flight, so one
    // activation row of 4- or 8-bit affine codes takes 32 (126 registers, no
    // spills; 25 -> 22.8 us at M1), two rows 16
    constexpr int RING2 = (MR == 1 && MODE == AFFINE && BITS >= 4) ? 32
                        : (MR <= 2 && MODE == AFFINE) ? 16 : (MR <= 4 ? 8 : 4);
    constexpr int NWAVES = NW;
    constexpr int RPS = 64 / WPB;                     // rows per step
    constexpr int PER = 32 / BITS;
    constexpr bool AFF = MODE == AFFINE;
    constexpr int SBYTES = AFF ? 2 : 1;               // bytes per scale value
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rr = lane / WPB, cl = lane % WPB;
    const int K = a.K, N = a.N;
    const int wcols = N / PER;                        // packed words per W row
    // Workgroups are dealt to the 8 XCDs round-robin. Neighbouring column
    // blocks share 128-byte lines of every weight row (a block uses WPB words
    // of a row), so renumber the blocks: each XCD walks a contiguous run of
    // them and the shared lines meet in that XCD's L2 instead of being
    // fetched once per XCD.
    int cb = blockIdx.x;
    if ((gridDim.x & 7) == 0) cb = (cb & 7) * (gridDim.x >> 3) + (cb >> 3);
    const int c = cb * WPB + cl;                      // word column of the lane
    const bool active = c < wcols;
    const int gpr = N / G;                            // groups per W row
    const int g0 = (cb * WPB * PER) / G;              // first group of the workgroup
    const int gl = active ? (c * PER) / G - g0 : 0;   // the lane's group, local

    // LDS: x [MR][K] bf16
    uint16_t* xs = (uint16_t*)smem;

    // ---- stage x with loads all issued before any use
    {
        const uint16_t* xg = a.x;
        const int xv8 = (a.M * K) / 8;                // 16-byte chunks of x (K % 8 == 0)
        constexpr int XI = (8 * 4096) / 8 / (64 * NW) > 0 ? (8 * 4096) / 8 / (64 * NW) : 1;
        for (int base = 0; base < MR * K / 8; base += 64 * NW * XI) {
            u32x4 v[XI];
#pragma unroll
            for (int t = 0; t < XI; ++t) {
                const int idx = base + t * 64 * NW + tid;
                v[t] = idx < xv8 ? *(const u32x4*)(xg + (size_t)idx * 8) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int t = 0; t < XI; ++t) {
                const int idx = base + t * 64 * NW + tid;
                if (idx < MR * K / 8) *(u32x4*)(xs + (size_t)idx * 8) = v[t];
            }
        }
    }
    __syncthreads();

    // K-slice of the wave: T steps of RPS rows, T a multiple of RING2. Every
    // weight load is unconditional on a clamped, valid address (so the
    // compiler's wait counts stay exact and the ring really overlaps); rows
    // outside the slice or past K get zero scale and bias and add nothing.
    const int steps_total = (K + RPS - 1) / RPS;
    const int T = ((steps_total + NWAVES - 1) / NWAVES + RING2 - 1) / RING2 * RING2;
    const int s0 = wv * T;

    float acc[MR][PER], zacc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        zacc[m] = 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[m][e] = 0.f;
    }

    const uint32_t* wp = a.wq + (active ? c : 0);
    uint32_t rw[RING2], rs[RING2], rz[RING2];
    const uint32_t sbytes_all = (uint32_t)K * (uint32_t)gpr * SBYTES;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.scales), (short)0, (int)sbytes_all, 0x00020000);
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(AFF ? a.biases : (const uint16_t*)a.scales), (short)0,
        (int)(AFF ? sbytes_all : 0u), 0x00020000);
    const uint32_t gcol = (uint32_t)(g0 + gl);  // the lane's group column
    auto fetch = [&](int slot, int st) {
        const int k = RPS * st + rr;
        const int kk = (active && k < K) ? k : 0;
        rw[slot] = wp[(size_t)kk * wcols];
        const uint32_t so = ((uint32_t)kk * (uint32_t)gpr + gcol) * (uint32_t)SBYTES;
        if constexpr (AFF) {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0);
            rz[slot] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0);
        } else {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b8(srs, (int)so, 0, 0);
        }
    };
    auto consume = [&](int slot, int st) {
        const uint32_t w = rw[slot];
        const int kr = RPS * st + rr;
        const bool ok = active && kr < K;
        const int k = ok ? kr : 0;
        float s, z = 0.f;
        if constexpr (AFF) {
            s = bf16_bits_to_f32(rs[slot] & 0xFFFFu);
            z = bf16_bits_to_f32(rz[slot] & 0xFFFFu);
        } else {
            const uint32_t b = rs[slot] & 0xFFu;
            s = MODE == NVFP4 ? e4m3_to_f32(b) : e8m0_to_f32(b);
        }
        s = ok ? s : 0.f;
        z = ok ? z : 0.f;
        float f[PER];
        if constexpr (AFF && BITS == 4) {
            const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[2 * q] = (float)((lo >> (8 * q)) & 0xFFu);
                f[2 * q + 1] = (float)((hi >> (8 * q)) & 0xFFu);
            }
        } else if constexpr (AFF && BITS == 8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) f[q] = (float)((w >> (8 * q)) & 0xFFu);
        } else if constexpr (AFF) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t mm = (w >> (2 * t)) & 0x03030303u;
#pragma unroll
                for (int q = 0; q < 4; ++q) f[4 * q + t] = (float)((mm >> (8 * q)) & 0xFFu);
            }
        } else if constexpr (MODE == MXFP8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) f[q] = e4m3_to_f32((w >> (8 * q)) & 0xFFu);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = e2m1_to_f32((w >> (4 * e)) & 0xFu);
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float xv = bf16_bits_to_f32(xs[m * K + k]);
            const float av = xv * s;
            if constexpr (AFF) zacc[m] = __builtin_fmaf(xv, z, zacc[m]);
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[m][e] = __builtin_fmaf(av, f[e], acc[m][e]);
        }
    };
#pragma unroll
    for (int r = 0; r < RING2; ++r) fetch(r, s0 + r);
    for (int b = s0; b < s0 + T - RING2; b += RING2) {
#pragma unroll
        for (int r = 0; r < RING2; ++r) {
            consume(r, b + r);
            fetch(r, b + r + RING2);
        }
    }
#pragma unroll
    for (int r = 0; r < RING2; ++r) consume(r, s0 + T - RING2 + r);

    // sum the 4 row-lanes of each word column, then the 16 waves in LDS
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            float v = acc[m][e] + zacc[m];
#pragma unroll
            for (int off = WPB; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            acc[m][e] = v;
        }
    __syncthreads();
    float* red = (float*)smem;  // [NWAVES][WPB][PER] per activation row
    // unrolled over the kernel's rows so acc[m] is a register, not a
    // dynamically indexed (scratch) array; rows past M stop (uniformly)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= a.M) break;
        if (rr == 0) {
#pragma unroll
            for (int e = 0; e < PER; ++e) red[(wv * WPB + cl) * PER + e] = acc[m][e];
        }
        __syncthreads();
        for (int o = tid; o < WPB * PER; o += 64 * NWAVES) {
            const int l = o / PER, e = o - l * PER;
            const int cc = cb * WPB + l;
            float v = 0.f;
#pragma unroll 4
            for (int w = 0; w < NWAVES; ++w) v += red[(w * WPB + l) * PER + e];
            if (cc < wcols)
                a.y[(size_t)m * N + cc * PER + e] = (uint16_t)f32_to_bf16_rne(add_out_bias(a.ob, cc * PER + e, v));
        }
        __syncthreads();
    }
}

// activation rows rounded up to the kernel's MR (1, 2, 4 or 8)
inline int nt_mr(int M) { return M <= 2 ? M : (M <= 4 ? 4 : 8); }

#ifndef QLIN_NT_WPB
#define QLIN_NT_WPB 8
#endif
#ifndef QLIN_NT_NW
#define QLIN_NT_NW 16
#endif

// waves per workgroup: 16 for up to 4 activation rows, 8 for more (the
// register ring then holds more accumulators per lane)
inline int nt_waves(int M) { return nt_mr(M) == 8 ? 8 : QLIN_NT_NW; }

inline size_t nt_shm(int M, int K, int per) {
    const int wpb = QLIN_NT_WPB;
    const size_t red_bytes = (size_t)nt_waves(M) * wpb * per * 4;
    const size_t stage = (size_t)nt_mr(M) * K * 2;
    return stage > red_bytes ? stage : red_bytes;
}

template <int MODE, int BITS, int G>
hipError_t launch_fmt(const QmmArgs& q, hipStream_t st) {
    NtArgs a;
    a.x = (const uint16_t*)q.x;
    a.wq = q.wq;
    a.scales = q.scales;
    a.biases = (const uint16_t*)q.biases;
    a.y = (uint16_t*)q.y;
    a.ob = q.ob;
    a.M = (int)q.M;
    a.N = (int)q.N;
    a.K = (int)q.K;
    constexpr int PER = 32 / BITS;
    const int wcols = a.N / PER;
    constexpr int WPB = QLIN_NT_WPB, NW = QLIN_NT_NW;
    const unsigned blocks = (unsigned)((wcols + WPB - 1) / WPB);
    const size_t shm = nt_shm(a.M, a.K, PER);
    auto run = [&](auto kern, int nw) -> hipError_t {
        if (shm > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            if (e != hipSuccess) return e;
        }
        kern<<<blocks, 64 * nw, shm, st>>>(a);
        return hipGetLastError();
    };
    switch (nt_mr(a.M)) {
    case 1: return run(qmm_nt_kernel<MODE, BITS, G, 1, WPB, NW>, NW);
    case 2: return run(qmm_nt_kernel<MODE, BITS, G, 2, WPB, NW>, NW);
    case 4: return run(qmm_nt_kernel<MODE, BITS, G, 4, WPB, NW>, NW);
    default: return run(qmm_nt_kernel<MODE, BITS, G, 8, WPB, 8>, 8);
    }
}

}  // namespace

bool qmm_nt_supports(const QmmArgs& q) {
    if (q.transpose || q.x_dtype != QLIN_BF16 || q.R != 0) return false;
    if (q.M < 1 || q.M > 8) return false;
    if (q.K > (1 << 20) || q.N > (1 << 28)) return false;
    if (q.K % 8 != 0 || ((uintptr_t)q.x & 15) != 0) return false;
    return nt_shm((int)q.M, (int)q.K, 32 / q.bits) <= 150 * 1024;
}

hipError_t launch_qmm_nt(const QmmArgs& q, hipStream_t st) {
    if (!qmm_nt_supports(q)) return hipErrorNotSupported;
    switch (q.mode) {
    case MXFP4: return launch_fmt<MXFP4, 4, 32>(q, st);
    case NVFP4: return launch_fmt<NVFP4, 4, 16>(q, st);
    case MXFP8: return launch_fmt<MXFP8, 8, 32>(q, st);
    default: break;
    }
    if (q.bits == 4) {
        if (q.group_size == 32) return launch_fmt<AFFINE, 4, 32>(q, st);
        if (q.group_size == 64) return launch_fmt<AFFINE, 4, 64>(q, st);
        return launch_fmt<AFFINE, 4, 128>(q, st);
    }
    if (q.bits == 8) {
        if (q.group_size == 32) return launch_fmt<AFFINE, 8, 32>(q, st);
        if (q.group_size == 64) return launch_fmt<AFFINE, 8, 64>(q, st);
        return launch_fmt<AFFINE, 8, 128>(q, st);
    }
    if (q.group_size == 32) return launch_fmt<AFFINE, 2, 32>(q, st);
    if (q.group_size == 64) return launch_fmt<AFFINE, 2, 64>(q, st);
    return launch_fmt<AFFINE, 2, 128>(q, st);
}

}  // namespace qlin
