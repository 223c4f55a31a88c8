// qmm_decode.hip -- small-M quantized matmul on the MFMA cores (gfx950).
//
// y[m, n] = sum_k x[m, k] * dequant(W)[n, k] for M <= 16 rows and the
// [out, in] layout ("EMLX.Quantization", quantized_matmul; "Emily.Quantization.
// Layers", quantized_dense with transpose true), bf16 activations and output.
// This is the decode case the layer page calls the single-kernel path: the
// packed weight is streamed once from HBM and never written back dense.
//
// Design (one workgroup = KS waves x CB column blocks of 16 output columns):
//  * x [M, K] is staged once per workgroup into LDS, already permuted into
//    the order the weight codes are unpacked in, so every MFMA A-fragment is
//    one ds_read_b128. Rows >= M read a zero row.
//  * Each wave owns a K-slice and streams its 16-row weight blocks with
//    128-bit loads (lane (i, j) reads 16 bytes of row i), prefetched PF units
//    ahead; a 4x4 word transpose across the four lane rows (permlane16/32
//    swaps) gives each lane the words one MFMA K-step needs, so every 32-wide
//    K-step stays inside one quantization group.
//  * Affine codes become exact bf16 values 128+q with two bit operations per
//    pair. One MFMA accumulates sum x*(128+q) per group and a second MFMA
//    against an all-ones operand accumulates sum x over the same group, so
//    the group's scale s and bias z are applied once per group and row:
//        y += s * acc + (z - 128 s) * sum_x.
//    (8-bit codes are converted exactly with the byte-to-float instructions.)
//  * Microscaled codes are decoded and multiplied by their per-group scale
//    before the MFMA, exactly in bf16, so one MFMA chain accumulates the whole
//    K-slice: one gfx950 instruction (v_cvt_scalef32_pk_bf16_fp4 / _fp8) for
//    the power-of-two E8M0 scales of mxfp4/mxfp8; for nvfp4's E4M3 scale a
//    unit-scale decode and an fp32 multiply (the scaled convert applies only
//    the exponent of its scale operand).
//  * Partial sums of the KS K-slices meet in LDS; fp32 accumulation.
//  * 2-bit codes with 32-element groups: one K-step spans two groups, so the
//    MFMA rows are split into two slots of 8 rows (block-diagonal A), which
//    limits that case to M <= 8.

#include "qlin_common.h"

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 4x4 word transpose across the lane rows j = lane/16:
// before, lane row j holds v[c] = W[j][c]; after, v[c] = W[c][j].
__device__ __forceinline__ void xpose4(u32x4& v) {
    auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    v[0] = a[0];
    v[2] = a[1];
    auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    v[1] = b[0];
    v[3] = b[1];
    auto c = __builtin_amdgcn_permlane16_swap(v[0], v[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    auto d = __builtin_amdgcn_permlane16_swap(v[2], v[3], false, false);
    v[2] = d[0];
    v[3] = d[1];
}

// Compile-time description of one (mode, bits, group) case.
template <int MODE, int BITS, int G>
struct Fmt {
    static constexpr int PER = 32 / BITS;          // codes per word
    static constexpr int RK = 16 * PER;            // k per region (16 words per row)
    static constexpr int SPR = RK / 32;            // MFMA K-steps per region
    static constexpr int U = RK > G ? RK : G;      // k per unit (scale prefetch granule)
    static constexpr int RPU = U / RK;             // regions per unit
    static constexpr int GPU = U / G;              // groups per unit
    static constexpr bool AFF = MODE == AFFINE;
    static constexpr int S = (AFF && BITS == 2 && G == 32) ? 2 : 1;  // row slots
    static constexpr int WS = S == 2 ? 2 : (G >= 32 ? G / 32 : 1);   // steps per window
    static constexpr float OFF = (AFF && BITS != 8) ? 128.0f : 0.0f;  // code offset
    static constexpr int WPU = (RPU * SPR) / WS;   // affine windows per unit
    static constexpr int STEPS = RPU * SPR;        // MFMA K-steps per unit

    // k (within the 32- or 64-wide block of global step gs) of element e of
    // the A/B fragment held by lane row j. Must match unpack() below.
    __device__ static int chunk_k(int gs, int j, int e) {
        if constexpr (BITS == 4 && AFF) {
            const int perm[8] = {0, 4, 1, 5, 2, 6, 3, 7};
            return 8 * (4 * gs + j) + perm[e];
        } else if constexpr (BITS == 4) {
            return 8 * (4 * gs + j) + e;  // fp4 pairs decode in natural order
        } else if constexpr (BITS == 8) {
            return 32 * gs + (e < 4 ? 4 * j + e : 16 + 4 * j + (e - 4));
        } else {  // 2-bit: steps (c, h) of a 64-wide block b, gs = 2b + h
            const int perm[2][8] = {{0, 8, 1, 9, 2, 10, 3, 11}, {4, 12, 5, 13, 6, 14, 7, 15}};
            int b = gs >> 1, h = gs & 1;
            return 16 * (4 * b + j) + perm[h][e];
        }
    }
};

// Unpack step t of a region into an MFMA B operand. `w` holds the lane's
// four words after xpose4 (word 4c + j of the region in w[c]); `sc` is the
// fp32 decode scale of the step (microscaled only).
template <int MODE, int BITS, int G>
__device__ __forceinline__ u32x4 unpack(const u32x4& w, int t, float sc) {
    u32x4 b;
    if constexpr (MODE == AFFINE && BITS == 4) {
        const uint32_t v = w[t], M4 = 0x000F000Fu, MAG = 0x43004300u;
        b[0] = (v & M4) | MAG;
        b[1] = ((v >> 4) & M4) | MAG;
        b[2] = ((v >> 8) & M4) | MAG;
        b[3] = ((v >> 12) & M4) | MAG;
    } else if constexpr (MODE == AFFINE && BITS == 2) {
        const uint32_t v = w[t >> 1], M2 = 0x00030003u, MAG = 0x43004300u;
        const int s0 = (t & 1) * 4;  // pairs (s, s+8) for s = s0 .. s0+3
        b[0] = ((v >> (2 * s0)) & M2) | MAG;
        b[1] = ((v >> (2 * s0 + 2)) & M2) | MAG;
        b[2] = ((v >> (2 * s0 + 4)) & M2) | MAG;
        b[3] = ((v >> (2 * s0 + 6)) & M2) | MAG;
    } else if constexpr (MODE == AFFINE && BITS == 8) {
        // byte -> fp32 (v_cvt_f32_ubyteN) -> packed bf16 (v_cvt_pk_bf16_f32); exact
        const uint32_t va = w[2 * t], vb = w[2 * t + 1];
        auto pk = [](uint32_t v, int sh) {
            bf16x2 r = {(__bf16)(float)((v >> sh) & 0xFFu), (__bf16)(float)((v >> (sh + 8)) & 0xFFu)};
            return __builtin_bit_cast(uint32_t, r);
        };
        b[0] = pk(va, 0);
        b[1] = pk(va, 16);
        b[2] = pk(vb, 0);
        b[3] = pk(vb, 16);
    } else if constexpr (MODE == NVFP4) {
        // E2M1 x E4M3 scale. The scaled convert instruction applies only the
        // exponent of its scale operand (MX semantics), so decode with unit
        // scale and multiply in fp32 (exact: at most 6 significant bits).
        const uint32_t v = w[t];
        b[0] = e2m1_pair_times<0>(v, sc);
        b[1] = e2m1_pair_times<1>(v, sc);
        b[2] = e2m1_pair_times<2>(v, sc);
        b[3] = e2m1_pair_times<3>(v, sc);
    } else if constexpr (BITS == 4) {  // mxfp4: E2M1 x E8M0 (power-of-two) scale
        const uint32_t v = w[t];
        b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 0));
        b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 1));
        b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 2));
        b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, sc, 3));
    } else {  // mxfp8: E4M3 x scale
        const uint32_t va = w[2 * t], vb = w[2 * t + 1];
        b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(va, sc, false));
        b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(va, sc, true));
        b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vb, sc, false));
        b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vb, sc, true));
    }
    return b;
}

template <int MODE>
__device__ __forceinline__ float scale_byte_to_f32(uint32_t byte) {
    return MODE == NVFP4 ? e4m3_to_f32(byte) : e8m0_to_f32(byte);
}

struct DecodeArgs {
    const uint16_t* x;   // bf16 [M, K]
    const uint32_t* wq;  // [N, K/PER]
    const void* scales;  // bf16 [N, K/G] (affine) or u8
    const uint16_t* biases;
    uint16_t* y;         // bf16 [M, N]
    int M, N, K;
};

// LDS layout: (M+1) rows of K/8 16-byte chunks (row M is zero), each row
// padded by 16 bytes, then the cross-wave reduction buffer.
__host__ __device__ constexpr int xrow_bytes(int K) { return K * 2 + 16; }

template <int MODE, int BITS, int G, int CB, int KS, int MREG, int PF>
__global__ void __launch_bounds__(64 * KS) qmm_decode_kernel(DecodeArgs a) {
    using F = Fmt<MODE, BITS, G>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int i = lane & 15, j = lane >> 4;
    const int K = a.K, M = a.M;
    const int rowb = xrow_bytes(K);
    const int nchunks = K / 8;

    // ---- stage x into LDS in fragment order (row M = zeros)
    for (int idx = tid; idx < (M + 1) * nchunks; idx += 64 * KS) {
        const int r = idx / nchunks, q = idx - r * nchunks;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < M) {
            const int gs = q >> 2, jj = q & 3;
            const uint16_t* xr = a.x + (size_t)r * K;
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = xr[F::chunk_k(gs, jj, e)];
            v[0] = h[0] | (h[1] << 16);
            v[1] = h[2] | (h[3] << 16);
            v[2] = h[4] | (h[5] << 16);
            v[3] = h[6] | (h[7] << 16);
        }
        *(u32x4*)(smem + r * rowb + q * 16) = v;
    }
    float* red = (float*)(smem + (M + 1) * rowb);  // [KS][CB][16 rows][16 cols]
    __syncthreads();

    // ---- this lane's A row (zero row when it carries no real x row)
    int arow;
    if constexpr (F::S == 2) arow = (i / 8 == j / 2 && (i & 7) < M) ? (i & 7) : M;
    else arow = (i < M) ? i : M;
    const unsigned char* abase = smem + arow * rowb + j * 16;

    // ---- K-slice of this wave, in units of F::U
    const int nunits = K / F::U;
    const int u0 = (wv * nunits) / KS, u1 = ((wv + 1) * nunits) / KS;
    const int n0 = blockIdx.x * (16 * CB);
    const int wpr = K / F::PER;           // words per weight row
    const int gpr = K / G;                // groups per weight row
    const uint32_t* wrow[CB];
    int ncol[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        int n = n0 + 16 * c + i;
        ncol[c] = n < a.N ? n : a.N - 1;  // ragged N: re-read the last row, never stored
        wrow[c] = a.wq + (size_t)ncol[c] * wpr + 4 * j;
    }

    // prefetch ring: PF units of weights and scale data per column block.
    // Affine: per window, the scale/bias (bf16 bits) of this lane's group.
    // Microscaled: per K-step, the scale byte of this lane's 8 codes.
    constexpr int NSC = F::AFF ? F::WPU : F::STEPS;
    u32x4 wbuf[PF][CB][F::RPU];
    uint32_t sbuf[PF][CB][NSC];
    uint32_t zbuf[PF][CB][F::AFF ? NSC : 1];
    auto issue = [&](int slot, int u) {
#pragma unroll
        for (int c = 0; c < CB; ++c) {
#pragma unroll
            for (int r = 0; r < F::RPU; ++r)
                wbuf[slot][c][r] = *(const u32x4*)(wrow[c] + (size_t)(u * F::RPU + r) * 16);
            const size_t rowg = (size_t)ncol[c] * gpr;
#pragma unroll
            for (int w = 0; w < NSC; ++w) {
                if constexpr (F::AFF) {
                    const int grp = u * F::GPU + (F::S == 2 ? 2 * w + (j >> 1) : w);
                    sbuf[slot][c][w] = ((const uint16_t*)a.scales)[rowg + grp];
                    zbuf[slot][c][w] = a.biases[rowg + grp];
                } else {
                    const int gs = u * F::STEPS + w;
                    const int grp = F::chunk_k(gs, j, 0) / G;
                    sbuf[slot][c][w] = ((const uint8_t*)a.scales)[rowg + grp];
                }
            }
        }
    };

    f32x4 acc[CB], dsum = {0.f, 0.f, 0.f, 0.f};
    float ysum[CB][MREG];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        acc[c] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < MREG; ++r) ysum[c][r] = 0.f;
    }
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (u0 + p < u1) issue(p, u0 + p);

    for (int ub = u0; ub < u1; ub += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int u = ub + p;
            if (u < u1) {
#pragma unroll
                for (int c = 0; c < CB; ++c)
#pragma unroll
                    for (int r = 0; r < F::RPU; ++r) xpose4(wbuf[p][c][r]);
#pragma unroll
                for (int r = 0; r < F::RPU; ++r) {
#pragma unroll
                    for (int t = 0; t < F::SPR; ++t) {
                        const int ls = r * F::SPR + t;               // step within unit
                        const int gs = (u * F::RPU + r) * F::SPR + t;  // global step
                        const u32x4 av = *(const u32x4*)(abase + gs * 64);
                        const bool first = F::AFF && (ls % F::WS == 0);
                        if constexpr (F::AFF) {
                            dsum = mfma_bf16(av, ones, first ? f32x4{0.f, 0.f, 0.f, 0.f} : dsum);
                        }
#pragma unroll
                        for (int c = 0; c < CB; ++c) {
                            float sc = 0.f;
                            if constexpr (!F::AFF) sc = scale_byte_to_f32<MODE>(sbuf[p][c][ls]);
                            const u32x4 bv = unpack<MODE, BITS, G>(wbuf[p][c][r], t, sc);
                            acc[c] = mfma_bf16(av, bv, first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[c]);
                        }
                        if constexpr (F::AFF) {
                            if (ls % F::WS == F::WS - 1) {
                                // window done: apply the group's scale and bias
#pragma unroll
                                for (int c = 0; c < CB; ++c) {
                                    const int wi = ls / F::WS;
                                    const float s = bf16_bits_to_f32(sbuf[p][c][wi]);
                                    const float z = bf16_bits_to_f32(zbuf[p][c][wi]);
                                    const float zz = __builtin_fmaf(-F::OFF, s, z);
#pragma unroll
                                    for (int rr = 0; rr < MREG; ++rr) {
                                        ysum[c][rr] = __builtin_fmaf(s, acc[c][rr], ysum[c][rr]);
                                        ysum[c][rr] = __builtin_fmaf(zz, dsum[rr], ysum[c][rr]);
                                    }
                                }
                            }
                        }
                    }
                }
                if (u + PF < u1) issue(p, u + PF);
            }
        }
    }
    if constexpr (!F::AFF) {
#pragma unroll
        for (int c = 0; c < CB; ++c)
#pragma unroll
            for (int rr = 0; rr < MREG; ++rr) ysum[c][rr] = acc[c][rr];
    }

    // ---- cross-wave reduction: red[wv][c][row][col]
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int rr = 0; rr < MREG; ++rr) red[((wv * CB + c) * 16 + 4 * j + rr) * 16 + i] = ysum[c][rr];
    __syncthreads();
    for (int o = tid; o < CB * M * 16; o += 64 * KS) {
        const int c = o / (M * 16), rem = o - c * M * 16, m = rem / 16, col = rem & 15;
        const int n = n0 + 16 * c + col;
        if (n >= a.N) continue;
        // row of MFMA output holding (slot, m)
        float v = 0.f;
        for (int w = 0; w < KS; ++w) {
            if constexpr (F::S == 2) {
                v += red[((w * CB + c) * 16 + m) * 16 + col];
                v += red[((w * CB + c) * 16 + 8 + m) * 16 + col];
            } else {
                v += red[((w * CB + c) * 16 + m) * 16 + col];
            }
        }
        a.y[(size_t)m * a.N + n] = (uint16_t)f32_to_bf16_rne(v);
    }
}

template <int MODE, int BITS, int G>
hipError_t launch_fmt(const QmmArgs& q, hipStream_t st) {
    using F = Fmt<MODE, BITS, G>;
    DecodeArgs a;
    a.x = (const uint16_t*)q.x;
    a.wq = q.wq;
    a.scales = q.scales;
    a.biases = (const uint16_t*)q.biases;
    a.y = (uint16_t*)q.y;
    a.M = (int)q.M;
    a.N = (int)q.N;
    a.K = (int)q.K;
    constexpr int CB = 1, KS = 4, PF = 4;
    const unsigned blocks = (unsigned)((q.N + 16 * CB - 1) / (16 * CB));
    const size_t shm = (size_t)(a.M + 1) * xrow_bytes(a.K) + (size_t)KS * CB * 16 * 16 * 4;
    // rows per lane register that can hold a real output row
    const int mreg = (F::S == 2) ? (a.M > 4 ? 4 : a.M) : (a.M > 4 ? 4 : a.M);
    if (mreg <= 1)
        qmm_decode_kernel<MODE, BITS, G, CB, KS, 1, PF><<<blocks, 64 * KS, shm, st>>>(a);
    else if (mreg == 2)
        qmm_decode_kernel<MODE, BITS, G, CB, KS, 2, PF><<<blocks, 64 * KS, shm, st>>>(a);
    else
        qmm_decode_kernel<MODE, BITS, G, CB, KS, 4, PF><<<blocks, 64 * KS, shm, st>>>(a);
    return hipGetLastError();
}

}  // namespace

bool qmm_decode_supports(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16 || q.R != 0) return false;
    if (q.M < 1 || q.M > 16 || q.N < 1) return false;
    const int per = 32 / q.bits;
    const int rk = 16 * per;
    const int u = rk > q.group_size ? rk : q.group_size;
    if (q.K % u != 0) return false;
    if (q.mode == AFFINE && q.bits == 2 && q.group_size == 32 && q.M > 8) return false;
    if (q.K > (1 << 20)) return false;
    const size_t shm = (size_t)(q.M + 1) * xrow_bytes((int)q.K) + 4 * 16 * 16 * 4;
    if (shm > 96 * 1024) return false;
    // 16-byte aligned weight rows
    if (((uintptr_t)q.wq & 15) != 0) return false;
    return true;
}

hipError_t launch_qmm_decode(const QmmArgs& q, hipStream_t st) {
    if (!qmm_decode_supports(q)) return hipErrorNotSupported;
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
