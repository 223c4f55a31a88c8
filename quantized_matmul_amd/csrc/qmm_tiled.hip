// qmm_tiled.hip -- LDS-tiled MFMA quantized matmul for many rows, plain or
// expert-gathered (gfx950).
//
// y = x . dequant(W)^T for the [out, in] layout with bf16 activations
// ("EMLX.Quantization", quantized_matmul) -- the prefill case, which is a
// dense contraction -- and its mixture-of-experts form
// ("EMLX.Quantization", gather_quantized_matmul): rows are bucketed by
// expert on the device (gather_index.hip) and every expert's weight tile
// is read in place once per row tile, never copied per row.
//
// Per K-iteration (64 k) a workgroup of 256 threads:
//   * loads its W tile (BN rows x 64 k, packed) with 128-bit loads and
//     dequantizes it once into LDS as bf16: affine w = fmaf(s, q, z) rounded
//     to nearest-even bf16; microscaled codes are decoded and scaled exactly
//     (v_cvt_scalef32_pk_bf16_fp4/_fp8 for E8M0 scales, a unit-scale decode
//     plus an fp32 multiply for nvfp4's E4M3 scale);
//   * loads its x tile (BM rows x 64 k, bf16) into LDS (gathered rows for
//     the expert form);
//   * runs v_mfma_f32_16x16x32_bf16 with W as the A operand and x as the B
//     operand, so each lane ends with 4 consecutive output columns of one row
//     (8-byte stores);
// with the next tile's global loads in flight during the MFMAs (double-
// buffered LDS). Accumulation is fp32.

#include "qlin_common.h"

#include <atomic>

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BK = 64;                 // k per iteration
constexpr int LROW = BK * 2 + 16;      // LDS row pitch in bytes (padded against bank conflicts)
constexpr int NTHREADS = 256;

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, nearest-even
    return __builtin_bit_cast(uint32_t, r);
}

struct TiledArgs {
    const uint16_t* x;       // bf16 [rows, K]
    const uint32_t* wq;      // [E][N][K/PER]
    const void* scales;      // [E][N][K/G]
    const uint16_t* biases;
    uint16_t* y;             // bf16
    int M, N, K;             // M: activation rows per index row (gather) or total rows
    // gather form
    const uint32_t* lhs;     // [R] or null
    const uint32_t* perm;    // [R] index rows sorted by expert (null: plain matmul)
    const uint32_t* offsets; // [E+1] index-row offsets per expert
    const uint32_t* tiles;   // [E+1] row-tile prefix per expert
    int E;
    int B;                   // activation batch entries (lhs values must be below)
    OutBias ob;              // dense-layer bias (plain form)
};

// Dequantize one 16-byte chunk of packed codes (128/BITS codes starting at
// global k index k0 of weight row `row`) into bf16 pairs, natural k order.
template <int MODE, int BITS, int G>
__device__ __forceinline__ void dequant_chunk(const u32x4 w, const void* scales,
                                              const uint16_t* biases, size_t srow, int k0,
                                              uint32_t* out /* [64/BITS] */) {
    constexpr int PER = 32 / BITS;
    constexpr int CODES = 4 * PER;
    if constexpr (MODE == AFFINE) {
        // codes of a chunk span ceil(CODES/G) groups
        constexpr int NG = CODES > G ? CODES / G : 1;
        float s[NG], z[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const size_t gi = srow + (k0 + g * G) / G;
            s[g] = bf16_bits_to_f32(((const uint16_t*)scales)[gi]);
            z[g] = bf16_bits_to_f32(biases[gi]);
        }
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            uint32_t v = w[wd];
            float f[PER];
            if constexpr (BITS == 4) {
                const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
                    f[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
                }
            } else if constexpr (BITS == 8) {
#pragma unroll
                for (int b = 0; b < 4; ++b) f[b] = (float)((v >> (8 * b)) & 0xFFu);
            } else {
                const uint32_t b0 = v & 0x03030303u, b1 = (v >> 2) & 0x03030303u,
                               b2 = (v >> 4) & 0x03030303u, b3 = (v >> 6) & 0x03030303u;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f[4 * b] = (float)((b0 >> (8 * b)) & 0xFFu);
                    f[4 * b + 1] = (float)((b1 >> (8 * b)) & 0xFFu);
                    f[4 * b + 2] = (float)((b2 >> (8 * b)) & 0xFFu);
                    f[4 * b + 3] = (float)((b3 >> (8 * b)) & 0xFFu);
                }
            }
#pragma unroll
            for (int e = 0; e < PER; e += 2) {
                const int c0 = wd * PER + e;  // code index within the chunk
                const int g0 = (NG == 1) ? 0 : c0 / G;
                const float d0 = __builtin_fmaf(s[g0], f[e], z[g0]);
                const float d1 = __builtin_fmaf(s[g0], f[e + 1], z[g0]);
                out[c0 / 2] = pack_bf16(d0, d1);
            }
        }
    } else {
        // microscaled: one scale byte per group; chunks never straddle more than
        // CODES/G groups; decode and scale in one instruction
        constexpr int NG = CODES / G;  // mxfp4: 1, nvfp4: 2, mxfp8: 1 (16 codes)
        float sc[NG > 0 ? NG : 1];
#pragma unroll
        for (int g = 0; g < (NG > 0 ? NG : 1); ++g) {
            const uint32_t byte = ((const uint8_t*)scales)[srow + (k0 + g * G) / G];
            sc[g] = MODE == NVFP4 ? e4m3_to_f32(byte) : e8m0_to_f32(byte);
        }
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            const uint32_t v = w[wd];
            if constexpr (MODE == NVFP4) {
                // the scaled convert applies only the exponent of its scale:
                // decode with unit scale, multiply by the E4M3 scale in fp32
                const float s = sc[(wd * 8) / G];
                out[wd * 4 + 0] = e2m1_pair_times<0>(v, s);
                out[wd * 4 + 1] = e2m1_pair_times<1>(v, s);
                out[wd * 4 + 2] = e2m1_pair_times<2>(v, s);
                out[wd * 4 + 3] = e2m1_pair_times<3>(v, s);
            } else if constexpr (BITS == 4) {
                const float s = sc[(wd * 8) / G < NG ? (wd * 8) / G : 0];
                out[wd * 4 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 0));
                out[wd * 4 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 1));
                out[wd * 4 + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 2));
                out[wd * 4 + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, s, 3));
            } else {
                const float s = sc[0];
                out[wd * 2 + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, s, false));
                out[wd * 2 + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, s, true));
            }
        }
    }
}

// BM x BN tile per workgroup, WM x WN waves; each wave owns (BM/WM) rows of
// x and (BN/WN) columns of W.
template <int MODE, int BITS, int G, int BM, int BN, int WM, int WN, bool GATHER>
__global__ void __launch_bounds__(NTHREADS) qmm_tiled_kernel(TiledArgs a) {
    constexpr int PER = 32 / BITS;
    constexpr int WROWB = BK * BITS / 8;               // packed bytes per W row per iteration
    constexpr int WCH = WROWB / 16;                    // 16-byte chunks per W row (1, 2 or 4)
    constexpr int WCHUNKS = BN * WCH;                  // chunks per W tile
    constexpr int WPT = (WCHUNKS + NTHREADS - 1) / NTHREADS;
    constexpr int XCHUNKS = BM * (BK * 2 / 16);        // 16-byte chunks per x tile
    constexpr int XPT = XCHUNKS / NTHREADS;
    constexpr int MW = BM / WM, NW = BN / WN;          // wave tile
    constexpr int MT = MW / 16, NT = NW / 16;
    constexpr int CODES = 128 / BITS;                  // codes per 16-byte chunk
    static_assert(XCHUNKS % NTHREADS == 0, "x tile must split evenly");
    static_assert(WM * WN == NTHREADS / 64, "4 waves");

    extern __shared__ __align__(16) unsigned char smem[];
    // LDS: x tiles [2][BM][LROW], then W tiles [2][BN][LROW]
    auto xs = [&](int b) { return smem + b * (BM * LROW); };
    auto ws = [&](int b) { return smem + 2 * BM * LROW + b * (BN * LROW); };

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int i = lane & 15, j = lane >> 4;
    const int wm = wv / WN, wn = wv % WN;

    // ---- which tile: plain (m-tile, n-tile) or (expert, row tile, n-tile)
    const int ntiles_n = (a.N + BN - 1) / BN;
    int tile_m = blockIdx.x / ntiles_n;
    const int tile_n = blockIdx.x % ntiles_n;
    int expert = 0, row_begin = 0, row_count = a.M;  // GEMM rows of this expert
    if constexpr (GATHER) {
        if (tile_m >= (int)a.tiles[a.E]) return;       // beyond the real tile count
        int lo = 0, hi = a.E;                          // find e: tiles[e] <= tile_m < tiles[e+1]
        while (hi - lo > 1) {
            int mid = (lo + hi) >> 1;
            if ((int)a.tiles[mid] <= tile_m) lo = mid; else hi = mid;
        }
        expert = lo;
        tile_m -= (int)a.tiles[lo];
        row_begin = (int)a.offsets[lo];
        row_count = ((int)a.offsets[lo + 1] - row_begin) * a.M;
    }
    const int m0 = tile_m * BM;   // first GEMM row of the tile (within the expert)
    const int n0 = tile_n * BN;

    // GEMM row rho (within expert) -> x row and y row
    auto map_row = [&](int rho, int& xrow, int& yrow) {
        if constexpr (GATHER) {
            const int ir = (int)a.perm[row_begin + rho / a.M];
            const int mm = rho % a.M;
            int b = a.lhs ? (int)a.lhs[ir] : ir;
            if ((unsigned)b >= (unsigned)a.B) b = 0;   // precondition broken: stay in x
            xrow = b * a.M + mm;
            yrow = ir * a.M + mm;
        } else {
            xrow = rho;
            yrow = rho;
        }
    };

    // ---- per-thread x chunk sources (fixed over K)
    const uint16_t* xsrc[XPT];
    bool xvalid[XPT];
#pragma unroll
    for (int p = 0; p < XPT; ++p) {
        const int c = tid + p * NTHREADS;
        const int r = c / (BK * 2 / 16), cc = c % (BK * 2 / 16);
        const int rho = m0 + r;
        xvalid[p] = rho < row_count;
        int xrow = 0, yrow = 0;
        if (xvalid[p]) map_row(rho, xrow, yrow);
        xsrc[p] = a.x + (size_t)xrow * a.K + cc * 8;
    }
    // ---- per-thread W chunk sources
    const size_t wrow_words = a.K / PER, srow_groups = a.K / G;
    const uint32_t* wsrc[WPT];
    size_t srow[WPT];
    int wkoff[WPT];
    bool wactive[WPT];
#pragma unroll
    for (int p = 0; p < WPT; ++p) {
        const int c = tid + p * NTHREADS;
        wactive[p] = c < WCHUNKS;
        const int r = wactive[p] ? c / WCH : 0, cc = c % WCH;
        int n = n0 + r;
        n = n < a.N ? n : a.N - 1;
        const size_t erow = (size_t)expert * a.N + n;
        wsrc[p] = a.wq + erow * wrow_words + cc * 4;
        srow[p] = erow * srow_groups;
        wkoff[p] = cc * CODES;
    }

    u32x4 xreg[XPT], wreg[WPT];
    auto gload = [&](int kt) {
#pragma unroll
        for (int p = 0; p < XPT; ++p)
            xreg[p] = xvalid[p] ? *(const u32x4*)(xsrc[p] + kt * BK) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int p = 0; p < WPT; ++p)
            if (wactive[p]) wreg[p] = *(const u32x4*)(wsrc[p] + (size_t)kt * (BK / PER));
    };
    auto lstore = [&](int buf, int kt) {
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int c = tid + p * NTHREADS;
            const int r = c / (BK * 2 / 16), cc = c % (BK * 2 / 16);
            *(u32x4*)(xs(buf) + r * LROW + cc * 16) = xreg[p];
        }
#pragma unroll
        for (int p = 0; p < WPT; ++p) {
            if (!wactive[p]) continue;
            const int c = tid + p * NTHREADS;
            const int r = c / WCH;
            uint32_t o[CODES / 2];
            dequant_chunk<MODE, BITS, G>(wreg[p], a.scales, a.biases, srow[p], kt * BK + wkoff[p], o);
            unsigned char* dst = ws(buf) + r * LROW + wkoff[p] * 2;
#pragma unroll
            for (int q = 0; q < CODES / 8; ++q)
                *(u32x4*)(dst + q * 16) = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
        }
    };

    // accumulators start at zero, or at the dense-layer bias of the lane's
    // output columns n = n0 + wn*NW + 16t + 4j + r (added once per output;
    // the output stage is the plain matmul's)
    f32x4 acc[NT][MT];
    if (a.ob.kind == OB_NONE) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int s = 0; s < MT; ++s) acc[t][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 b;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n0 + wn * NW + t * 16 + 4 * j + r;
                b[r] = n < a.N ? out_bias_at(a.ob, n) : 0.f;
            }
#pragma unroll
            for (int s = 0; s < MT; ++s) acc[t][s] = b;
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // bias loads before the tile loads

    const int nk = a.K / BK;
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int kh = 0; kh < BK / 32; ++kh) {
            u32x4 af[NT], bfr[MT];
#pragma unroll
            for (int t = 0; t < NT; ++t)
                af[t] = *(const u32x4*)(ws(buf) + (wn * NW + t * 16 + i) * LROW + (kh * 32 + 8 * j) * 2);
#pragma unroll
            for (int s = 0; s < MT; ++s)
                bfr[s] = *(const u32x4*)(xs(buf) + (wm * MW + s * 16 + i) * LROW + (kh * 32 + 8 * j) * 2);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int s = 0; s < MT; ++s) acc[t][s] = mfma_bf16(af[t], bfr[s], acc[t][s]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1, kt + 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds D[n = 4j + r][m = i] of each (t, s) tile
#pragma unroll
    for (int s = 0; s < MT; ++s) {
        const int rho = m0 + wm * MW + s * 16 + i;
        if (rho >= row_count) continue;
        int xrow, yrow;
        map_row(rho, xrow, yrow);
        uint16_t* yr = a.y + (size_t)yrow * a.N;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = n0 + wn * NW + t * 16 + 4 * j;
            const f32x4 v = acc[t][s];
            if (n + 3 < a.N && ((a.N & 3) == 0)) {
                uint2 pk;
                pk.x = pack_bf16(v[0], v[1]);
                pk.y = pack_bf16(v[2], v[3]);
                *(uint2*)(yr + n) = pk;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < a.N) yr[n + r] = (uint16_t)f32_to_bf16_rne(v[r]);
            }
        }
    }
}

template <int MODE, int BITS, int G, int BM, int BN, int WM, int WN, bool GATHER>
hipError_t launch_cfg(const TiledArgs& t, int grid, hipStream_t st) {
    const size_t shm = (size_t)2 * (BM + BN) * LROW;
    auto kern = qmm_tiled_kernel<MODE, BITS, G, BM, BN, WM, WN, GATHER>;
    // one kernel per instantiation: the attribute is set once (an atomic
    // flag, so concurrent callers at worst set it twice)
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    kern<<<grid, NTHREADS, shm, st>>>(t);
    return hipGetLastError();
}

constexpr int GATHER_BM = kTiledGatherRows;

template <int MODE, int BITS, int G>
hipError_t launch_fmt(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                      hipStream_t st) {
    TiledArgs t{};
    t.x = (const uint16_t*)q.x;
    t.wq = q.wq;
    t.scales = q.scales;
    t.biases = (const uint16_t*)q.biases;
    t.y = (uint16_t*)q.y;
    t.M = (int)q.M;
    t.N = (int)q.N;
    t.K = (int)q.K;
    t.ob = q.ob;
    if (q.R == 0) {
        constexpr int BM = 256, BN = 128;
        const int grid = (int)(((q.M + BM - 1) / BM) * ((q.N + BN - 1) / BN));
        return launch_cfg<MODE, BITS, G, BM, BN, 2, 2, false>(t, grid, st);
    }
    t.lhs = q.lhs;
    t.perm = perm;
    t.offsets = offsets;
    t.tiles = offsets + (q.E + 1);
    t.E = (int)q.E;
    t.B = (int)q.batch_x;
    constexpr int BM = GATHER_BM, BN = 256;
    // upper bound on row tiles: every expert may add one partial tile
    const int64_t mt = (q.R * q.M + BM - 1) / BM + q.E;
    const int grid = (int)(mt * ((q.N + BN - 1) / BN));
    return launch_cfg<MODE, BITS, G, BM, BN, 1, 4, true>(t, grid, st);
}

}  // namespace

bool qmm_tiled_supports(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16) return false;
    if (q.K % BK != 0 || q.K > (1 << 24)) return false;
    if (q.R > 0 && (q.E > 8192 || q.R * q.M >= (1LL << 30))) return false;
    if (((uintptr_t)q.wq & 15) || ((uintptr_t)q.x & 15)) return false;
    return true;
}

hipError_t launch_qmm_tiled(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                            hipStream_t st) {
    if (!qmm_tiled_supports(q)) return hipErrorNotSupported;
    if (q.R > 0 && (!perm || !offsets)) return hipErrorInvalidValue;
    switch (q.mode) {
    case MXFP4: return launch_fmt<MXFP4, 4, 32>(q, perm, offsets, st);
    case NVFP4: return launch_fmt<NVFP4, 4, 16>(q, perm, offsets, st);
    case MXFP8: return launch_fmt<MXFP8, 8, 32>(q, perm, offsets, st);
    default: break;
    }
    if (q.bits == 4) {
        if (q.group_size == 32) return launch_fmt<AFFINE, 4, 32>(q, perm, offsets, st);
        if (q.group_size == 64) return launch_fmt<AFFINE, 4, 64>(q, perm, offsets, st);
        return launch_fmt<AFFINE, 4, 128>(q, perm, offsets, st);
    }
    if (q.bits == 8) {
        if (q.group_size == 32) return launch_fmt<AFFINE, 8, 32>(q, perm, offsets, st);
        if (q.group_size == 64) return launch_fmt<AFFINE, 8, 64>(q, perm, offsets, st);
        return launch_fmt<AFFINE, 8, 128>(q, perm, offsets, st);
    }
    if (q.group_size == 32) return launch_fmt<AFFINE, 2, 32>(q, perm, offsets, st);
    if (q.group_size == 64) return launch_fmt<AFFINE, 2, 64>(q, perm, offsets, st);
    return launch_fmt<AFFINE, 2, 128>(q, perm, offsets, st);
}

}  // namespace qlin
