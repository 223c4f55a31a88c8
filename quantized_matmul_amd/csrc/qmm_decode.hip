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
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

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
    // x elements per fragment-order permutation block
    static constexpr int XBLOCK = (BITS == 4) ? 8 : (BITS == 8 ? 32 : 64);

    // k (within the 32- or 64-wide block of global step gs) of element e of
    // the A/B fragment held by lane row j. Must match unpack() below.
    __device__ static int chunk_k(int gs, int j, int e) {
        if constexpr (BITS == 4 && AFF) {
            const int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
            return 8 * (4 * gs + j) + perm[e];
        } else if constexpr (BITS == 4) {
            return 8 * (4 * gs + j) + e;  // fp4 pairs decode in natural order
        } else if constexpr (BITS == 8) {
            return 32 * gs + (e < 4 ? 4 * j + e : 16 + 4 * j + (e - 4));
        } else {  // 2-bit: steps (c, h) of a 64-wide block b, gs = 2b + h
            const int perm[2][8] = {{0, 4, 1, 5, 2, 6, 3, 7}, {8, 12, 9, 13, 10, 14, 11, 15}};
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
        // nibbles -> bytes (even / odd codes), then v_perm pairs each code
        // byte with 0x43: bf16 0x43nn = 128 + nn exactly.
        const uint32_t v = w[t], C = 0x43434343u;
        const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
        b[0] = __builtin_amdgcn_perm(C, lo, 0x04010400u);  // codes 0, 2
        b[1] = __builtin_amdgcn_perm(C, lo, 0x04030402u);  // codes 4, 6
        b[2] = __builtin_amdgcn_perm(C, hi, 0x04010400u);  // codes 1, 3
        b[3] = __builtin_amdgcn_perm(C, hi, 0x04030402u);  // codes 5, 7
    } else if constexpr (MODE == AFFINE && BITS == 2) {
        // 2-bit codes s, s+4, s+8, s+12 in the bytes of (v >> 2s) & 0x03030303;
        // step half h takes byte pairs (0,1) or (2,3) of the four masks.
        const uint32_t v = w[t >> 1], C = 0x43434343u;
        const uint32_t sel = (t & 1) ? 0x04030402u : 0x04010400u;
        b[0] = __builtin_amdgcn_perm(C, v & 0x03030303u, sel);
        b[1] = __builtin_amdgcn_perm(C, (v >> 2) & 0x03030303u, sel);
        b[2] = __builtin_amdgcn_perm(C, (v >> 4) & 0x03030303u, sel);
        b[3] = __builtin_amdgcn_perm(C, (v >> 6) & 0x03030303u, sel);
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

// Value of another lane of the same DPP row (ctrl: a quad_perm or mirror pattern).
template <int CTRL>
__device__ __forceinline__ float lane_xchg(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 0xF, 0xF, false));
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
    int M, N, K;         // gather: M = GEMM rows per row tile (the tile height)
    int cols;            // output columns per workgroup (<= 16, the MFMA width)
    // gather form (GATHER kernels), wq/scales/biases stacking E experts:
    // bucketed (perm != null): blockIdx.y is a row tile of one expert;
    // direct (perm == null): blockIdx.y is index row r, expert rhs[r]
    const uint32_t* perm;     // [R] index rows in expert order
    const uint32_t* offsets;  // [E+1] index-row offset of each expert
    const uint32_t* tiles;    // [E+1] row-tile prefix of each expert
    const uint32_t* rhs;      // [R] expert of each index row (direct form)
    const uint32_t* lhs;      // [R] x batch entry of each index row, or null (identity)
    int E, Mx, R, xrows;      // experts; x rows per index row; index rows; rows of x
    OutBias ob;               // dense-layer bias (plain form)
};

// LDS layout: (M+1) rows of K/8 16-byte chunks (row M is zero), each row
// padded by 16 bytes, then the cross-wave reduction buffer.
__host__ __device__ constexpr int xrow_bytes(int K) { return K * 2 + 16; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wait for this wave's LDS operations only (vector-memory loads may stay in
// flight), then a workgroup barrier without the memory fence __syncthreads
// implies: the weight loads issued before it keep streaming.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ u32x4 interleave16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1) {
    // (a0.lo, b0.lo), (a0.hi, b0.hi), (a1.lo, b1.lo), (a1.hi, b1.hi)
    return u32x4{__builtin_amdgcn_perm(b0, a0, 0x05040100u), __builtin_amdgcn_perm(b0, a0, 0x07060302u),
                 __builtin_amdgcn_perm(b1, a1, 0x05040100u), __builtin_amdgcn_perm(b1, a1, 0x07060302u)};
}

// Write one block of x (natural order, in registers) to LDS in fragment
// order (the k order chunk_k() defines). Blocks: 8 elements (4-bit), 32
// (8-bit: chunk j = pieces j and 4+j of 4 elements), 64 (2-bit).
template <int MODE, int BITS>
__device__ __forceinline__ void store_fragment_block(u32x4* dst, const u32x4* v) {
    constexpr bool AFF = MODE == AFFINE;
    if constexpr (BITS == 4 && !AFF) {
        dst[0] = v[0];  // fp4 pairs decode in natural order
    } else if constexpr (BITS == 4) {
        // (x0,x2), (x4,x6), (x1,x3), (x5,x7)
        const u32x4 c = v[0];
        dst[0] = u32x4{__builtin_amdgcn_perm(c[1], c[0], 0x05040100u),
                       __builtin_amdgcn_perm(c[3], c[2], 0x05040100u),
                       __builtin_amdgcn_perm(c[1], c[0], 0x07060302u),
                       __builtin_amdgcn_perm(c[3], c[2], 0x07060302u)};
    } else if constexpr (BITS == 8) {
        const u32x4 c0 = v[0], c1 = v[1], c2 = v[2], c3 = v[3];
        dst[0] = u32x4{c0[0], c0[1], c2[0], c2[1]};
        dst[1] = u32x4{c0[2], c0[3], c2[2], c2[3]};
        dst[2] = u32x4{c1[0], c1[1], c3[0], c3[1]};
        dst[3] = u32x4{c1[2], c1[3], c3[2], c3[3]};
    } else {
        // 16-element word segment jj = natural chunks (2jj, 2jj+1); fragment
        // chunk 4h + jj = natural chunk 2jj + h as (x0,x4),(x1,x5),(x2,x6),(x3,x7)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 c = v[2 * jj + h];
                dst[4 * h + jj] = interleave16(c[0], c[1], c[2], c[3]);
            }
    }
}

// Workgroup: KS waves, wave w owning K-slice [w*UPW*U, (w+1)*UPW*U) of one
// 16-column block. A wave first issues its slice of x and its scale data
// (ordinary loads, before any weight), then the first PF weight units; it
// writes its x slice into its own columns of the LDS x rows (already in
// fragment order) and streams the remaining units through a PF-deep ring,
// waiting only for the oldest unit. Waves meet once, for the final
// cross-wave sum.
// DX (microscaled codes only, whose fragment order is the natural k order
// in 16-byte or 8-byte pieces): instead of staging x in LDS, every lane loads
// its A fragments from global memory together with the weight unit they
// multiply; x of any size then fits one launch (the LDS keeps only the
// cross-wave sums).
// GATHER (staged path only): blockIdx.y is a row tile of one expert
// (bucketed rows, tile height a.M); the workgroup's weight, scales and biases
// are that expert's, its x rows come through the row permutation and lhs,
// and its y rows go back to the index rows' places. The index loads are
// issued first, the weight stream next, and the x loads (which need them)
// last, so the weight stream never waits on the index chain.
// CB = 2 (direct x fragments, microscaled codes): a wave covers two column
// blocks with the same x fragments, halving the x the workgroups re-read
// from L2 (at M = 16 those reads, not the weight stream, set the time);
// at most 8 waves per workgroup then, for the registers.
template <int MODE, int BITS, int G, int UPW, int PF, int MREG, bool DX, bool XS, bool GATHER, int CB,
          bool NS = false>
__global__ void __launch_bounds__(CB == 1 ? 1024 : 512) qmm_decode_kernel(DecodeArgs a) {
    using F = Fmt<MODE, BITS, G>;
    // NS (nvfp4, at most 8 rows): a K-step spans two 16-element groups, so
    // the MFMA rows are split into two slots as for 2-bit g32 codes: codes
    // go into the MFMA at unit scale (one convert per pair) and each step's
    // two group sums take their E4M3 scales on the fp32 accumulator.
    static_assert(!NS || (MODE == NVFP4 && !DX && !GATHER), "nvfp4 row slots: staged x, plain form");
    constexpr int SL = NS ? 2 : F::S;   // row slots
    static_assert(CB == 1 || CB == 2 || CB == 4, "one, two or four column blocks per wave");
    static_assert(!DX || MODE != AFFINE, "direct x fragments need natural-order codes");
    static_assert(!XS || (F::AFF && F::S == 1 && !DX), "x group sums: affine codes, one row slot");
    static_assert(!GATHER || !DX, "the gather form stages x in LDS");
    constexpr int KW = UPW * F::U;                 // k per wave
    extern __shared__ __align__(16) unsigned char smem[];
    const int KS = (int)(blockDim.x >> 6);
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index as a scalar: the weight loads take per-wave offsets in the
    // scalar offset operand, which must be provably wave-uniform
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, j = lane >> 4;
    const int K = a.K;
    // rows of this workgroup's problem; gather: its tile of one expert
    int M = a.M, m0 = 0, row_begin = 0;
    const uint32_t* wqp = a.wq;
    const unsigned char* scp = (const unsigned char*)a.scales;
    const uint16_t* bip = a.biases;
    if (GATHER && !a.perm) {
        // direct form: one index row per tile
        row_begin = blockIdx.y;
        const uint32_t ex = a.rhs[row_begin];
        if (ex >= (uint32_t)a.E) return;             // out-of-range expert: row left unwritten
        const int lo = (int)ex;
        M = a.Mx;
        const size_t erows = (size_t)lo * (size_t)a.N;   // stacked weight rows before expert lo
        wqp += erows * (size_t)(K / F::PER);
        scp += erows * (size_t)(K / G) * (F::AFF ? 2 : 1);
        if constexpr (F::AFF) bip += erows * (size_t)(K / G);
    } else if constexpr (GATHER) {
        // the expert: tiles[] is non-decreasing from tiles[0] = 0, so the
        // number of entries <= tile, less one, is the lo with tiles[lo] <=
        // tile < tiles[lo + 1] (one load per lane per 64 entries and a
        // ballot count instead of a chain of dependent loads)
        const uint32_t tile = blockIdx.y;
        int cnt = 0;
        for (int b0 = 0; b0 <= a.E; b0 += 64) {
            const int e = b0 + lane;
            const uint32_t t = a.tiles[e <= a.E ? e : a.E];
            cnt += __popcll(__ballot(e <= a.E && t <= tile));
        }
        if (cnt > a.E) return;                       // past the real tile count
        const int lo = cnt - 1;
        m0 = ((int)tile - (int)a.tiles[lo]) * a.M;
        row_begin = (int)a.offsets[lo];
        const int rows = ((int)a.offsets[lo + 1] - row_begin) * a.Mx;
        M = min(a.M, rows - m0);
        const size_t erows = (size_t)lo * (size_t)a.N;   // stacked weight rows before expert lo
        wqp += erows * (size_t)(K / F::PER);
        scp += erows * (size_t)(K / G) * (F::AFF ? 2 : 1);
        if constexpr (F::AFF) bip += erows * (size_t)(K / G);
    }
    const int rowb = xrow_bytes(K);
    float* red = (float*)(smem + (DX ? 0 : (M + 1) * rowb));  // [KS][16 rows][16 cols]

    const int k0 = wv * KW;                       // first k of this wave
    const int u_begin = wv * UPW;
    const int n0 = blockIdx.x * a.cols * CB;
    const int wpr = K / F::PER;                   // words per weight row
    const int gpr = K / G;                        // groups per weight row
    // Lane row i carries output column n0 + i. Columns past this workgroup's
    // share (or past N) read zeros through the buffer range check: no memory
    // traffic, never stored.
    bool colv[CB];
    uint32_t ncol[CB], woff[CB];
#pragma unroll
    for (int b = 0; b < CB; ++b) {
        ncol[b] = (uint32_t)(n0 + b * a.cols + i);
        colv[b] = i < a.cols && (int)ncol[b] < a.N;
    }
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(wqp), (short)0, (int)((uint32_t)a.N * (uint32_t)wpr * 4u), 0x00020000);
#pragma unroll
    for (int b = 0; b < CB; ++b)
        woff[b] = colv[b] ? (ncol[b] * (uint32_t)wpr + 4u * j) * 4u : 0x80000000u;
    auto wload = [&](int b, int unit_region) -> u32x4 {   // 16 bytes of region (u * RPU + r)
        return __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)woff[b], unit_region * 64, 0);
    };

    // ---- 1. this wave's x slice (staged path): M rows x KW elements, in blocks of BE
    // elements (the unit of the fragment-order permutation), spread over the
    // lanes; 16-byte chunks, at most XPL per lane
    constexpr int BE = F::XBLOCK;                  // elements per permutation block
    constexpr int CPB = BE / 8;                    // chunks per block
    // chunk registers per lane: enough for the most rows this instantiation
    // takes (host guarantees M * KW <= 4096, i.e. at most 8)
    constexpr int MMAX = (MREG == 4 && !XS) ? 16 : MREG;
    constexpr int XNEED = (MMAX * KW + 511) / 512;
    constexpr int XPL = DX ? 0 : ((XNEED < 8 ? XNEED : 8) + CPB - 1) / CPB * CPB;
    const int xchunks = M * (KW / 8);              // host guarantees <= 64 * XPL
    // Buffer loads: chunks past the last row read as zero, so the loads need
    // no branch (a branch around a load makes the compiler drain every load
    // in flight, which would hold back the weight stream).
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x), (short)0,
        (int)((uint32_t)(GATHER ? a.xrows : M) * (uint32_t)K * 2u), 0x00020000);
    u32x4 xr[XPL > 0 ? XPL : 1];
    // chunk c of this lane: row m of the slice (possibly >= M: zeros), chunk q
    auto chunk_mq = [&](int c, int& m, int& q) {
        // chunk id: lane-major within blocks so one lane owns whole blocks
        const int blk = (c / CPB) * 64 + lane, part = c % CPB;
        const int cid = blk * CPB + part;
        m = cid / (KW / 8);
        q = cid - m * (KW / 8);
    };
    if constexpr (!GATHER) {
#pragma unroll
        for (int c = 0; c < XPL; ++c) {
            int m, q;
            chunk_mq(c, m, q);
            xr[c] = __builtin_amdgcn_raw_buffer_load_b128(
                xrs, (int)(((uint32_t)m * (uint32_t)K + (uint32_t)(k0 + q * 8)) * 2u), 0, 0);
        }
    }
    // gather: the index row of each chunk's GEMM row (rows past the tile
    // read the tile's last row; their x loads are skipped below)
    uint32_t xir[GATHER ? (XPL > 0 ? XPL : 1) : 1];
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(GATHER ? a.perm : nullptr), (short)0,
        (GATHER && a.perm) ? a.R * 4 : 0, 0x00020000);
    if constexpr (GATHER) {
        const uint32_t direct = a.perm ? 0u : 1u;
#pragma unroll
        for (int c = 0; c < XPL; ++c) {
            int m, q;
            chunk_mq(c, m, q);
            const int rho = m0 + (m < M ? m : M - 1);
            const uint32_t pos = (uint32_t)(row_begin + rho / a.Mx);
            const uint32_t ir = __builtin_amdgcn_raw_buffer_load_b32(prs, (int)(pos * 4u), 0, 0);
            xir[c] = direct ? pos : ir;
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // x (gather: its index rows) first

    // ---- 2. scale data of the slice (contiguous in the row); after x, so
    // that staging x waits only for x (loads complete in order)
    constexpr int SB = F::AFF ? UPW * F::GPU * 2 : UPW * F::GPU;  // bytes per slice
    constexpr int SW = (SB + 3) / 4;
    uint32_t sraw[CB][SW], zraw[CB][F::AFF ? SW : 1];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
        constexpr uint32_t SBYTES = F::AFF ? 2u : 1u;
        const uint32_t sbytes_all = (uint32_t)a.N * (uint32_t)gpr * SBYTES;
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<unsigned char*>(scp), (short)0, (int)sbytes_all, 0x00020000);
        const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(F::AFF ? bip : (const uint16_t*)scp), (short)0,
            (int)(F::AFF ? sbytes_all : 0u), 0x00020000);
        const uint32_t soff = colv[cb] ? (ncol[cb] * (uint32_t)gpr + (uint32_t)(u_begin * F::GPU)) * SBYTES
                                       : 0x80000000u;
        if constexpr (SB >= 16) {
#pragma unroll
            for (int v = 0; v < SB / 16; ++v) {
                const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(srs, (int)soff, 16 * v, 0);
                sraw[cb][4 * v] = t[0]; sraw[cb][4 * v + 1] = t[1];
                sraw[cb][4 * v + 2] = t[2]; sraw[cb][4 * v + 3] = t[3];
                if constexpr (F::AFF) {
                    const u32x4 tz = __builtin_amdgcn_raw_buffer_load_b128(zrs, (int)soff, 16 * v, 0);
                    zraw[cb][4 * v] = tz[0]; zraw[cb][4 * v + 1] = tz[1];
                    zraw[cb][4 * v + 2] = tz[2]; zraw[cb][4 * v + 3] = tz[3];
                }
            }
        } else if constexpr (SB == 8) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(srs, (int)soff, 0, 0);
            sraw[cb][0] = t[0]; sraw[cb][1] = t[1];
            if constexpr (F::AFF) {
                const u32x2 tz = __builtin_amdgcn_raw_buffer_load_b64(zrs, (int)soff, 0, 0);
                zraw[cb][0] = tz[0]; zraw[cb][1] = tz[1];
            }
        } else if constexpr (SB == 4) {
            sraw[cb][0] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)soff, 0, 0);
            if constexpr (F::AFF) zraw[cb][0] = __builtin_amdgcn_raw_buffer_load_b32(zrs, (int)soff, 0, 0);
        } else {
            sraw[cb][0] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)soff, 0, 0);
            if constexpr (F::AFF) zraw[cb][0] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)soff, 0, 0);
        }
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- this lane's A row (zero row when it carries no real x row)
    int arow;
    if constexpr (SL == 2) arow = (i / 8 == j / 2 && (i & 7) < M) ? (i & 7) : M;
    else arow = (i < M) ? i : M;

    // DX: A fragments of unit u from global memory. Fragment of global step
    // gs: k in [32 gs + 8 j, +8) for 4-bit codes; [32 gs + 4 j, +4) and
    // [32 gs + 16 + 4 j, +4) for 8-bit codes. Rows >= M read zeros.
    constexpr int XF = DX ? F::STEPS : 1;
    const uint32_t xfoff = arow < M ? ((uint32_t)arow * (uint32_t)K + (BITS == 4 ? 8u : 4u) * j) * 2u
                                    : 0x80000000u;
    u32x4 xfr[DX ? PF : 1][XF];
    auto load_xf = [&](u32x4 (&dst)[XF], int u) {
        if constexpr (DX) {
#pragma unroll
            for (int ls = 0; ls < F::STEPS; ++ls) {
                const int so = (u * F::STEPS + ls) * 64;  // bytes: 32 elements per step
                if constexpr (BITS == 4) {
                    dst[ls] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)xfoff, so, 0);
                } else {
                    const auto p0 = __builtin_amdgcn_raw_buffer_load_b64(xrs, (int)xfoff, so, 0);
                    const auto p1 = __builtin_amdgcn_raw_buffer_load_b64(xrs, (int)xfoff, so + 32, 0);
                    dst[ls] = u32x4{p0[0], p0[1], p1[0], p1[1]};
                }
            }
        }
    };

    // ---- 3. the first PF weight units (and their x fragments)
    u32x4 wbuf[PF][CB][F::RPU];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < UPW) {
#pragma unroll
            for (int b = 0; b < CB; ++b)
#pragma unroll
                for (int r = 0; r < F::RPU; ++r)
                    wbuf[p][b][r] = wload(b, (u_begin + p) * F::RPU + r);
            if constexpr (DX) load_xf(xfr[p], u_begin + p);
        }

    // ---- gather: x rows through lhs, issued after the weight stream (the
    // staging below then also waits for the weight units, which were issued
    // first)
    if constexpr (GATHER) {
        const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t*>(a.lhs), (short)0, a.lhs ? a.R * 4 : 0, 0x00020000);
        const uint32_t has_lhs = a.lhs ? 1u : 0u;
#pragma unroll
        for (int c = 0; c < XPL; ++c) {
            const uint32_t lb = __builtin_amdgcn_raw_buffer_load_b32(lrs, (int)(xir[c] * 4u), 0, 0);
            xir[c] = has_lhs ? lb : xir[c];       // x batch entry of the index row
        }
#pragma unroll
        for (int c = 0; c < XPL; ++c) {
            int m, q;
            chunk_mq(c, m, q);
            const int rho = m0 + m;
            const uint32_t xrow = xir[c] * (uint32_t)a.Mx + (uint32_t)(rho % a.Mx);
            const uint32_t off = m < M ? (xrow * (uint32_t)K + (uint32_t)(k0 + q * 8)) * 2u : 0x80000000u;
            xr[c] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, 0, 0);
        }
    }

    // ---- 4. x slice -> LDS (fragment order) + this slice of the zero row
#pragma unroll
    for (int c = 0; c < XPL; c += CPB) {
        const int blk = (c / CPB) * 64 + lane;
        const int cid = blk * CPB;
        if (cid < xchunks) {
            const int m = cid / (KW / 8), q = cid - m * (KW / 8);
            u32x4* dst = (u32x4*)(smem + m * rowb + (k0 / 8 + q) * 16);
            store_fragment_block<MODE, BITS>(dst, &xr[c]);
        }
    }
    if constexpr (!DX)
        for (int q = lane; q < KW / 8; q += 64)
            *(u32x4*)(smem + M * rowb + (k0 / 8 + q) * 16) = u32x4{0u, 0u, 0u, 0u};

    // XS (at most 4 rows): sum x over every quantization group of the slice
    // once, from the chunks this lane loaded (a permutation block of BE
    // elements per lane, G / BE consecutive lanes per group), instead of a
    // second MFMA against an all-ones operand per K-step. Every lane of a
    // group ends with the group's sum; the epilogue reads it with readlane
    // (rows < 4 are the only rows a lane row j = 0 holds, and rows of other
    // lane rows are past M and never stored).
    constexpr int NB = XS ? XPL / CPB : 1;
    float bsum[NB];
    if constexpr (XS) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float t = 0.f;
#pragma unroll
            for (int part = 0; part < CPB; ++part) {
                const u32x4 c = xr[b * CPB + part];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    t += bf16_bits_to_f32(c[e] & 0xFFFFu) + bf16_bits_to_f32(c[e] >> 16);
            }
            constexpr int LG = G / BE;  // lanes per group
            if constexpr (LG >= 2) t += lane_xchg<0xB1>(t);   // quad_perm [1,0,3,2]
            if constexpr (LG >= 4) t += lane_xchg<0x4E>(t);   // quad_perm [2,3,0,1]
            if constexpr (LG >= 8) t += lane_xchg<0x141>(t);  // row_half_mirror
            if constexpr (LG >= 16) t += lane_xchg<0x140>(t); // row_mirror
            bsum[b] = t;
        }
    }
    // sum of x row m over local group gl of this wave's slice (XS only)
    auto xgroup_sum = [&](int m, int gl) -> float {
        const int cid0 = m * (KW / 8) + gl * (G / 8);
        const int blk0 = cid0 / CPB;
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, bsum[(blk0 / 64) < NB ? blk0 / 64 : 0]), blk0 % 64));
    };
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes done (loads stay in flight)
    __builtin_amdgcn_wave_barrier();

    const unsigned char* abase = smem + arow * rowb + j * 16;

    f32x4 acc[CB], dsum = {0.f, 0.f, 0.f, 0.f};
    float ysum[CB][MREG];
#pragma unroll
    for (int b = 0; b < CB; ++b) {
        acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < MREG; ++r) ysum[b][r] = 0.f;
    }
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const int u = u_begin + uu;
        u32x4 wcur[CB][F::RPU];
#pragma unroll
        for (int b = 0; b < CB; ++b)
#pragma unroll
            for (int r = 0; r < F::RPU; ++r) {
                wcur[b][r] = wbuf[uu % PF][b][r];
                xpose4(wcur[b][r]);
            }
        u32x4 xcur[XF];
        if constexpr (DX) {
#pragma unroll
            for (int ls = 0; ls < XF; ++ls) xcur[ls] = xfr[uu % PF][ls];
        }
        // refill the ring slot with unit uu + PF
        if (uu + PF < UPW) {
#pragma unroll
            for (int b = 0; b < CB; ++b)
#pragma unroll
                for (int r = 0; r < F::RPU; ++r)
                    wbuf[uu % PF][b][r] = wload(b, (u + PF) * F::RPU + r);
            if constexpr (DX) load_xf(xfr[uu % PF], u + PF);
        }
#pragma unroll
        for (int r = 0; r < F::RPU; ++r) {
#pragma unroll
            for (int t = 0; t < F::SPR; ++t) {
                const int ls = r * F::SPR + t;                 // step within unit
                const int gs = (u * F::RPU + r) * F::SPR + t;  // global step
                u32x4 av;
                if constexpr (DX) av = xcur[ls];
                else av = *(const u32x4*)(abase + gs * 64);
                const bool first = (F::AFF && (ls % F::WS == 0)) || NS;
                if constexpr (F::AFF && !XS) dsum = mfma_bf16(av, ones, first ? zero4 : dsum);
#pragma unroll
                for (int b = 0; b < CB; ++b) {
                    float sc = 0.f;
                    if constexpr (!F::AFF) {
                        int byte;
                        if constexpr (MODE == NVFP4) byte = uu * F::GPU + 2 * ls + (j >> 1);
                        else byte = uu * F::GPU + ls;
                        const int wd = (MODE == NVFP4) ? (uu * F::GPU + 2 * ls) / 4 : byte / 4;
                        sc = scale_byte_to_f32<MODE>((sraw[b][wd] >> (8 * (byte & 3))) & 0xFFu);
                    }
                    u32x4 bv;
                    if constexpr (NS) bv = unpack<MXFP4, 4, 32>(wcur[b][r], t, 1.0f);   // E2M1 at unit scale
                    else bv = unpack<MODE, BITS, G>(wcur[b][r], t, sc);
                    acc[b] = mfma_bf16(av, bv, first ? zero4 : acc[b]);
                    if constexpr (NS) {
#pragma unroll
                        for (int rr = 0; rr < MREG; ++rr) ysum[b][rr] = __builtin_fmaf(sc, acc[b][rr], ysum[b][rr]);
                    }
                }
                if constexpr (F::AFF) {
                    if (ls % F::WS == F::WS - 1) {
                        // window done: apply the group's scale and bias
                        const int wi = ls / F::WS;
                        const int gw = uu * F::GPU + (F::S == 2 ? 2 * wi : wi);
                        const int sh = (F::S == 2) ? 16 * (j >> 1) : 16 * (gw & 1);
#pragma unroll
                        for (int b = 0; b < CB; ++b) {
                            const float s = bf16_bits_to_f32((sraw[b][gw >> 1] >> sh) & 0xFFFFu);
                            const float z = bf16_bits_to_f32((zraw[b][gw >> 1] >> sh) & 0xFFFFu);
                            const float zz = __builtin_fmaf(-F::OFF, s, z);
#pragma unroll
                            for (int rr = 0; rr < MREG; ++rr) {
                                float xs;
                                if constexpr (XS) xs = xgroup_sum(rr, gw);
                                else xs = dsum[rr];
                                ysum[b][rr] = __builtin_fmaf(s, acc[b][rr], ysum[b][rr]);
                                ysum[b][rr] = __builtin_fmaf(zz, xs, ysum[b][rr]);
                            }
                        }
                    }
                }
            }
        }
    }
    if constexpr (!F::AFF && !NS) {
#pragma unroll
        for (int b = 0; b < CB; ++b)
#pragma unroll
            for (int rr = 0; rr < MREG; ++rr) ysum[b][rr] = acc[b][rr];
    }

    // ---- cross-wave reduction: red[wave][block][row][col]
#pragma unroll
    for (int b = 0; b < CB; ++b)
#pragma unroll
        for (int rr = 0; rr < MREG; ++rr) red[((wv * CB + b) * 16 + 4 * j + rr) * 16 + i] = ysum[b][rr];
    __syncthreads();
    for (int o = tid; o < CB * M * 16; o += 64 * KS) {
        const int b = CB == 1 ? 0 : o / (M * 16), mo = o - b * (M * 16);
        const int m = mo >> 4, col = mo & 15;
        const int n = n0 + b * a.cols + col;
        if (n >= a.N || col >= a.cols) continue;
        float v = 0.f;
        for (int w = 0; w < KS; ++w) {
            if constexpr (SL == 2) {
                v += red[((w * CB + b) * 16 + m) * 16 + col];
                v += red[((w * CB + b) * 16 + 8 + m) * 16 + col];
            } else {
                v += red[((w * CB + b) * 16 + m) * 16 + col];
            }
        }
        size_t yrow = (size_t)m;
        if constexpr (GATHER) {
            const int rho = m0 + m;
            const int pos = row_begin + rho / a.Mx;
            yrow = (size_t)(a.perm ? a.perm[pos] : (uint32_t)pos) * a.Mx + (size_t)(rho % a.Mx);
        }
        a.y[yrow * a.N + n] = (uint16_t)f32_to_bf16_rne(add_out_bias(a.ob, n, v));
    }
}

// Decomposition: a wave's slice is KW = UPW units (choose_upw below); a
// workgroup has KS = nunits / UPW <= 16 waves. Shorter slices (more waves per
// workgroup) measured faster: UPW 4 beats 8 by about 5 % at M = 1.
constexpr int kDecodeUpwMax = 4;   // units per wave (power of two, <= 16)
constexpr int kDecodePf = 4;       // weight units in flight per wave

// Output columns per workgroup: all workgroups of a launch are resident at
// once, so a CU's share is ceil(workgroups / CUs) of them; take the widest
// block (at most the 16 MFMA columns) that minimises the columns per CU.
// N = 14336 on 256 CUs: 14 columns, 1024 workgroups, 4 per CU (16 columns
// would give half the CUs 4 workgroups and half 3).
int decode_columns(int N, int cus) {
    int best = 16;
    int64_t best_load = 0;
    for (int c = 16; c >= 8; --c) {
        const int64_t wgs = (N + c - 1) / c;
        const int64_t load = (wgs + cus - 1) / cus * c;
        if (c == 16 || load < best_load) {
            best = c;
            best_load = load;
        }
    }
    return best;
}

// Units per wave: start from kDecodeUpwMax (half that for two-region
// units), grow while the workgroup would need more than 16 waves, then
// shrink until it divides the unit count and (staged path) the wave's x
// slice fits 8 chunk registers per lane. 0: no valid decomposition.
int choose_upw(int nunits, int64_t M, int U, int RPU, bool dx) {
    const int64_t xlim = dx ? (1LL << 40) : 4096;
    int upw = RPU >= 2 ? kDecodeUpwMax / 2 : kDecodeUpwMax;
    if (upw < 1) upw = 1;
    while (upw < 16 && nunits / upw > 16) upw <<= 1;
    while (upw > 1 && (nunits % upw || M * upw * U > xlim)) upw >>= 1;
    if (nunits % upw || M * upw * U > xlim || nunits / upw > 16) return 0;
    return upw;
}

template <int MODE, int BITS, int G>
int pick_upw(int nunits, int M, bool dx) {
    using F = Fmt<MODE, BITS, G>;
    return choose_upw(nunits, M, F::U, F::RPU, dx);
}

// gather_tiles > 0: the gather form, blockIdx.y over that many row tiles
// (an upper bound; tiles past the real count leave at once).
template <int MODE, int BITS, int G, int UPW, bool DX, int CB = 1, bool NS = false>
hipError_t launch_upw(const DecodeArgs& a, int ks, int mreg, int gather_tiles, hipStream_t st) {
    constexpr int PF = UPW < kDecodePf ? UPW : kDecodePf;
    if (CB >= 2 && ks > 8) return hipErrorNotSupported;   // 512-thread kernels
    const unsigned blocks = (unsigned)((a.N + a.cols * CB - 1) / (a.cols * CB));
    const dim3 grid(blocks, gather_tiles > 0 ? (unsigned)gather_tiles : 1u);
    const unsigned threads = 64u * (unsigned)ks;
    const size_t shm = (DX ? 0 : (size_t)(a.M + 1) * xrow_bytes(a.K)) + (size_t)ks * CB * 16 * 16 * 4;
    auto run = [&](auto kern) -> hipError_t {
        if (shm > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void*)kern,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            if (e != hipSuccess) return e;
        }
        kern<<<grid, threads, shm, st>>>(a);
        return hipGetLastError();
    };
    // group sums of x instead of the all-ones MFMA: affine, one row slot, M <= 4
    constexpr bool XSOK = Fmt<MODE, BITS, G>::AFF && Fmt<MODE, BITS, G>::S == 1 && !DX;
    if constexpr (NS) {   // nvfp4 row slots: staged x, plain form, at most 8 rows
        if (gather_tiles > 0 || a.M > 8) return hipErrorNotSupported;
        if constexpr (DX) {
            return hipErrorNotSupported;
        } else if constexpr (CB == 4) {
            return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, false, 4, true>);
        } else if constexpr (CB == 2) {
            if (mreg <= 2) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 2, false, false, false, 2, true>);
            return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, false, 2, true>);
        } else {
            if (mreg <= 1) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 1, false, false, false, 1, true>);
            if (mreg == 2) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 2, false, false, false, 1, true>);
            return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, false, 1, true>);
        }
    } else if constexpr (CB == 4) {
        // staged x, 5..8 rows, plain form only
        return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, false, 4>);
    } else if constexpr (CB == 2) {
        if constexpr (DX) {
            // direct x, microscaled: rows past 4 in registers (MREG 4)
            return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, true, false, false, 2>);
        } else {
            if (gather_tiles > 0) {   // gather form: both blocks of one row tile
                if (XSOK && a.M <= 4)
                    return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, XSOK, true, 2>);
                return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, true, 2>);
            }
            // staged x shared by the wave's two column blocks (M >= 2)
            if (mreg <= 2) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 2, false, XSOK, false, 2>);
            if (XSOK && a.M <= 4) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, XSOK, false, 2>);
            return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, false, 2>);
        }
    } else {
        if constexpr (!DX) {
            if (gather_tiles > 0) {   // a tile holds 1 .. a.M rows
                if (XSOK && a.M <= 4)
                    return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, XSOK, true, 1>);
                return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, false, false, true, 1>);
            }
        }
        if (mreg <= 1) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 1, DX, XSOK, false, 1>);
        if (mreg == 2) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 2, DX, XSOK, false, 1>);
        if (XSOK && a.M <= 4) return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, DX, XSOK, false, 1>);
        return run(qmm_decode_kernel<MODE, BITS, G, UPW, PF, 4, DX, false, false, 1>);
    }
}

// Plain form (perm == null) or gather form: rows bucketed by expert into
// tiles of tile_rows GEMM rows (launch_bucket with the same tile height).
template <int MODE, int BITS, int G, bool DX, bool NS = false>
hipError_t launch_fmt(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets, int tile_rows,
                      hipStream_t st) {
    using F = Fmt<MODE, BITS, G>;
    DecodeArgs a{};
    a.x = (const uint16_t*)q.x;
    a.wq = q.wq;
    a.scales = q.scales;
    a.biases = (const uint16_t*)q.biases;
    a.y = (uint16_t*)q.y;
    a.ob = q.ob;
    a.M = (int)q.M;
    a.N = (int)q.N;
    a.K = (int)q.K;
    const int cus = device_shape().cus;
    a.cols = decode_columns(a.N, cus);
    int gather_tiles = 0;
    if (tile_rows < 0) {
        // direct gather form: one tile per index row, its rows = x rows per index row
        a.Mx = (int)q.M;
        a.M = (int)q.M;
        a.rhs = q.rhs;
        a.lhs = q.lhs;
        a.E = (int)q.E;
        a.R = (int)q.R;
        a.xrows = (int)(q.batch_x * q.M);
        gather_tiles = (int)q.R;
    } else if (perm) {
        // GEMM rows = index rows x rows per index row; a tile is tile_rows of
        // one expert, so the tile count is at most rows / tile_rows plus one
        // per expert that has rows
        const int64_t rows = q.R * q.M;
        a.Mx = (int)q.M;
        a.M = tile_rows;
        a.perm = perm;
        a.offsets = offsets;
        a.tiles = offsets + (q.E + 1);
        a.lhs = q.lhs;
        a.E = (int)q.E;
        a.R = (int)q.R;
        a.xrows = (int)(q.batch_x * q.M);
        gather_tiles = (int)(rows / tile_rows + (q.E < q.R ? q.E : q.R));
    }
    // the gather grid spans many row tiles (several rounds of workgroups):
    // full 16-column blocks halve the workgroups and their fixed costs
    if (gather_tiles > 0) a.cols = 16;
    const int mreg = a.M > 4 ? 4 : a.M;
    const int nunits = a.K / F::U;
    const int upw = pick_upw<MODE, BITS, G>(nunits, a.M, DX);
    if (upw == 0) return hipErrorNotSupported;
    const int ks = nunits / upw;
    // two column blocks per wave (at most 8 waves: longer slices): direct x
    // fragments always; staged x from two rows up,
    // where every workgroup re-reading all of x from L2 rivals the weight
    // stream (M8: 64 KB of x per workgroup against 56 KB of weights), and
    // for 8-bit affine codes at one row too (M1 int8 15.5 -> 13.9 us; 4-bit
    // and microscaled one-row shapes measured slower this way)
    const bool staged_cb2 = a.M >= 2 || (F::AFF && BITS == 8);
    // gather form: two blocks per wave share the tile's expert lookup, index
    // loads and x (2 tokens x top-8 10.1 -> 9.5 us, 8 tokens 27.6 -> 23.7 us,
    // 16 tokens 37.7 -> 31.5 us) while the grid keeps two workgroups per CU
    // (1 token: 8 tiles would leave 384 workgroups, 7.2 -> 7.7 us)
    const bool gather_cb2 = gather_tiles > 0 &&
                            (int64_t)gather_tiles * ((a.N + 2 * a.cols - 1) / (2 * a.cols)) >=
                                2 * (int64_t)cus;
    if (DX || (!DX && gather_tiles == 0 && staged_cb2) ||
        (!DX && gather_cb2)) {
        int upw2 = upw;
        while (upw2 < 16 && nunits / upw2 > 8) upw2 <<= 1;
        // staged x: a wave's slice of every row fits its chunk registers
        const bool fits = DX || (int64_t)a.M * upw2 * F::U <= 4096;
        if (fits && nunits % upw2 == 0 && nunits / upw2 <= 8) {
            DecodeArgs a2 = a;
            const int ks2 = nunits / upw2;
            if constexpr (!DX) {
                // 5..8 staged rows: four column blocks per wave, so each
                // workgroup's read of x from L2 serves four times the columns
                if (gather_tiles <= 0 && a.M > 4 && upw2 == 4) {
                    a2.cols = decode_columns((a.N + 3) / 4, cus);
                    return launch_upw<MODE, BITS, G, 4, false, 4, NS>(a2, ks2, mreg, 0, st);
                }
            }
            if (gather_tiles <= 0) a2.cols = decode_columns((a.N + 1) / 2, cus);
            switch (upw2) {
            case 16: return launch_upw<MODE, BITS, G, 16, DX, 2, NS>(a2, ks2, mreg, gather_tiles, st);
            case 8: return launch_upw<MODE, BITS, G, 8, DX, 2, NS>(a2, ks2, mreg, gather_tiles, st);
            case 4: return launch_upw<MODE, BITS, G, 4, DX, 2, NS>(a2, ks2, mreg, gather_tiles, st);
            case 2: return launch_upw<MODE, BITS, G, 2, DX, 2, NS>(a2, ks2, mreg, gather_tiles, st);
            default: return launch_upw<MODE, BITS, G, 1, DX, 2, NS>(a2, ks2, mreg, gather_tiles, st);
            }
        }
    }
    switch (upw) {
    case 16: return launch_upw<MODE, BITS, G, 16, DX, 1, NS>(a, ks, mreg, gather_tiles, st);
    case 8: return launch_upw<MODE, BITS, G, 8, DX, 1, NS>(a, ks, mreg, gather_tiles, st);
    case 4: return launch_upw<MODE, BITS, G, 4, DX, 1, NS>(a, ks, mreg, gather_tiles, st);
    case 2: return launch_upw<MODE, BITS, G, 2, DX, 1, NS>(a, ks, mreg, gather_tiles, st);
    default: return launch_upw<MODE, BITS, G, 1, DX, 1, NS>(a, ks, mreg, gather_tiles, st);
    }
}

}  // namespace

namespace {

constexpr size_t kDecodeLdsLimit = 150 * 1024;

int decode_upw(const QmmArgs& q, int64_t m, bool dx) {
    const int per = 32 / q.bits;
    const int rk = 16 * per;
    const int u = rk > q.group_size ? rk : q.group_size;
    if (q.K % u != 0) return 0;
    return choose_upw((int)(q.K / u), m, u, u / rk, dx);
}

// Shape rules of the staged decode kernel for m activation rows.
bool decode_shape_ok(const QmmArgs& q, int64_t m) {
    if (q.mode == AFFINE && q.bits == 2 && q.group_size == 32 && m > 8) return false;
    if (decode_upw(q, m, false) == 0) return false;
    const size_t shm = (size_t)(m + 1) * xrow_bytes((int)q.K) + 16 * 16 * 16 * 4;
    return shm <= kDecodeLdsLimit;
}

// Largest number of activation rows one staged launch takes (0: none).
int64_t decode_rows_per_pass(const QmmArgs& q) {
    for (int64_t m = q.M < 16 ? q.M : 16; m >= 1; --m)
        if (decode_shape_ok(q, m)) return m;
    return 0;
}

// Microscaled codes unpack in natural k order, so when x does not fit one
// staged launch the A fragments come straight from global memory instead.
bool decode_direct_x(const QmmArgs& q) {
    return q.mode != AFFINE && decode_rows_per_pass(q) < q.M && decode_upw(q, q.M, true) > 0;
}

template <bool DX>
hipError_t launch_mode(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets, int tile_rows,
                       hipStream_t st) {
    switch (q.mode) {
    case MXFP4: return launch_fmt<MXFP4, 4, 32, DX>(q, perm, offsets, tile_rows, st);
    case NVFP4:
        // staged x, plain form, at most 8 rows: the row-slot kernel
        if constexpr (!DX)
            if (!perm && tile_rows == 0 && q.M <= 8)
                return launch_fmt<NVFP4, 4, 16, false, true>(q, perm, offsets, tile_rows, st);
        return launch_fmt<NVFP4, 4, 16, DX>(q, perm, offsets, tile_rows, st);
    case MXFP8: return launch_fmt<MXFP8, 8, 32, DX>(q, perm, offsets, tile_rows, st);
    default: break;
    }
    if constexpr (DX) {
        return hipErrorNotSupported;
    } else {
        if (q.bits == 4)
            return q.group_size == 32 ? launch_fmt<AFFINE, 4, 32, false>(q, perm, offsets, tile_rows, st)
                 : q.group_size == 64 ? launch_fmt<AFFINE, 4, 64, false>(q, perm, offsets, tile_rows, st)
                                      : launch_fmt<AFFINE, 4, 128, false>(q, perm, offsets, tile_rows, st);
        if (q.bits == 8)
            return q.group_size == 32 ? launch_fmt<AFFINE, 8, 32, false>(q, perm, offsets, tile_rows, st)
                 : q.group_size == 64 ? launch_fmt<AFFINE, 8, 64, false>(q, perm, offsets, tile_rows, st)
                                      : launch_fmt<AFFINE, 8, 128, false>(q, perm, offsets, tile_rows, st);
        return q.group_size == 32 ? launch_fmt<AFFINE, 2, 32, false>(q, perm, offsets, tile_rows, st)
             : q.group_size == 64 ? launch_fmt<AFFINE, 2, 64, false>(q, perm, offsets, tile_rows, st)
                                  : launch_fmt<AFFINE, 2, 128, false>(q, perm, offsets, tile_rows, st);
    }
}

}  // namespace

bool qmm_decode_supports(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16 || q.R != 0) return false;
    if (q.M < 1 || q.M > 16 || q.N < 1 || q.K > (1 << 20)) return false;
    // 32-bit buffer offsets into x, the weight and its scales
    if (q.M * q.K * 2 >= (1LL << 31) || q.N * q.K * q.bits / 8 >= (1LL << 31)) return false;
    if (q.N * (q.K / q.group_size) * 2 >= (1LL << 31)) return false;
    // 16-byte aligned weight rows, x rows and per-wave scale blocks
    if (((uintptr_t)q.wq & 15) != 0 || ((uintptr_t)q.x & 15) != 0) return false;
    if (((uintptr_t)q.scales & 15) != 0 || ((uintptr_t)q.biases & 15) != 0) return false;
    const int64_t gpr = q.K / q.group_size;
    if ((q.mode == AFFINE ? gpr * 2 : gpr) % 16 != 0) return false;
    if (decode_direct_x(q)) return true;
    // x rows that do not fit one launch's LDS run as several launches, each
    // streaming the weight again (at most 4)
    const int64_t rpp = decode_rows_per_pass(q);
    return rpp > 0 && (q.M + rpp - 1) / rpp <= 4;
}

hipError_t launch_qmm_decode(const QmmArgs& q0, hipStream_t st) {
    if (!qmm_decode_supports(q0)) return hipErrorNotSupported;
    if (decode_direct_x(q0)) return launch_mode<true>(q0, nullptr, nullptr, 0, st);
    const int64_t rpp = decode_rows_per_pass(q0);
    for (int64_t m0 = 0; m0 < q0.M; m0 += rpp) {
        QmmArgs q = q0;
        q.M = (q0.M - m0) < rpp ? (q0.M - m0) : rpp;
        q.x = (const uint16_t*)q0.x + m0 * q0.K;
        q.y = (uint16_t*)q0.y + m0 * q0.N;
        hipError_t e = launch_mode<false>(q, nullptr, nullptr, 0, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int qmm_decode_gather_tile_rows(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16 || q.R <= 0 || q.M < 1 || q.E < 1) return 0;
    const int64_t rows = q.R * q.M;
    int rt;
    if (rows * 2 <= q.E && q.M <= 4) rt = -1;   // direct: rows rarely share an expert
    else if (rows <= 2 * q.E) rt = 4;
    else if (rows <= 8 * q.E) rt = (q.mode == AFFINE && q.bits == 2 && q.group_size == 32) ? 8 : 16;
    else return 0;
    if (q.N < 1 || q.K > (1 << 20) || q.K % 8 != 0) return 0;
    // 32-bit buffer offsets into x, one expert's weight and its scales; grid y
    if (q.batch_x * q.M * q.K * 2 >= (1LL << 31) || q.N * q.K * q.bits / 8 >= (1LL << 31)) return 0;
    if (q.N * (q.K / q.group_size) * 2 >= (1LL << 31) || q.R * 4 >= (1LL << 31)) return 0;
    if ((rt > 0 ? rows / rt + q.E : q.R) >= 65536) return 0;
    // 16-byte aligned weight rows of every expert, x rows and per-wave scale blocks
    if (((uintptr_t)q.wq & 15) != 0 || ((uintptr_t)q.x & 15) != 0) return 0;
    if (((uintptr_t)q.scales & 15) != 0 || ((uintptr_t)q.biases & 15) != 0) return 0;
    if ((q.N * q.K * q.bits / 8) % 16 != 0) return 0;
    const int64_t gpr = q.K / q.group_size;
    if ((q.mode == AFFINE ? gpr * 2 : gpr) % 16 != 0) return 0;
    return decode_shape_ok(q, rt > 0 ? rt : q.M) ? rt : 0;
}

hipError_t launch_qmm_decode_gather(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                                    int tile_rows, hipStream_t st) {
    if (tile_rows == 0 || tile_rows != qmm_decode_gather_tile_rows(q)) return hipErrorNotSupported;
    if (tile_rows > 0 && (!perm || !offsets)) return hipErrorInvalidValue;
    return launch_mode<false>(q, tile_rows > 0 ? perm : nullptr, offsets, tile_rows, st);
}

}  // namespace qlin
