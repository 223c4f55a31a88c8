// qmm_prefill.hip -- many-row quantized matmul on bf16 MFMA (gfx950).
//
// y = x . dequant(W)^T, [out, in] weight layout, bf16 activations
// ("EMLX.Quantization", quantized_matmul; "Emily.QuantizedWeight", Layout
// and Microscaled modes). With thousands of activation rows this is a dense
// contraction, so the weight is dequantized once per workgroup tile and fed
// to v_mfma_f32_16x16x32_bf16; the dense weight never reaches HBM.
//
// Workgroup tile: BM activation rows x BN weight rows, K in steps of 64.
//   * Activations go from global memory straight into a three-stage LDS
//     ring (buffer->LDS loads, no registers), two steps ahead of their use.
//   * Packed weight codes for step k+2 are loaded into registers during step
//     k, and dequantized during step k+1 into the other of two LDS buffers,
//     CPC codes (one scale/bias pair) per chunk; one barrier per step.
//   * Loads use buffer resources, so rows past the end of x or W read as
//     zero and need no clamping or branches.
//   * The blockIdx -> tile map keeps one row of tiles on one XCD, so the
//     activation rows it shares stay in that XCD's L2.
// Accumulation is fp32; lane (i, j) of an MFMA tile ends with 4 consecutive
// output columns of one row (8-byte stores).

#include "qlin_common.h"

#include <stdlib.h>

#include <atomic>
#include <type_traits>

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int BK = 64;              // k per step
constexpr int LROW = BK * 2 + 16;   // LDS row pitch in bytes (16 bytes of padding)

struct PrefillArgs {
    const uint16_t* x;     // bf16 [M, K]; gather: [B, M, K]
    const uint32_t* wq;    // [N, K/PER]; gather: [E][N][K/PER]
    const void* scales;    // [N, K/G] bf16 (affine) or u8 (microscaled); gather: per expert
    const uint16_t* biases;
    uint16_t* y;           // bf16 [M, N]; gather: [R, M, N]
    int M, N, K;           // gather: M = activation rows per index row
    // gather form (expert-bucketed rows)
    const uint32_t* lhs;      // [R] or null (identity)
    const uint32_t* perm;     // [R] index rows in expert order
    const uint32_t* offsets;  // [E+1] index-row offset of each expert
    const uint32_t* tiles;    // [E+1] row-tile prefix of each expert
    int E, B;
    int xcds;                 // XCDs of the device
    int lds_nan;              // debug: fill LDS with NaN before the tile
    int xgm;                  // plain form: the XCDs as an xgm x (xcds/xgm) grid of tile blocks (0: rows)
    OutBias ob;               // dense-layer bias (plain form)
};

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};  // nearest-even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    // raw buffer (stride 0): loads at offsets >= bytes return zero. Rows past
    // the end already have their per-lane offset past the end, so the check
    // holds whether or not the scalar offset takes part in it.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// s_waitcnt immediate for vmcnt(vm) lgkmcnt(0). Fields: vmcnt [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8].
constexpr int vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | ((vm >> 4) << 14); }

// f(integral_constant<int, U>) for U = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void unroll(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        unroll<B + 1, E>(f);
    }
}

// Packed codes of one chunk: WORDS = CPC * BITS / 32 dwords.
template <int WORDS>
struct Chunk {
    uint32_t w[WORDS];
};

// voff: per-lane byte offset (loop invariant); soff: wave-uniform byte
// offset of the step. A lane whose voff is past the end reads zeros.
template <int WORDS>
__device__ __forceinline__ Chunk<WORDS> load_chunk(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   int soff) {
    Chunk<WORDS> c;
    if constexpr (WORDS == 8) {
        const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
        const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff + 16, soff, 0);
        c.w[0] = v0.x; c.w[1] = v0.y; c.w[2] = v0.z; c.w[3] = v0.w;
        c.w[4] = v1.x; c.w[5] = v1.y; c.w[6] = v1.z; c.w[7] = v1.w;
    } else if constexpr (WORDS == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
        c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
    } else if constexpr (WORDS == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, soff, 0);
        c.w[0] = v.x; c.w[1] = v.y;
    } else {
        c.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0);
    }
    return c;
}

// NB bytes (1, 2, 4, 8 or 16) at voff + soff, in BD = max(1, NB/4) dwords.
template <int NB, int BD = (NB < 4 ? 1 : NB / 4)>
__device__ __forceinline__ void load_bytes(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff,
                                           uint32_t (&d)[BD]) {
    if constexpr (NB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else if constexpr (NB == 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, soff, 0);
        d[0] = v.x; d[1] = v.y;
    } else if constexpr (NB == 4) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, soff, 0);
    } else if constexpr (NB == 2) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, soff, 0);
    } else {
        static_assert(NB == 1, "1, 2, 4, 8 or 16 bytes");
        d[0] = __builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, soff, 0);
    }
}

// Dequantization of one chunk in small pieces, so that the pieces can sit
// between single MFMAs: prepare (scale, bias and, for packed integer codes,
// the codes split into bytes), then one packed bf16 pair per piece.
// Affine: bf16(fmaf(s, q, z)), the dequantized value rounded once to the
// MFMA input type. Microscaled: exact decode times the group scale.
template <int MODE, int BITS>
struct DqPre {
    static constexpr int N = MODE == AFFINE && BITS == 4 ? 2 : (MODE == AFFINE && BITS == 2 ? 4 : 1);
};
template <int MODE, int BITS, int NWO>
struct DqState {
    float s, z;
    uint32_t pre[DqPre<MODE, BITS>::N];
    uint32_t o[NWO];
};

// The codes of a chunk (WORDS dwords) split into bytes: 4-bit codes as the
// low and high nibbles of each byte, 2-bit codes as four planes. The empty
// asm keeps the masked words opaque, so each code is one byte convert
// instead of a bit-field extract and a convert.
template <int MODE, int BITS, int WORDS, int NWO>
__device__ __forceinline__ void dq_prepare(DqState<MODE, BITS, NWO>& st, const uint32_t* w) {
    if constexpr (MODE == AFFINE && BITS == 4) {
        uint32_t lo = w[0] & 0x0F0F0F0Fu, hi = (w[0] >> 4) & 0x0F0F0F0Fu;
        asm("" : "+v"(lo));
        asm("" : "+v"(hi));
        st.pre[0] = lo;
        st.pre[1] = hi;
    } else if constexpr (MODE == AFFINE && BITS == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t b = (w[0] >> (2 * j)) & 0x03030303u;
            asm("" : "+v"(b));
            st.pre[j] = b;
        }
    }
}

template <int B>
__device__ __forceinline__ float byte_f32(uint32_t v) {
    return (float)((v >> (8 * B)) & 0xFFu);
}

// Packed bf16 pair Q (codes 2Q and 2Q + 1 of the chunk, natural k order).
template <int MODE, int BITS, int WORDS, int NWO, int Q>
__device__ __forceinline__ uint32_t dq_pair(const DqState<MODE, BITS, NWO>& st, const uint32_t* w) {
    const float s = st.s, z = st.z;
    if constexpr (MODE == AFFINE && BITS == 4) {
        return pack_bf16(__builtin_fmaf(s, byte_f32<Q>(st.pre[0]), z),
                         __builtin_fmaf(s, byte_f32<Q>(st.pre[1]), z));
    } else if constexpr (MODE == AFFINE && BITS == 8) {
        const uint32_t v = w[Q / 2];
        return pack_bf16(__builtin_fmaf(s, byte_f32<(2 * Q) % 4>(v), z),
                         __builtin_fmaf(s, byte_f32<(2 * Q) % 4 + 1>(v), z));
    } else if constexpr (MODE == AFFINE) {   // 2-bit: code 4b + j is byte b of plane j
        return pack_bf16(__builtin_fmaf(s, byte_f32<Q / 2>(st.pre[2 * (Q % 2)]), z),
                         __builtin_fmaf(s, byte_f32<Q / 2>(st.pre[2 * (Q % 2) + 1]), z));
    } else if constexpr (MODE == NVFP4) {
        return e2m1_pair_times<Q>(w[0], s);
    } else if constexpr (BITS == 4) {        // mxfp4: the E8M0 scale is a power of two
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], s, Q));
    } else {                                  // mxfp8
        return __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[Q / 2], s, (Q % 2) == 1));
    }
}

// BM activation rows x BN weight rows per workgroup of WM x WN waves; CPC
// codes per dequant chunk (8 or 16), chunks dealt round-robin to threads.
template <int MODE, int BITS, int G, int BM, int BN, int WM, int WN, int CPC, bool GATHER, int WPF, bool OB>
__global__ void __launch_bounds__(WM * WN * 64) qmm_prefill_kernel(PrefillArgs a) {
    constexpr int NTH = WM * WN * 64;
    constexpr int PER = 32 / BITS;
    constexpr int WORDS = CPC / PER;                  // packed dwords per chunk
    constexpr int CROW = BK / CPC;                    // chunks per weight row per step
    constexpr int NCH = BN * CROW;                    // chunks per step
    // run length: chunks of one row a thread dequantizes per step
    constexpr int RCH = (NCH % NTH == 0 && NCH / NTH <= CROW && CROW % (NCH / NTH) == 0) ? NCH / NTH : 1;
    constexpr int CPT = RCH > 1 ? 1 : (NCH + NTH - 1) / NTH;   // runs (or chunks) per thread
    constexpr int RWORDS = RCH * WORDS;               // packed dwords per run
    constexpr int MW = BM / WM, NW = BN / WN;         // wave tile
    constexpr int MT = MW / 16, NT = NW / 16;
    static_assert(WORDS >= 1 && G % CPC == 0, "a chunk lies inside one group");
    static_assert(MW % 16 == 0 && NW % 16 == 0, "wave tile is a multiple of the MFMA tile");
    constexpr int NWV = WM * WN;
    // activations are loaded XLA = 2 steps ahead into XST = 3 LDS stages
    constexpr int XLA = 2, XST = XLA + 1, XSTAGE = BM * BK * 2, WSTAGE = BN * LROW;
    constexpr int XDMA = BM * 8 / NTH;                 // activation loads per thread per step
    static_assert(XDMA * NTH == BM * 8, "activation tile splits into whole wave loads");

    // LDS: XST activation stages [BM][128 B] (swizzled), then two
    // dequantized weight buffers [BN][LROW]
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int i = lane & 15, j = lane >> 4;
    const int wm = wv / WN, wn_ = wv % WN;

    const int ntn = (a.N + BN - 1) / BN;
    int m0, n0;
    int expert = 0, row_begin = 0, row_count = a.M;   // GEMM rows of this tile's problem
    if constexpr (GATHER) {
        // (expert, row tile, column tile): the grid holds an upper bound on
        // the row tiles; tiles past the real count leave at once
        int tile_m = blockIdx.x / ntn;
        n0 = (blockIdx.x % ntn) * BN;
        if (tile_m >= (int)a.tiles[a.E]) return;
        int lo = 0, hi = a.E;                     // tiles[lo] <= tile_m < tiles[lo + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if ((int)a.tiles[mid] <= tile_m) lo = mid; else hi = mid;
        }
        expert = lo;
        m0 = (tile_m - (int)a.tiles[lo]) * BM;
        row_begin = (int)a.offsets[lo];
        row_count = ((int)a.offsets[lo + 1] - row_begin) * a.M;
    } else {
        // Blocks are dealt to the XCDs round-robin (XCD = blockIdx % xcds).
        // With xgm > 0 the host has split the tile grid into xgm x
        // (xcds/xgm) equal blocks, one per XCD, so an XCD's L2 fetches only
        // its block's share of x and W (each XCD walking a row of tiles
        // fetched all of W); otherwise each XCD walks a contiguous run of
        // tiles along N.
        const int b = blockIdx.x;
        if (a.xgm > 0) {
            const int xgn = a.xcds / a.xgm, ntm = (a.M + BM - 1) / BM;
            const int mt = ntm / a.xgm, nt = ntn / xgn;      // tiles per XCD block
            const int x = b % a.xcds, j = b / a.xcds;
            m0 = ((x / xgn) * mt + j / nt) * BM;
            n0 = ((x % xgn) * nt + j % nt) * BN;
        } else {
            const int bb = xcd_block(b, gridDim.x, a.xcds);
            m0 = (bb / ntn) * BM;
            n0 = (bb % ntn) * BN;
        }
    }
    if (a.lds_nan) {   // debug: every LDS byte of the tile starts as NaN
        constexpr int LDS_BYTES = XST * XSTAGE + 2 * WSTAGE;
        static_assert(LDS_BYTES % 16 == 0, "16-byte fill");
        for (int o = tid * 16; o < LDS_BYTES; o += NTH * 16)
            *(u32x4*)(smem + o) = u32x4{~0u, ~0u, ~0u, ~0u};
        __syncthreads();
    }
    // GEMM row rho of the tile's problem -> index row (gather) / x row / y row
    auto x_row = [&](int rho) -> uint32_t {
        if constexpr (GATHER) {
            const uint32_t ir = a.perm[row_begin + rho / a.M];
            const uint32_t bx = a.lhs ? a.lhs[ir] : ir;
            return bx * (uint32_t)a.M + (uint32_t)(rho % a.M);
        } else {
            return (uint32_t)rho;
        }
    };
    auto y_row = [&](int rho) -> size_t {
        if constexpr (GATHER)
            return (size_t)a.perm[row_begin + rho / a.M] * a.M + (size_t)(rho % a.M);
        else
            return (size_t)rho;
    };

    const uint32_t K = (uint32_t)a.K;
    const uint32_t xrows = GATHER ? (uint32_t)a.B * (uint32_t)a.M : (uint32_t)a.M;
    const uint32_t nrows = (uint32_t)(GATHER ? a.E : 1) * (uint32_t)a.N;  // stacked weight rows
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, xrows * K * 2u);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wq, nrows * (K / PER) * 4u);
    const uint32_t ngroups = K / G;
    constexpr uint32_t SB = MODE == AFFINE ? 2u : 1u;  // scale bytes
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.scales, nrows * ngroups * SB);
    const __amdgpu_buffer_rsrc_t br =
        make_rsrc(MODE == AFFINE ? (const void*)a.biases : a.scales,
                  MODE == AFFINE ? nrows * ngroups * 2u : 0u);

    // ---- activation tile: XST stages in LDS, each BM rows x 128 bytes,
    // filled by buffer->LDS loads. One wave instruction moves 8 rows (1 KB,
    // 16 bytes per lane, lane order). Row r keeps its 16-byte chunk c in slot
    // c ^ (r & 7), so the 16 rows an MFMA fragment reads at one k hit 8
    // different slots. (Also flipping the slot with bit 3 of the row, which
    // spreads the 16 rows over 16 bank groups, measured 1-2 % slower.)
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    uint32_t xdoff[XDMA];
#pragma unroll
    for (int q = 0; q < XDMA; ++q) {
        const int r = (q * NWV + wv) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        // rows past the problem read zeros: their offset is past the buffer
        xdoff[q] = m0 + r < row_count ? (x_row(m0 + r) * K + (uint32_t)c * 8u) * 2u : 0x80000000u;
    }
    auto dma_x = [&](int stage, int kt) {
#pragma unroll
        for (int q = 0; q < XDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(smem + stage * XSTAGE + (q * NWV + wvu) * 1024),
                16, (int)xdoff[q], kt * (BK * 2), 0, 0);
    };
    // fragment (s, kh) of this lane: row wm*MW + s*16 + i, chunk 4 kh + j
    const uint32_t xfrag0 = (uint32_t)(wm * MW + i) * 128u;

    // ---- dequant work. With runs (RCH > 1) a thread owns RCH consecutive
    // chunks of one weight row per step: one load of RCH*CPC codes and one
    // scale (and bias) load of the groups they span. Otherwise chunk
    // c = tid + p*NTH -> weight row c / CROW, chunk c % CROW; spare slots of an
    // uneven split reload the last chunk and skip the store.
    uint32_t woff[CPT], rowg[CPT], ldsoff[CPT];
    int ccv[CPT];
    bool cact[CPT];
#pragma unroll
    for (int p = 0; p < CPT; ++p) {
        int r, cc;
        if constexpr (RCH > 1) {
            r = tid / (CROW / RCH);
            cc = (tid % (CROW / RCH)) * RCH;
            cact[p] = true;
        } else {
            int c = tid + p * NTH;
            cact[p] = c < NCH;
            c = c < NCH ? c : NCH - 1;
            r = c / CROW;
            cc = c % CROW;
        }
        // rows past N read the next expert's rows (or zeros past the end);
        // their outputs are never stored
        const uint32_t n = (uint32_t)expert * (uint32_t)a.N + (uint32_t)(n0 + r);
        woff[p] = (n * (K / PER) + (uint32_t)cc * WORDS) * 4u;
        rowg[p] = n * ngroups * SB;                         // first scale byte of the row
        ccv[p] = cc;
        ldsoff[p] = (uint32_t)r * LROW + (uint32_t)cc * CPC * 2u;
    }
    // Scales and biases: one load per weight row for a batch of WPF steps
    // (the groups those steps cover, NBB bytes), instead of one small load per
    // chunk and step: the lanes of a row share one request. Batch b covers
    // steps [b * WPF, (b + 1) * WPF); the host picks WPF dividing the step
    // count, so a batch is NBB-aligned in every row. Bits stay raw until the
    // dequant step, so nothing waits on these loads before they are needed.
    constexpr bool WHOLE = (WPF * BK) % G == 0;         // a batch covers whole groups
    constexpr int NGB = WHOLE ? WPF * BK / G : 1;       // groups per batch
    constexpr int NBB = NGB * (int)SB;                  // bytes per batch and row
    constexpr int BD = NBB < 4 ? 1 : NBB / 4;           // dwords per batch and row
    static_assert(NBB <= 16, "a batch is at most 16 bytes per row");
    auto load_codes = [&](Chunk<RWORDS> (&dst)[CPT], int kt) {
#pragma unroll
        for (int p = 0; p < CPT; ++p) dst[p] = load_chunk<RWORDS>(wr, woff[p], kt * (BK / PER) * 4);
    };
    auto load_batch = [&](uint32_t (&ds)[CPT][BD], uint32_t (&dz)[CPT][BD], int kt0) {
        const int first = (kt0 * BK) / G;  // first group of the batch (scalar)
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            load_bytes<NBB>(sr, rowg[p], first * (int)SB, ds[p]);
            if constexpr (MODE == AFFINE) load_bytes<NBB>(br, rowg[p], first * (int)SB, dz[p]);
        }
    };
    // Dequantization of one step (step place T in its batch) as NITEM
    // items: per chunk (p, h) of this thread, one item that decodes the
    // scale and bias and splits the codes, NWO items of one packed bf16 pair
    // each, and one item that writes the chunk to LDS. The group of chunk
    // (p, h) is (T * BK + k) / G within the batch, k its offset in the step;
    // a step's scale bytes never straddle a dword, so the dword is known at
    // compile time and only the byte shift depends on the lane.
    constexpr int NWO = CPC / 2;                  // packed bf16 pairs per chunk
    constexpr int NCK = CPT * RCH;                // chunks per thread and step
    constexpr int NITEM = NCK * (NWO + 2);
    using DqSt = DqState<MODE, BITS, NWO>;
    auto dq_item = [&](auto ic, DqSt (&st)[NCK], unsigned char* base, const Chunk<RWORDS> (&wc)[CPT],
                       const uint32_t (&sc)[CPT][BD], const uint32_t (&zc)[CPT][BD], auto tc) {
        constexpr int I = decltype(ic)::value, T = decltype(tc)::value;
        constexpr int C = I / (NWO + 2), R = I % (NWO + 2);
        constexpr int P = C / RCH, H = C % RCH;
        constexpr int DW = WHOLE ? (((T * BK) / G) * (int)SB) / 4 : 0;
        static_assert(DW < BD, "batch dword");
        if constexpr (R == 0) {
            int sh = 0;
            if constexpr (WHOLE && G >= BK) {
                sh = 8 * ((((T * BK) / G) * (int)SB) & 3);
            } else if constexpr (WHOLE) {
                const int byte = ((T * BK + (ccv[P] + H) * CPC) / G) * (int)SB;
                sh = 8 * (byte - 4 * DW);
            }
            if constexpr (MODE == AFFINE) {
                st[C].s = bf16_bits_to_f32((sc[P][DW] >> sh) & 0xFFFFu);
                st[C].z = bf16_bits_to_f32((zc[P][DW] >> sh) & 0xFFFFu);
            } else {
                const uint32_t byte = (sc[P][DW] >> sh) & 0xFFu;
                st[C].s = MODE == NVFP4 ? e4m3_to_f32(byte) : e8m0_to_f32(byte);
                st[C].z = 0.f;
            }
            dq_prepare<MODE, BITS, WORDS, NWO>(st[C], &wc[P].w[H * WORDS]);
        } else if constexpr (R <= NWO) {
            st[C].o[R - 1] = dq_pair<MODE, BITS, WORDS, NWO, R - 1>(st[C], &wc[P].w[H * WORDS]);
        } else {
            if (RCH == 1 && NCH % NTH != 0 && !cact[P]) return;
#pragma unroll
            for (int q = 0; q < CPC / 8; ++q)
                *(u32x4*)(base + ldsoff[P] + H * CPC * 2 + q * 16) =
                    u32x4{st[C].o[4 * q], st[C].o[4 * q + 1], st[C].o[4 * q + 2], st[C].o[4 * q + 3]};
        }
    };
    // the whole dequantization of one step, item after item
    auto store_w = [&](unsigned char* base, const Chunk<RWORDS> (&wc)[CPT], const uint32_t (&sc)[CPT][BD],
                       const uint32_t (&zc)[CPT][BD], auto tc) {
        DqSt st[NCK];
        unroll<0, NITEM>([&](auto ic) { dq_item(ic, st, base, wc, sc, zc, tc); });
    };

    // accumulators start at zero, or (OB: the dense layer's bias, a separate
    // instantiation so the plain kernel's code is untouched) at the bias of
    // the lane's output columns n = n0 + wn_*NW + 16t + 4j + r, added once
    // per output; the output stage is the plain matmul's
    f32x4 acc[NT][MT];
    if constexpr (!OB) {
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
                const int n = n0 + wn_ * NW + t * 16 + 4 * j + r;
                b[r] = n < a.N ? out_bias_at(a.ob, n) : 0.f;
            }
#pragma unroll
            for (int s = 0; s < MT; ++s) acc[t][s] = b;
        }
        __builtin_amdgcn_sched_barrier(0);   // bias loads before the tile loads
    }

    const int nk = a.K / BK;
    // WPF register sets hold the packed codes of steps kt+1 .. kt+WPF; set
    // u % WPF belongs to step u. The step loop is unrolled WPF times so set
    // indices are compile-time.
    Chunk<RWORDS> wset[WPF][CPT];
    // scale/bias batches: the current one (steps kt0 .. kt0+WPF-1) and the next
    uint32_t scur[CPT][BD], zcur[CPT][BD], snxt[CPT][BD], znxt[CPT][BD];
    unsigned char* const wbuf = smem + XST * XSTAGE;

    constexpr int WL = CPT * (RWORDS == 8 ? 2 : 1);            // code loads per step
    constexpr int BL = CPT * (MODE == AFFINE ? 2 : 1);         // batch loads (steps U = 0)
    auto rd_a = [&](const unsigned char* wt, int kh, int t) -> u32x4 {
        return *(const u32x4*)(wt + (wn_ * NW + t * 16 + i) * LROW + (kh * 32 + 8 * j) * 2);
    };
    auto rd_b = [&](const unsigned char* xt, int kh, int s2) -> u32x4 {
        return *(const u32x4*)(xt + xfrag0 + s2 * 2048 + (((kh * 4 + j) ^ (i & 7)) << 4));
    };
    constexpr int RB = NT >= 2 ? NT - 2 : 0;   // row during which the other half's activation fragments are read

    if constexpr (WPF == 4) {
        // ---- Pipelined form (batches of 4 steps). One barrier per step, in
        // its middle, so that no wave starts MFMAs on fragments it has just
        // asked for:
        //   first half of step kt : MFMAs of k half 0; read k half 1's
        //     fragments of step kt; dequantization items [NH, NITEM) of step
        //     kt+1 (into W buffer (kt+1)&1)
        //   barrier B_kt          : activations of step kt+1 in LDS, every
        //     wave's dequantization of step kt+1 and reads of step kt's W
        //     buffer and x stage complete (vmcnt as below, lgkmcnt(0))
        //   second half           : DMA of step kt+3 (into step kt's x
        //     stage), codes of step kt+4 (into step kt's code set), the next
        //     batch of scales (U = 0); MFMAs of k half 1; read k half 0's
        //     fragments of step kt+1; items [0, NH) of step kt+2 (into step
        //     kt's W buffer, free since B_kt)
        // Loads past the last step are clamped to it and their results are
        // never used (reads of LDS the last steps overwrite are never used
        // either).
        constexpr int NH = NITEM / 2;
        constexpr int SLOTS = NT * MT;
        // vm operations complete in order. At B_kt the DMA of step kt+1
        // (issued in the second half of step kt-2) must have landed; issued
        // after it: the codes of that half, its batch when it opened one
        // (U = 2), the next half's DMA and codes, and its batch (U = 1).
        static_assert(XDMA + 2 * WL + BL < 64, "vmcnt range");
        DqSt st[NCK];   // dequantization state carried from one half to the next
        auto items = [&](auto lo, auto hi, auto q, auto span, DqSt (&s)[NCK], unsigned char* base,
                         const Chunk<RWORDS> (&wc)[CPT], const uint32_t (&sc)[CPT][BD],
                         const uint32_t (&zc)[CPT][BD], auto tc) {
            // items [LO, HI) spread over SPAN slots; those of slot Q
            constexpr int LO = decltype(lo)::value, HI = decltype(hi)::value;
            constexpr int Q = decltype(q)::value, SP = decltype(span)::value;
            constexpr int N = HI - LO;
            constexpr int A = LO + (Q * N + SP - 1) / SP, B = LO + ((Q + 1) * N + SP - 1) / SP;
            unroll<(A < HI ? A : HI), (B < HI ? B : HI)>([&](auto ic) { dq_item(ic, s, base, wc, sc, zc, tc); });
        };
        constexpr int SPAN = SLOTS > 1 ? SLOTS - 1 : 1;   // the last slot of a half carries no items

        // prologue. vm issue order: batch 0, codes 0, DMA 0, codes 1, DMA 1,
        // codes 2, DMA 2, codes 3 -- after DMA 1 the loop's count for B_0
        // (codes, DMA, codes); after DMA 2 that of B_1 with step 0's loads.
        load_batch(scur, zcur, 0);
        load_codes(wset[0], 0);
        __builtin_amdgcn_sched_barrier(0);
        dma_x(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(wset[1], 1);
        __builtin_amdgcn_sched_barrier(0);
        dma_x(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(wset[2], 2);
        __builtin_amdgcn_sched_barrier(0);
        dma_x(2, 2);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(wset[3], 3);
        __builtin_amdgcn_sched_barrier(0);
        // step 0's weights whole; the first half of step 1's items
        store_w(wbuf, wset[0], scur, zcur, std::integral_constant<int, 0>{});
        unroll<0, NH>([&](auto ic) {
            dq_item(ic, st, wbuf + WSTAGE, wset[1], scur, zcur, std::integral_constant<int, 1>{});
        });
        // activations of step 0 in LDS (issued after them: codes 1, DMA 1,
        // codes 2, DMA 2, codes 3), this wave's W writes done
        __builtin_amdgcn_s_waitcnt(vm_lgkm0(2 * XDMA + 3 * WL));
        asm volatile("s_barrier" ::: "memory");
        u32x4 af[NT], bf0[MT], bf1[MT];
#pragma unroll
        for (int t = 0; t < NT; ++t) af[t] = rd_a(wbuf, 0, t);
#pragma unroll
        for (int s2 = 0; s2 < MT; ++s2) bf0[s2] = rd_b(smem, 0, s2);
        __builtin_amdgcn_sched_barrier(0);

        auto step = [&](int kt, auto uc) {
            constexpr int U = decltype(uc)::value;       // kt % 4
            const unsigned char* xt = smem + (kt % XST) * XSTAGE;
            const unsigned char* wt = wbuf + (kt & 1) * WSTAGE;
            const unsigned char* xn = smem + ((kt + 1) % XST) * XSTAGE;
            const unsigned char* wn = wbuf + ((kt + 1) & 1) * WSTAGE;
            unsigned char* const w1 = wbuf + ((kt + 1) & 1) * WSTAGE;   // step kt+1's W buffer
            unsigned char* const w2 = wbuf + (kt & 1) * WSTAGE;         // step kt+2's W buffer
            // ---- first half
            unroll<0, SLOTS>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                constexpr int TT = Q / MT, SS = Q % MT;
                acc[TT][SS] = mfma_bf16(af[TT], bf0[SS], acc[TT][SS]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SS == MT - 1) af[TT] = rd_a(wt, 1, TT);
                if constexpr (TT == RB) bf1[SS] = rd_b(xt, 1, SS);
                // step kt+1 = 4b + U + 1: batch b for U < 3, else b + 1
                if constexpr (U < 3)
                    items(std::integral_constant<int, NH>{}, std::integral_constant<int, NITEM>{}, qc,
                          std::integral_constant<int, SPAN>{}, st, w1, wset[(U + 1) % 4], scur, zcur,
                          std::integral_constant<int, (U + 1) % 4>{});
                else
                    items(std::integral_constant<int, NH>{}, std::integral_constant<int, NITEM>{}, qc,
                          std::integral_constant<int, SPAN>{}, st, w1, wset[(U + 1) % 4], snxt, znxt,
                          std::integral_constant<int, (U + 1) % 4>{});
                __builtin_amdgcn_sched_barrier(0);
            });
            __builtin_amdgcn_s_waitcnt(vm_lgkm0(XDMA + 2 * WL + ((U == 1 || U == 2) ? BL : 0)));
            asm volatile("s_barrier" ::: "memory");
            // ---- second half: loads first (the waits count on their order)
            dma_x(kt % XST, kt + 3 < nk ? kt + 3 : nk - 1);
            __builtin_amdgcn_sched_barrier(0);
            load_codes(wset[U], kt + 4 < nk ? kt + 4 : nk - 1);
            if constexpr (U == 0) load_batch(snxt, znxt, kt + 4 < nk ? kt + 4 : nk - 4);
            __builtin_amdgcn_sched_barrier(0);
            unroll<0, SLOTS>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                constexpr int TT = Q / MT, SS = Q % MT;
                acc[TT][SS] = mfma_bf16(af[TT], bf1[SS], acc[TT][SS]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (SS == MT - 1) af[TT] = rd_a(wn, 0, TT);
                if constexpr (TT == RB) bf0[SS] = rd_b(xn, 0, SS);
                // step kt+2 = 4b + U + 2: batch b for U < 2, else b + 1
                if constexpr (U < 2)
                    items(std::integral_constant<int, 0>{}, std::integral_constant<int, NH>{}, qc,
                          std::integral_constant<int, SPAN>{}, st, w2, wset[(U + 2) % 4], scur, zcur,
                          std::integral_constant<int, (U + 2) % 4>{});
                else
                    items(std::integral_constant<int, 0>{}, std::integral_constant<int, NH>{}, qc,
                          std::integral_constant<int, SPAN>{}, st, w2, wset[(U + 2) % 4], snxt, znxt,
                          std::integral_constant<int, (U + 2) % 4>{});
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // the host picks WPF dividing the step count: every unrolled step runs
        for (int kt = 0; kt < nk; kt += 4) {
            unroll<0, 4>([&](auto u) { step(kt + decltype(u)::value, u); });
#pragma unroll
            for (int p = 0; p < CPT; ++p)
#pragma unroll
                for (int d = 0; d < BD; ++d) {
                    scur[p][d] = snxt[p][d];
                    zcur[p][d] = znxt[p][d];
                }
        }
    } else {
        // prologue: activations of steps 0 and 1 and codes of steps 0 .. WPF-1
        // in flight, step by step, each step's activation loads first (the
        // scheduling barriers keep that order: the waits below count on it);
        // step 0's weights dequantized into buffer 0
        constexpr int PRO = XLA > WPF ? XLA : WPF;
        unroll<0, PRO>([&](auto u) {
            constexpr int U = decltype(u)::value;
            if constexpr (U < XLA) dma_x(U, U < nk ? U : nk - 1);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (U < WPF) load_codes(wset[U], U < nk ? U : nk - 1);
            if constexpr (U == 0) load_batch(scur, zcur, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
        // waits for step 0's codes, issued after its activations
        store_w(wbuf, wset[0], scur, zcur, std::integral_constant<int, 0>{});
        __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): this wave's LDS writes done
        asm volatile("s_barrier" ::: "memory");

        // One step. Activation loads issued here land two steps later, code
        // loads WPF steps later. vm operations complete in order; at the end of
        // step kt the activations of step kt+1 (issued first in step kt-1, or in
        // the prologue) must be in LDS, so the wait may leave outstanding only
        // loads issued after them: step kt-1's code loads (and its batch of
        // scales and biases when it opened a batch) and all of step kt's loads.
        // With one step per batch (WPF = 1) only step kt's loads are counted
        // (the prologue issues nothing after step 1's activations). The step ends
        // with that wait, lgkmcnt(0) (this wave's LDS writes done) and a plain
        // s_barrier: a fenced barrier would also wait for this step's loads.
        auto wait_imm = [](int U) constexpr {
            int vm = XDMA + WL + (U == 0 ? BL : 0);                // this step
            if (WPF > 1) vm += WL + (U == 1 ? BL : 0);             // step kt-1 after its activations
            // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
            return (vm & 15) | (7 << 4) | (0 << 8) | ((vm >> 4) << 14);
        };
        static_assert(XDMA + 2 * WL + 2 * BL < 64, "vmcnt range");
        auto step = [&](int kt, auto uc) {
            constexpr int U = decltype(uc)::value;          // kt % WPF
            constexpr int CUR = (U + 1) % WPF;              // set of step kt+1 (dequantized now)
            const int kx = kt + XLA < nk ? kt + XLA : nk - 1;
            const int kw = kt + WPF < nk ? kt + WPF : nk - 1;
            dma_x((kt + XLA) % XST, kx);
            __builtin_amdgcn_sched_barrier(0);              // activations first (the wait counts on it)
            load_codes(wset[U], kw);                        // set U held step kt, dequantized last step
            if constexpr (U == 0) {
                // the next batch (steps kt+WPF .. kt+2*WPF-1; past the end: the last batch)
                load_batch(snxt, znxt, kt + WPF < nk ? kt + WPF : nk - WPF);
            }
            __builtin_amdgcn_sched_barrier(0);
            const unsigned char* xt = smem + (kt % XST) * XSTAGE;
            const unsigned char* wt = wbuf + (kt & 1) * WSTAGE;
            auto rd_a = [&](int kh, int t) -> u32x4 {
                return *(const u32x4*)(wt + (wn_ * NW + t * 16 + i) * LROW + (kh * 32 + 8 * j) * 2);
            };
            auto rd_b = [&](int kh, int s2) -> u32x4 {
                return *(const u32x4*)(xt + xfrag0 + s2 * 2048 + (((kh * 4 + j) ^ (i & 7)) << 4));
            };
            // Issue order (scheduling barriers keep it): the first k half's
            // fragments; then the step's 2 * NT * MT MFMAs one by one, after each
            // its share of the next step's dequantization items (a few VALU
            // instructions, which run while the MFMA does); the second half's
            // weight fragment of row t is read once row t's first-half MFMAs are
            // issued (same registers), its activation fragments during the
            // first half's last rows.
            constexpr int NS = 2 * NT * MT;
            constexpr int SPAN = NS > 2 ? NS - 2 : 1;     // the last slots carry no items
            constexpr int RB = NT >= 2 ? NT - 2 : 0;
            u32x4 af[NT], bf0[MT], bf1[MT];
    #pragma unroll
            for (int t = 0; t < NT; ++t) af[t] = rd_a(0, t);
    #pragma unroll
            for (int s2 = 0; s2 < MT; ++s2) bf0[s2] = rd_b(0, s2);
            __builtin_amdgcn_sched_barrier(0);
            DqSt st[NCK];
            constexpr int TN = U + 1 < WPF ? U + 1 : 0;  // step kt+1's place in its batch
            unsigned char* const wnext = wbuf + ((kt + 1) & 1) * WSTAGE;
            unroll<0, NS>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                constexpr int KH = Q / (NT * MT), TT = (Q % (NT * MT)) / MT, SS = Q % MT;
                if constexpr (KH == 0)
                    acc[TT][SS] = mfma_bf16(af[TT], bf0[SS], acc[TT][SS]);
                else
                    acc[TT][SS] = mfma_bf16(af[TT], bf1[SS], acc[TT][SS]);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (KH == 0 && SS == MT - 1) af[TT] = rd_a(1, TT);
                if constexpr (KH == 0 && TT == RB) bf1[SS] = rd_b(1, SS);
                // items I with I * SPAN / NITEM == Q
                constexpr int ILO = (Q * NITEM + SPAN - 1) / SPAN, IHI = ((Q + 1) * NITEM + SPAN - 1) / SPAN;
                unroll<(ILO < NITEM ? ILO : NITEM), (IHI < NITEM ? IHI : NITEM)>([&](auto ic) {
                    // step kt+1 is the next batch's first step when U is the last place
                    if constexpr (U + 1 < WPF)
                        dq_item(ic, st, wnext, wset[CUR], scur, zcur, std::integral_constant<int, TN>{});
                    else
                        dq_item(ic, st, wnext, wset[CUR], snxt, znxt, std::integral_constant<int, TN>{});
                });
                __builtin_amdgcn_sched_barrier(0);
            });
            constexpr int WAIT_IMM = wait_imm(U);
            __builtin_amdgcn_s_waitcnt(WAIT_IMM);
            asm volatile("s_barrier" ::: "memory");
        };
        // the host picks WPF dividing the step count, so every unrolled step runs
        // (a conditional step would blur the compiler's load-count bookkeeping)
        for (int kt = 0; kt < nk; kt += WPF) {
            unroll<0, WPF>([&](auto u) { step(kt + decltype(u)::value, u); });
    #pragma unroll
            for (int p = 0; p < CPT; ++p)
    #pragma unroll
                for (int d = 0; d < BD; ++d) {
                    scur[p][d] = snxt[p][d];
                    zcur[p][d] = znxt[p][d];
                }
        }

    }
    // nothing of this workgroup may still be landing in LDS when it ends
    __builtin_amdgcn_s_waitcnt(0);

    // ---- epilogue: lane holds D[n = 4j + r][m = i] of each (t, s) tile
#pragma unroll
    for (int s = 0; s < MT; ++s) {
        const int m = m0 + wm * MW + s * 16 + i;
        if (m >= row_count) continue;
        uint16_t* yr = a.y + y_row(m) * a.N;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int n = n0 + wn_ * NW + t * 16 + 4 * j;
            const f32x4 v = acc[t][s];
            if (n + 3 < a.N && (a.N & 3) == 0) {
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

// code prefetch depth (steps): the plain and gather tiles alike
constexpr int kPrefillWpf = 4;


// Launch one kernel with `shm` bytes of dynamic LDS; the attribute that
// allows more than the default is set once per kernel (an atomic flag each,
// so concurrent callers at worst set it twice).
template <auto KERN>
hipError_t launch_with_lds(const PrefillArgs& t, int grid, int threads, size_t shm, hipStream_t st) {
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    KERN<<<grid, threads, shm, st>>>(t);
    return hipGetLastError();
}

template <int MODE, int BITS, int G, int BM, int BN, int WM, int WN, int CPC0, bool GATHER,
          bool OB = false>
hipError_t launch_cfg(const PrefillArgs& t, int grid, hipStream_t st) {
    // a chunk holds at least one packed dword
    constexpr int CPC = CPC0 < 32 / BITS ? 32 / BITS : CPC0;
    // The pipelined form (4-step batches) fits the registers of wave tiles
    // of up to 16 MFMA tiles. On the 64 x 96 wave tile it needs 4-bit codes
    // and batches of at most 8 bytes per row: 2-bit codes (four code planes
    // per chunk), 8-bit codes (two dwords per chunk) or 16-byte batches (two
    // sets) spill there (2-bit g64 ran 2.6x slower); those take the two-step
    // form.
    constexpr int SBY = MODE == AFFINE ? 2 : 1;
    constexpr int B4 = (4 * BK / G > 0 ? 4 * BK / G : 1) * SBY;
    constexpr int WTILES = (BM / WM / 16) * (BN / WN / 16);
    constexpr bool PIPE = WTILES <= 16 || (B4 <= 8 && BITS == 4);
    // gather tiles 384 rows wide hold twice the codes per thread and take
    // the two-step form (the pipelined one spilled: 108 against 77 us)
    constexpr int WPF = GATHER ? (BN > 192 ? 2 : kPrefillWpf) : (PIPE ? kPrefillWpf : 2);
    const size_t shm = (size_t)3 * BM * BK * 2 + (size_t)2 * BN * LROW;
    static_assert(3 * BM * BK * 2 + 2 * BN * LROW <= 160 * 1024, "LDS budget");
    constexpr int NTH = WM * WN * 64;
    // the code prefetch depth must divide the number of 64-wide steps
    const int nk = t.K / BK;
    if (nk % WPF == 0)
        return launch_with_lds<qmm_prefill_kernel<MODE, BITS, G, BM, BN, WM, WN, CPC, GATHER, WPF, OB>>(
            t, grid, NTH, shm, st);
    if (nk % 2 == 0)
        return launch_with_lds<qmm_prefill_kernel<MODE, BITS, G, BM, BN, WM, WN, CPC, GATHER, 2, OB>>(
            t, grid, NTH, shm, st);
    return launch_with_lds<qmm_prefill_kernel<MODE, BITS, G, BM, BN, WM, WN, CPC, GATHER, 1, OB>>(
        t, grid, NTH, shm, st);
}

// XCD grid for the plain form: the xcds XCDs take an xgm x (xcds/xgm) grid
// of equal tile blocks; xgm minimises what the XCDs fetch in all, xgm copies
// of the weight plus xcds/xgm copies of x (0: the tile grid does not split
// evenly).
inline int xcd_grid_rows(int64_t ntm, int64_t ntn, double w_bytes, double x_bytes, int xcds) {
    int best = 0;
    double best_cost = 0;
    for (int gm = 1; gm <= xcds; ++gm) {
        if (xcds % gm) continue;
        const int gn = xcds / gm;
        if (ntm % gm || ntn % gn) continue;
        const double cost = gm * w_bytes + gn * x_bytes;
        if (best == 0 || cost < best_cost) {
            best = gm;
            best_cost = cost;
        }
    }
    return best;
}

template <int MODE, int BITS, int G, int BM, int BN, int WM, int WN, int CPC0>
hipError_t launch_plain(const PrefillArgs& t0, hipStream_t st) {
    PrefillArgs t = t0;
    const int64_t ntm = (t.M + BM - 1) / BM, ntn = (t.N + BN - 1) / BN;
    const double w_bytes = (double)t.N * t.K * BITS / 8.0, x_bytes = (double)t.M * t.K * 2.0;
    t.xcds = device_shape().xcds;
    t.xgm = xcd_grid_rows(ntm, ntn, w_bytes, x_bytes, t.xcds);
    const int grid = (int)(ntm * ntn);
    if (t.ob.kind != OB_NONE) return launch_cfg<MODE, BITS, G, BM, BN, WM, WN, CPC0, false, true>(t, grid, st);
    return launch_cfg<MODE, BITS, G, BM, BN, WM, WN, CPC0, false>(t, grid, st);
}

// Tile shapes, all 8 waves (two per SIMD): 256 x 192 (64 x 96 per wave) is
// the most efficient per tile; 256 x 128 and 128 x 128 give more tiles when
// the grid would not fill the chip. The choice minimises the tile area
// times the number of rounds of 256 workgroups, with a per-shape efficiency.
enum PrefillCfg { CFG_256x192 = 0, CFG_256x128 = 1, CFG_128x128 = 2, CFG_128x256 = 3 };

int pick_cfg(int64_t M, int64_t N) {
    const int64_t bm[4] = {256, 256, 128, 128}, bn[4] = {192, 128, 128, 256};
    const double eff[4] = {1.0, 0.95, 0.75, 0.9};
    int best = 0;
    double best_cost = 0;
    for (int c = 0; c < 4; ++c) {
        const int64_t tiles = ((M + bm[c] - 1) / bm[c]) * ((N + bn[c] - 1) / bn[c]);
        const double cost = (double)((tiles + 255) / 256) * (double)(bm[c] * bn[c]) / eff[c];
        if (c == 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

template <int MODE, int BITS, int G>
hipError_t launch_fmt(const QmmArgs& q, hipStream_t st) {
    PrefillArgs t{};
    t.x = (const uint16_t*)q.x;
    t.wq = q.wq;
    t.scales = q.scales;
    t.biases = (const uint16_t*)q.biases;
    t.y = (uint16_t*)q.y;
    t.M = (int)q.M;
    t.N = (int)q.N;
    t.K = (int)q.K;
    t.ob = q.ob;
    t.lds_nan = debug_lds_nan();
    int cfg = pick_cfg(q.M, q.N);
    if (const char* e = getenv("QLIN_PREFILL_TILE")) cfg = atoi(e) % 4;  // tests of each shape
    switch (cfg) {
    case CFG_256x128: return launch_plain<MODE, BITS, G, 256, 128, 4, 2, 8>(t, st);
    case CFG_128x128: return launch_plain<MODE, BITS, G, 128, 128, 2, 4, 8>(t, st);
    case CFG_128x256: return launch_plain<MODE, BITS, G, 128, 256, 2, 4, 8>(t, st);
    default: return launch_plain<MODE, BITS, G, 256, 192, 4, 2, 8>(t, st);
    }
}

// Expert-bucketed rows: BM = 64 or 128 rows of one expert (the same height
// as the bucketing, prefill_gather_tile_rows), 192 weight rows, 32 x 48 or
// 64 x 48 per wave.
template <int MODE, int BITS, int G>
hipError_t launch_gather_fmt(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                             hipStream_t st) {
    PrefillArgs t{};
    t.x = (const uint16_t*)q.x;
    t.wq = q.wq;
    t.scales = q.scales;
    t.biases = (const uint16_t*)q.biases;
    t.y = (uint16_t*)q.y;
    t.M = (int)q.M;
    t.N = (int)q.N;
    t.K = (int)q.K;
    t.lhs = q.lhs;
    t.perm = perm;
    t.offsets = offsets;
    t.tiles = offsets + (q.E + 1);
    t.E = (int)q.E;
    t.B = (int)q.batch_x;
    t.lds_nan = debug_lds_nan();
    constexpr int BN = 192;
    const int BM = prefill_gather_tile_rows(q.R * q.M, q.E);
    // upper bound on row tiles: every expert may add one partial tile
    const int64_t mt = (q.R * q.M + BM - 1) / BM + q.E;
    const int grid = (int)(mt * ((q.N + BN - 1) / BN));
    if (BM == 128) {
        // 128-row tiles of 4-bit codes whose scale batches fit the pipelined
        // form on a 64 x 96 wave tile: 384 weight rows per tile, half the
        // workgroups, and fragment reads from LDS per MFMA cut by 30 %
        // (64 x 96 wave tiles instead of 64 x 48)
        constexpr int SBY = MODE == AFFINE ? 2 : 1;
        constexpr bool WIDE = BITS == 4 && (4 * BK / G) * SBY <= 8;
        if constexpr (WIDE) {
            if (q.N > BN) {
                const int grid2 = (int)(mt * ((q.N + 2 * BN - 1) / (2 * BN)));
                return launch_cfg<MODE, BITS, G, 128, 2 * BN, 2, 4, 8, true>(t, grid2, st);
            }
        }
        return launch_cfg<MODE, BITS, G, 128, BN, 2, 4, 8, true>(t, grid, st);
    }
    return launch_cfg<MODE, BITS, G, 64, BN, 2, 4, 8, true>(t, grid, st);
}

}  // namespace

namespace {

template <int MODE, int BITS, int G>
struct FmtTag {};

// Calls fn(FmtTag<mode, bits, group>{}) for the (mode, bits, group) of q.
template <class Fn>
hipError_t dispatch_fmt(const QmmArgs& q, Fn&& fn) {
    switch (q.mode) {
    case MXFP4: return fn(FmtTag<MXFP4, 4, 32>{});
    case NVFP4: return fn(FmtTag<NVFP4, 4, 16>{});
    case MXFP8: return fn(FmtTag<MXFP8, 8, 32>{});
    default: break;
    }
    if (q.bits == 4) {
        if (q.group_size == 32) return fn(FmtTag<AFFINE, 4, 32>{});
        if (q.group_size == 64) return fn(FmtTag<AFFINE, 4, 64>{});
        return fn(FmtTag<AFFINE, 4, 128>{});
    }
    if (q.bits == 8) {
        if (q.group_size == 32) return fn(FmtTag<AFFINE, 8, 32>{});
        if (q.group_size == 64) return fn(FmtTag<AFFINE, 8, 64>{});
        return fn(FmtTag<AFFINE, 8, 128>{});
    }
    if (q.group_size == 32) return fn(FmtTag<AFFINE, 2, 32>{});
    if (q.group_size == 64) return fn(FmtTag<AFFINE, 2, 64>{});
    return fn(FmtTag<AFFINE, 2, 128>{});
}

template <int MODE, int BITS, int G>
hipError_t launch_tag(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                      hipStream_t st, FmtTag<MODE, BITS, G>) {
    if (q.R > 0) return launch_gather_fmt<MODE, BITS, G>(q, perm, offsets, st);
    return launch_fmt<MODE, BITS, G>(q, st);
}

}  // namespace

bool qmm_prefill_supports(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16) return false;
    // scales and biases are read in batches of up to 16 bytes per row
    if (((uintptr_t)q.scales & 15) != 0) return false;
    if (q.mode == AFFINE && ((uintptr_t)q.biases & 15) != 0) return false;
    if (q.K % BK != 0 || q.M < 1) return false;
    if (q.R > 0 && (q.E > 8192 || q.R * q.M >= (1LL << 30))) return false;
    // 32-bit buffer offsets over x, the (stacked) weight and its scales
    const int64_t xrows = q.R > 0 ? q.batch_x * q.M : q.M;
    const int64_t wrows = (q.R > 0 ? q.E : 1) * q.N;
    if (xrows * q.K * 2 >= (1LL << 31) || wrows * q.K * q.bits / 8 >= (1LL << 31)) return false;
    if (wrows * (q.K / q.group_size) * 2 >= (1LL << 31)) return false;
    return true;
}

hipError_t launch_qmm_prefill(const QmmArgs& q, const uint32_t* perm, const uint32_t* offsets,
                              hipStream_t st) {
    if (!qmm_prefill_supports(q)) return hipErrorNotSupported;
    if (q.R > 0 && (!perm || !offsets)) return hipErrorInvalidValue;
    return dispatch_fmt(q, [&](auto tag) { return launch_tag(q, perm, offsets, st, tag); });
}

}  // namespace qlin
