// qmm_prefill2.hip -- many-row quantized matmul for 4-bit affine weights on
// bf16 MFMA, software-pipelined (gfx950).
//
// y = x . dequant(W)^T for the [out, in] layout with bf16 activations
// ("EMLX.Quantization", quantized_matmul; "Emily.QuantizedWeight", Layout:
// 8 codes per uint32 along K, one scale and bias per group of G along K).
// The weight is dequantized in registers, straight into the MFMA operand;
// no dense weight tile exists anywhere, in memory or in LDS.
//
// Workgroup: 4 waves side by side along N, tile 128 activation rows (m) x
// 128 weight rows (n), each wave 128 x 32 (2 x 8 tiles of 16 x 16); two
// workgroups per CU, so one hides the other's barriers and LDS waits.
//  * Activations: global -> LDS by buffer->LDS loads into a 4-stage ring,
//    3 steps (of 64 k) ahead; row r keeps its 16-byte chunk c in slot
//    c ^ (r & 7) ^ ((r >> 3) & 1), so the 16 rows of a fragment read hit 16
//    distinct slots. The fragments of the next half step are read while the
//    MFMAs of the current one run.
//  * Weights: a lane loads 32 contiguous bytes of its row per block of 256
//    k (4 steps), the 4 lanes of a row together one whole 128-byte line; a
//    4 x 4 lane transpose (permlane16/32 swaps) then gives each lane, for
//    every step, the 8 codes its MFMA operand needs. Blocks are loaded one
//    block ahead.
//  * Dequantization: bf16(fmaf(s, q, z)) per code, the value rounded once to
//    the MFMA input type, the same as the first many-row kernel.
//  * One barrier per step, in its middle: before reading the next step's
//    first fragments, every wave's part of that step's activation tile has
//    landed. The waits are exact counts of loads issued in order.
// Rows past M or N read zeros (buffer range checks) and are never stored.

#include "qlin_common.h"

#include <atomic>

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int P2_BM = 128, P2_BN = 128, P2_NWV = 4, P2_THREADS = 64 * P2_NWV;
constexpr int P2_NT = P2_BN / P2_NWV / 16;   // weight tiles of 16 rows per wave
constexpr int P2_MT = P2_BM / 16;            // 8 activation tiles of 16 rows
constexpr int P2_BK = 64;                    // k per step
constexpr int P2_SPB = 4;                    // steps per code block (256 k = 128 bytes of a row)
constexpr int P2_XST = 4;                    // activation stages
constexpr int P2_XSTAGE = P2_BM * P2_BK * 2; // 16 KiB
constexpr int P2_XDMA = P2_BM / 8 / P2_NWV;  // activation DMA instructions per wave and step

struct P2Args {
    const uint16_t* x;       // bf16 [M, K]
    const uint32_t* wq;      // [N, K/8]
    const uint16_t* scales;  // bf16 [N, K/G]
    const uint16_t* biases;
    uint16_t* y;             // bf16 [M, N]
    int M, N, K;
    int xcds;                // XCDs of the device
    int lds_nan;             // debug: fill LDS with NaN before the tile
    int xgm;                 // the XCDs as an xgm x (xcds/xgm) grid of tile blocks (0: runs along N)
    OutBias ob;
};

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};   // nearest-even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 4x4 word transpose across the lane rows j = lane/16: before, lane row j
// holds v[c] = W[j][c]; after, v[c] = W[c][j].
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

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 8 codes of one word -> 8 dequantized bf16 values in k order (pairs).
__device__ __forceinline__ u32x4 deq8(uint32_t v, float s, float z) {
    const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
    u32x4 r;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        r[b] = pack_bf16(__builtin_fmaf(s, (float)((lo >> (8 * b)) & 0xFFu), z),
                         __builtin_fmaf(s, (float)((hi >> (8 * b)) & 0xFFu), z));
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Scale and bias bytes per row and block: one bf16 per group of the 256 k.
template <int G>
struct P2Scales {
    static constexpr int NB = (P2_SPB * P2_BK / G) * 2;   // 16 (G32), 8 (G64), 4 (G128)
    static constexpr int NW = NB / 4;
};

// Scales and biases of a lane's rows (one per tile) for one block.
template <int G>
struct P2Sc {
    uint32_t s[P2_NT][P2Scales<G>::NW], z[P2_NT][P2Scales<G>::NW];
};
// One block (4 steps) of a lane's weight data: 32 code bytes of its row in
// each of the wave's tiles, and the rows' scales and biases for the block.
template <int G>
struct P2Block {
    u32x4 c[P2_NT][2];
    P2Sc<G> sc;
};

template <int G, bool OB>
__global__ void __launch_bounds__(P2_THREADS, 2) qmm_prefill2_kernel(P2Args a) {
    using SC = P2Scales<G>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, j = lane >> 4;
    const uint32_t K = (uint32_t)a.K;

    // ---- tile: workgroups are dealt to the XCDs round-robin; with xgm > 0
    // the tile grid is split into xgm x (xcds/xgm) equal blocks, one per XCD
    const int ntn = (a.N + P2_BN - 1) / P2_BN, ntm = (a.M + P2_BM - 1) / P2_BM;
    int m0, n0;
    {
        const int b = blockIdx.x;
        if (a.xgm > 0) {
            const int xgn = a.xcds / a.xgm;
            const int mt = ntm / a.xgm, nt = ntn / xgn;
            const int x = b % a.xcds, q = b / a.xcds;
            m0 = ((x / xgn) * mt + q / nt) * P2_BM;
            n0 = ((x % xgn) * nt + q % nt) * P2_BN;
        } else {
            const int bb = xcd_block(b, gridDim.x, a.xcds);
            m0 = (bb / ntn) * P2_BM;
            n0 = (bb % ntn) * P2_BN;
        }
    }

    if (a.lds_nan) {   // debug: every LDS byte of the tile starts as NaN
        for (int o = tid * 16; o < P2_XST * P2_XSTAGE; o += P2_THREADS * 16)
            *(u32x4*)(smem + o) = u32x4{~0u, ~0u, ~0u, ~0u};
        __syncthreads();
    }
    const __amdgpu_buffer_rsrc_t xr = rsrc(a.x, (uint32_t)a.M * K * 2u);
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq, (uint32_t)a.N * (K / 2u));
    const uint32_t sbytes = (uint32_t)a.N * (K / G) * 2u;
    const __amdgpu_buffer_rsrc_t sr = rsrc(a.scales, sbytes);
    const __amdgpu_buffer_rsrc_t zr = rsrc(a.biases, sbytes);

    // ---- activation DMA: one wave instruction moves 8 rows x 128 bytes
    uint32_t xdoff[P2_XDMA];
#pragma unroll
    for (int q = 0; q < P2_XDMA; ++q) {
        const int r = (q * P2_NWV + wv) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        xdoff[q] = m0 + r < a.M ? ((uint32_t)(m0 + r) * K + (uint32_t)c * 8u) * 2u : 0x80000000u;
    }
    auto dma = [&](int stage, int kt) {
#pragma unroll
        for (int q = 0; q < P2_XDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(smem + stage * P2_XSTAGE + (q * P2_NWV + wv) * 1024),
                16, (int)xdoff[q], kt * P2_BK * 2, 0, 0);
    };
    // fragment (tile mt, k half kh) of this lane: row 16 mt + i, chunk 4 kh + j
    auto read_x = [&](int stage, int mt, int kh) -> u32x4 {
        const int r = 16 * mt + i;
        return *(const u32x4*)(smem + stage * P2_XSTAGE + r * (P2_BK * 2) + (((4 * kh + j) ^ swz(r)) << 4));
    };

    // ---- weight rows of this lane: n = n0 + (BN/4) wv + 16 t + i
    uint32_t woff[P2_NT], soff[P2_NT];
#pragma unroll
    for (int t = 0; t < P2_NT; ++t) {
        const int n = n0 + (P2_BN / P2_NWV) * wv + 16 * t + i;
        woff[t] = n < a.N ? (uint32_t)n * (K / 2u) + 32u * (uint32_t)j : 0x80000000u;
        soff[t] = n < a.N ? (uint32_t)n * (K / G) * 2u : 0x80000000u;
    }
    auto load_block = [&](P2Block<G>& d, int blk) {
        const int so = blk * 128;                 // code bytes of a row per block
        const int ss = blk * SC::NB;              // scale bytes of a row per block
#pragma unroll
        for (int t = 0; t < P2_NT; ++t) {
            d.c[t][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)woff[t], so, 0);
            d.c[t][1] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)woff[t], so + 16, 0);
            if constexpr (SC::NW == 4) {
                const u32x4 s4 = __builtin_amdgcn_raw_buffer_load_b128(sr, (int)soff[t], ss, 0);
                const u32x4 z4 = __builtin_amdgcn_raw_buffer_load_b128(zr, (int)soff[t], ss, 0);
#pragma unroll
                for (int w = 0; w < 4; ++w) { d.sc.s[t][w] = s4[w]; d.sc.z[t][w] = z4[w]; }
            } else if constexpr (SC::NW == 2) {
                const u32x2 s2 = __builtin_amdgcn_raw_buffer_load_b64(sr, (int)soff[t], ss, 0);
                const u32x2 z2 = __builtin_amdgcn_raw_buffer_load_b64(zr, (int)soff[t], ss, 0);
                d.sc.s[t][0] = s2[0]; d.sc.s[t][1] = s2[1]; d.sc.z[t][0] = z2[0]; d.sc.z[t][1] = z2[1];
            } else {
                d.sc.s[t][0] = __builtin_amdgcn_raw_buffer_load_b32(sr, (int)soff[t], ss, 0);
                d.sc.z[t][0] = __builtin_amdgcn_raw_buffer_load_b32(zr, (int)soff[t], ss, 0);
            }
        }
    };
    constexpr int LB = P2_NT * 4;   // vm loads per block (2 code pieces, scales, biases per tile)
    // transposed block: kh[t][h][s] = the word of step s, k half h
    auto transpose = [&](const P2Block<G>& d, u32x4 (&tw)[P2_NT][2]) {
#pragma unroll
        for (int t = 0; t < P2_NT; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                tw[t][h] = d.c[t][h];
                xpose4(tw[t][h]);
            }
    };
    // weight operand of (step s of the block, k half h) for tile t
    auto wfrag = [&](const u32x4 (&tw)[P2_NT][2], const P2Sc<G>& d, int t, int s, int h) -> u32x4 {
        // group of this 32-wide k window within the block, and its bf16
        const int gi = (s * P2_BK + h * 32) / G;
        const float sc = bf16_bits_to_f32((d.s[t][gi >> 1] >> (16 * (gi & 1))) & 0xFFFFu);
        const float zb = bf16_bits_to_f32((d.z[t][gi >> 1] >> (16 * (gi & 1))) & 0xFFFFu);
        return deq8(tw[t][h][s], sc, zb);
    };

    // ---- accumulators (OB: start at the dense layer's bias of each column)
    f32x4 acc[P2_NT][P2_MT];
#pragma unroll
    for (int t = 0; t < P2_NT; ++t) {
        f32x4 b0 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (OB) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int n = n0 + (P2_BN / P2_NWV) * wv + 16 * t + 4 * j + r;
                b0[r] = n < a.N ? out_bias_at(a.ob, n) : 0.f;
            }
        }
#pragma unroll
        for (int m = 0; m < P2_MT; ++m) acc[t][m] = b0;
    }
    if constexpr (OB) __builtin_amdgcn_sched_barrier(0);

    const int nk = (int)(K / P2_BK);           // multiple of 4 (host checks)
    const int nb = nk / P2_SPB;

    // ---- prologue. vm issue order: block 0, DMA 0, 1, 2, block 1 -- the
    // order the loop keeps (a block is loaded right after the DMA that
    // follows the block's last step), so the loop's wait counts hold from
    // step 0 on.
    P2Block<G> raw;
    P2Sc<G> cur;
    u32x4 tw[P2_NT][2];
    load_block(raw, 0);
#pragma unroll
    for (int u = 0; u < 3; ++u) dma(u, u < nk ? u : nk - 1);
    transpose(raw, tw);                        // waits for block 0 (the compiler counts it)
    cur = raw.sc;
    load_block(raw, nb > 1 ? 1 : 0);
    // the DMA of step 0 is in LDS: issued after it are DMA 1, 2 and block 1
    wait_vm<2 * P2_XDMA + LB>();
    __builtin_amdgcn_s_barrier();
    u32x4 xf0[P2_MT], xf1[P2_MT], wf0[P2_NT], wf1[P2_NT];
#pragma unroll
    for (int m = 0; m < P2_MT; ++m) xf0[m] = read_x(0, m, 0);
#pragma unroll
    for (int t = 0; t < P2_NT; ++t) wf0[t] = wfrag(tw, cur, t, 0, 0);

    // ---- main loop: one block (4 steps) per iteration, steps unrolled.
    // vm issue order from here: each step's second half issues the DMA of
    // step kt + 3; the last step of a block then loads block b + 2.
    for (int b = 0; b < nb; ++b) {
#pragma unroll
        for (int s = 0; s < P2_SPB; ++s) {
            const int kt = b * P2_SPB + s;
            const int stage = kt % P2_XST;
            // -- first half: read the k-half-1 fragments, MFMAs of k half 0
#pragma unroll
            for (int m = 0; m < P2_MT; ++m) xf1[m] = read_x(stage, m, 1);
#pragma unroll
            for (int t = 0; t < P2_NT; ++t) wf1[t] = wfrag(tw, cur, t, s, 1);
#pragma unroll
            for (int m = 0; m < P2_MT; ++m)
#pragma unroll
                for (int t = 0; t < P2_NT; ++t) acc[t][m] = mfma_bf16(wf0[t], xf0[m], acc[t][m]);
            // -- every wave's part of step kt+1's activations has landed. Loads
            // issued after DMA(kt+1), which was issued two steps ago: DMA(kt+2),
            // and block b+1 if one of the two previous steps ended a block.
            if (s <= 1) wait_vm<P2_XDMA + LB>();
            else wait_vm<P2_XDMA>();
            __builtin_amdgcn_s_barrier();
            // -- second half: next step's first fragments, the DMA three steps
            // ahead (into the stage last read two steps ago), MFMAs of k half 1
            const bool more = kt + 1 < nk;
            if (more) {
#pragma unroll
                for (int m = 0; m < P2_MT; ++m) xf0[m] = read_x((kt + 1) % P2_XST, m, 0);
            }
            dma((kt + 3) % P2_XST, kt + 3 < nk ? kt + 3 : nk - 1);
            if (s == P2_SPB - 1) {
                // block b+1 -> transposed words; its registers take block b+2
                transpose(raw, tw);
                cur = raw.sc;
                load_block(raw, b + 2 < nb ? b + 2 : nb - 1);
            }
            if (more) {
#pragma unroll
                for (int t = 0; t < P2_NT; ++t) wf0[t] = wfrag(tw, cur, t, (s + 1) % P2_SPB, 0);
            }
#pragma unroll
            for (int m = 0; m < P2_MT; ++m)
#pragma unroll
                for (int t = 0; t < P2_NT; ++t) acc[t][m] = mfma_bf16(wf1[t], xf1[m], acc[t][m]);
        }
    }

    // ---- epilogue: lane (i, j) holds D[n = 4j + r][m = i] of tile (t, m)
#pragma unroll
    for (int m = 0; m < P2_MT; ++m) {
        const int row = m0 + 16 * m + i;
        if (row >= a.M) continue;
        uint16_t* yr = a.y + (size_t)row * a.N;
#pragma unroll
        for (int t = 0; t < P2_NT; ++t) {
            const int n = n0 + (P2_BN / P2_NWV) * wv + 16 * t + 4 * j;
            const f32x4 v = acc[t][m];
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

template <auto KERN>
hipError_t launch_p2(const P2Args& t, int grid, hipStream_t st) {
    const size_t shm = (size_t)P2_XST * P2_XSTAGE;
    static std::atomic<bool> attr_set{false};
    if (!attr_set.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)shm);
        if (e != hipSuccess) return e;
        attr_set.store(true, std::memory_order_release);
    }
    KERN<<<grid, P2_THREADS, shm, st>>>(t);
    return hipGetLastError();
}

inline int p2_xcd_grid(int64_t ntm, int64_t ntn, double w_bytes, double x_bytes, int xcds) {
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

template <int G>
hipError_t launch_p2_g(const QmmArgs& q, hipStream_t st) {
    P2Args t{};
    t.x = (const uint16_t*)q.x;
    t.wq = q.wq;
    t.scales = (const uint16_t*)q.scales;
    t.biases = (const uint16_t*)q.biases;
    t.y = (uint16_t*)q.y;
    t.M = (int)q.M;
    t.N = (int)q.N;
    t.K = (int)q.K;
    t.ob = q.ob;
    t.lds_nan = debug_lds_nan();
    const int64_t ntm = (q.M + P2_BM - 1) / P2_BM, ntn = (q.N + P2_BN - 1) / P2_BN;
    t.xcds = device_shape().xcds;
    t.xgm = p2_xcd_grid(ntm, ntn, (double)q.N * q.K / 2.0, (double)q.M * q.K * 2.0, t.xcds);
    const int grid = (int)(ntm * ntn);
    if (q.ob.kind != OB_NONE) return launch_p2<qmm_prefill2_kernel<G, true>>(t, grid, st);
    return launch_p2<qmm_prefill2_kernel<G, false>>(t, grid, st);
}

}  // namespace

bool qmm_prefill2_supports(const QmmArgs& q) {
    if (!q.transpose || q.x_dtype != QLIN_BF16 || q.R != 0) return false;
    if (q.mode != AFFINE || q.bits != 4 || q.scale_dtype != QLIN_BF16) return false;
    if (q.K % (P2_SPB * P2_BK) != 0 || q.M < 1) return false;
    if (((uintptr_t)q.wq & 15) != 0 || ((uintptr_t)q.x & 15) != 0) return false;
    if (((uintptr_t)q.scales & 15) != 0 || ((uintptr_t)q.biases & 15) != 0) return false;
    if (q.M * q.K * 2 >= (1LL << 31) || q.N * q.K / 2 >= (1LL << 31)) return false;
    return true;
}

hipError_t launch_qmm_prefill2(const QmmArgs& q, hipStream_t st) {
    if (!qmm_prefill2_supports(q)) return hipErrorNotSupported;
    if (q.group_size == 32) return launch_p2_g<32>(q, st);
    if (q.group_size == 64) return launch_p2_g<64>(q, st);
    return launch_p2_g<128>(q, st);
}

}  // namespace qlin
