// qqmm_mx8.hip -- both-quantized matmul in mxfp8 on the CDNA4 scaled MFMA
// (gfx950: v_mfma_scale_f32_32x32x64_f8f6f4).
//
// mlx-rs "ops/quantization.rs", qqmm: x is quantized on the fly with the
// weight's mode and the product is taken between the two quantized
// operands. In mxfp8 ("Emily.QuantizedWeight", Microscaled modes table:
// group 32, E4M3 codes, one E8M0 scale byte per group) both operands are
// exactly the scaled MFMA's input format: E4M3 codes with a power-of-two
// scale per 32 values along K. The instruction multiplies the codes exactly,
// scales each 32-wide block by 2^(ex + ew) and accumulates in fp32, so
// y = sum over blocks 2^(ex+ew) * sum codes_x * codes_w is the oracle's
// dequant(x) . dequant(W)^T up to accumulation order, at the fp8 rate.
//
// Workgroup: 4 waves as 2 x 2, tile 128 weight rows (n) x 128 activation
// rows (m), each wave 64 x 64 (2 x 2 tiles of 32 x 32), K in steps of 128
// codes:
//  * Both code tiles go global -> LDS by buffer->LDS loads, XLA steps ahead
//    into XST-stage rings. One wave instruction moves 8 whole rows of a step
//    (8 x 128 bytes), so every request is a full 128-byte line; row r keeps
//    its 16-byte chunk c in slot c ^ (r & 7) ^ ((r >> 3) & 1), which gives the
//    16 rows one fragment read covers 16 distinct slots.
//  * Scale bytes (one per row and 32-wide block) go global -> LDS too, 16
//    bytes (four steps) per row and batch, one batch ahead, so no register
//    ever waits on a load the compiler cannot date.
//  * Per step a wave runs 2 (k halves) x 2 x 2 tiles of scaled MFMAs.
//  * Operand layout of the instruction for 8-bit codes (checked on the
//    device with a one-wave probe against a host model): lane (i, j) holds
//    32 codes of row (column) i, its first 16 from the first 32-wide scale
//    block of the 64 and its last 16 from the second: here k offsets
//    [16j, 16j + 16) and [32 + 16j, 32 + 16j + 16). The scale byte of block b
//    of row i is the one lane (i, b) supplies (byte op_sel of its register);
//    D[row][col] sits in lane col + 32 (row/4 % 2), register 4 (row/8) + row % 4.
// Rows past N or M read zeros (buffer range checks) and are never stored.

#include "qlin_common.h"

#include <atomic>

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int MX_BK = 128;             // k (bytes) per step
constexpr int MX_BN = 128;             // weight rows per workgroup
constexpr int MX_BM = 128;             // activation rows per workgroup
constexpr int MX_THREADS = 256;
constexpr int MX_XST = 4;              // LDS stages per operand
constexpr int MX_XLA = 3;              // steps in flight
constexpr int MX_SG = 4;               // steps per scale batch (16 scale bytes)
constexpr int MX_STAGE = 128 * MX_BK;  // 16 KiB per operand and stage

struct Mx8Args {
    const uint8_t* xq;    // E4M3 [M, K]
    const uint8_t* xs;    // E8M0 [M, K/32]
    const uint8_t* wq;    // E4M3 [N, K]
    const uint8_t* ws;    // E8M0 [N, K/32]
    uint16_t* y;          // bf16 [M, N]
    int M, N, K;
    int xcds;             // XCDs of the device (block renumbering)
    int lds_nan;          // debug: fill LDS with NaN before the tile
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    bf16x2 r = {(__bf16)lo, (__bf16)hi};   // nearest-even
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt unconstrained). Field
// layout: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__global__ void __launch_bounds__(MX_THREADS) qqmm_mx8_kernel(Mx8Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* const wlds = smem;                          // W stages
    unsigned char* const xlds = smem + MX_XST * MX_STAGE;      // x stages
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wv >> 1, wm = wv & 1;
    const int i = lane & 31, j = lane >> 5;          // MFMA lane: row/col i, k piece j
    const uint32_t K = (uint32_t)a.K;
    const uint32_t KS = K / 32;                      // scale bytes per row

    // tile of this workgroup: workgroups are dealt to the XCDs round-robin;
    // renumber so each XCD walks a contiguous run of tiles, m fastest, and
    // the activation tiles sharing one weight tile meet in one L2
    const int ntm = (a.M + MX_BM - 1) / MX_BM;
    const int b = xcd_block(blockIdx.x, gridDim.x, a.xcds);
    if (a.lds_nan) {   // debug: every LDS byte of the tile starts as NaN
        constexpr int LDS_BYTES = 2 * MX_XST * MX_STAGE + 2 * 4096;
        for (int o = tid * 16; o < LDS_BYTES; o += MX_THREADS * 16)
            *(u32x4*)(smem + o) = u32x4{~0u, ~0u, ~0u, ~0u};
        __syncthreads();
    }
    const int m0 = (b % ntm) * MX_BM, n0 = (b / ntm) * MX_BN;

    const __amdgpu_buffer_rsrc_t xr = rsrc(a.xq, (uint32_t)a.M * K);
    const __amdgpu_buffer_rsrc_t xsr = rsrc(a.xs, (uint32_t)a.M * KS);
    const __amdgpu_buffer_rsrc_t wr = rsrc(a.wq, (uint32_t)a.N * K);
    const __amdgpu_buffer_rsrc_t wsr = rsrc(a.ws, (uint32_t)a.N * KS);

    // ---- DMA: each wave instruction moves 8 rows x 128 bytes of one
    // operand; 16 instructions per stage and operand, 4 per wave each
    constexpr int NDMA = 128 / 8 / 4;
    uint32_t xdoff[NDMA], wdoff[NDMA];
#pragma unroll
    for (int q = 0; q < NDMA; ++q) {
        const int r = (q * 4 + wv) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        xdoff[q] = m0 + r < a.M ? (uint32_t)(m0 + r) * K + (uint32_t)c * 16u : 0x80000000u;
        wdoff[q] = n0 + r < a.N ? (uint32_t)(n0 + r) * K + (uint32_t)c * 16u : 0x80000000u;
    }
    auto dma = [&](int stage, int kt) {
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void*)(wlds + stage * MX_STAGE + (q * 4 + wv) * 1024),
                16, (int)wdoff[q], kt * MX_BK, 0, 0);
#pragma unroll
        for (int q = 0; q < NDMA; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void*)(xlds + stage * MX_STAGE + (q * 4 + wv) * 1024),
                16, (int)xdoff[q], kt * MX_BK, 0, 0);
    };

    // ---- scales through LDS too: one wave instruction per batch of 4 steps
    // moves 16 scale bytes of 64 rows (wave 0/1: weight rows 0-63 / 64-127,
    // wave 2/3: activation rows 0-63 / 64-127) into the batch's stage
    unsigned char* const slds = smem + 2 * MX_XST * MX_STAGE;   // [2][256 rows][16 B]
    uint32_t sdoff;
    {
        const int r = 64 * (wv & 1) + lane;
        if (wv < 2) sdoff = n0 + r < a.N ? (uint32_t)(n0 + r) * KS : 0x80000000u;
        else sdoff = m0 + r < a.M ? (uint32_t)(m0 + r) * KS : 0x80000000u;
    }
    auto dma_scales = [&](int sstage, int g) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wv < 2 ? wsr : xsr, (__attribute__((address_space(3))) void*)(slds + sstage * 4096 + wv * 1024),
            16, (int)sdoff, g * 16, 0, 0);
    };
    // this lane's scale rows in a stage: weight tile rows then activation rows
    uint32_t srow[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        srow[t] = (uint32_t)(64 * wn + 32 * t + i) * 16u;
        srow[2 + t] = (uint32_t)(128 + 64 * wm + 32 * t + i) * 16u;
    }

    const int nk = (int)(K / MX_BK);
    const int ng = (nk + MX_SG - 1) / MX_SG;
    f32x16 acc[2][2];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tn][tm][r] = 0.f;

    // vm operations in issue order: prologue: scales of batch 0 (1), DMA of
    // steps 0 .. XLA-1 (2 * NDMA = 8 each); each step: DMA of step kt + XLA
    // (8), then at a batch's first step the next batch's scales (1)
    static_assert(NDMA == 4 && MX_XLA == 3 && MX_SG == 4 && MX_XST == 4, "wait counts assume these");
    dma_scales(0, 0);
#pragma unroll
    for (int u = 0; u < MX_XLA; ++u) dma(u, u < nk ? u : nk - 1);

    for (int g0 = 0; g0 < ng; g0 += 2) {
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
            const int g = g0 + gg;
#pragma unroll
            for (int u = 0; u < MX_SG; ++u) {
                const int kt = g * MX_SG + u;
                // Step kt needs its DMA, issued XLA steps ago (the prologue's
                // for kt < XLA), and its batch of scales, issued before that
                // DMA. Loads issued after DMA(kt): the DMAs of steps kt-2 and
                // kt-1 (16) and one scale load if one of steps kt-3 .. kt-1
                // opened a batch, which happens unless kt opens one (u == 0);
                // at kt = 0: DMA(1), DMA(2).
                if (u != 0) wait_vm<2 * 2 * NDMA + 1>();
                else wait_vm<2 * 2 * NDMA>();
                __builtin_amdgcn_s_barrier();
                if (kt < nk) {
                    const int stage = kt % MX_XST;
                    const unsigned char* wt = wlds + stage * MX_STAGE;
                    const unsigned char* xt = xlds + stage * MX_STAGE;
                    const unsigned char* st = slds + (gg & 1) * 4096;
                    // fragments of this step: tile t, k half h, pieces at
                    // chunks 4h + j and 4h + 2 + j
                    u32x4 af[2][2][2], bf[2][2][2];
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const int ra = 64 * wn + 32 * t + i, rb = 64 * wm + 32 * t + i;
                            const int c0 = 4 * h + j;
                            af[h][t][0] = *(const u32x4*)(wt + ra * MX_BK + ((c0 ^ swz(ra)) << 4));
                            af[h][t][1] = *(const u32x4*)(wt + ra * MX_BK + (((c0 + 2) ^ swz(ra)) << 4));
                            bf[h][t][0] = *(const u32x4*)(xt + rb * MX_BK + ((c0 ^ swz(rb)) << 4));
                            bf[h][t][1] = *(const u32x4*)(xt + rb * MX_BK + (((c0 + 2) ^ swz(rb)) << 4));
                        }
                    // scale dword u of each of the lane's 4 rows; lane j takes
                    // blocks 2h + j -> shift by 8j, op_sel 2h
                    uint32_t sw[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) sw[q] = *(const uint32_t*)(st + srow[q] + 4 * u) >> (8 * j);
                    // next DMA (into the stage read XST - XLA = 1 step ago,
                    // whose reads every wave finished before the barrier);
                    // at a batch's first step also the next batch's scales
                    // (into the stage the previous batch used)
                    const int kx = kt + MX_XLA < nk ? kt + MX_XLA : nk - 1;
                    dma((kt + MX_XLA) % MX_XST, kx);
                    if (u == 0) dma_scales((gg + 1) & 1, g + 1 < ng ? g + 1 : ng - 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int tn = 0; tn < 2; ++tn) {
                            i32x8 A;
                            A[0] = af[h][tn][0][0]; A[1] = af[h][tn][0][1]; A[2] = af[h][tn][0][2]; A[3] = af[h][tn][0][3];
                            A[4] = af[h][tn][1][0]; A[5] = af[h][tn][1][1]; A[6] = af[h][tn][1][2]; A[7] = af[h][tn][1][3];
#pragma unroll
                            for (int tm = 0; tm < 2; ++tm) {
                                i32x8 B;
                                B[0] = bf[h][tm][0][0]; B[1] = bf[h][tm][0][1]; B[2] = bf[h][tm][0][2]; B[3] = bf[h][tm][0][3];
                                B[4] = bf[h][tm][1][0]; B[5] = bf[h][tm][1][1]; B[6] = bf[h][tm][1][2]; B[7] = bf[h][tm][1][3];
                                if (h == 0)
                                    acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                        A, B, acc[tn][tm], 0, 0, 0, (int)sw[tn], 0, (int)sw[2 + tm]);
                                else
                                    acc[tn][tm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                        A, B, acc[tn][tm], 0, 0, 2, (int)sw[tn], 2, (int)sw[2 + tm]);
                            }
                        }
                }
            }
        }
    }

    // ---- epilogue: acc[tn][tm][r] = D[n row][m col]: m = m0 + 64 wm + 32 tm +
    // lane%32, n = n0 + 64 wn + 32 tn + 8 (r/4) + 4 (lane/32) + r%4
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
        const int m = m0 + 64 * wm + 32 * tm + i;
        if (m >= a.M) continue;
        uint16_t* yr = a.y + (size_t)m * a.N;
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nn = n0 + 64 * wn + 32 * tn + 8 * q + 4 * j;
                const f32x16& v = acc[tn][tm];
                if (nn + 3 < a.N && (a.N & 3) == 0) {
                    uint2 pk;
                    pk.x = pack2(v[4 * q], v[4 * q + 1]);
                    pk.y = pack2(v[4 * q + 2], v[4 * q + 3]);
                    *(uint2*)(yr + nn) = pk;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (nn + r < a.N) yr[nn + r] = (uint16_t)f32_to_bf16_rne(v[4 * q + r]);
                }
            }
    }
}

}  // namespace

bool qqmm_mx8_supports(int64_t M, int64_t N, int64_t K, const void* wq, const void* ws) {
    // K % 512: whole batches of 4 steps and 16-byte aligned scale rows
    if (M < 1 || N < 1 || K < 512 || K % 512 != 0) return false;
    if (M * K >= (1LL << 31) || N * K >= (1LL << 31)) return false;
    if (((uintptr_t)wq & 15) != 0 || ((uintptr_t)ws & 3) != 0) return false;
    return true;
}

hipError_t launch_qqmm_mx8(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                           uint16_t* y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    if (!qqmm_mx8_supports(M, N, K, wq, ws)) return hipErrorNotSupported;
    Mx8Args a{xq, xs, wq, ws, y, (int)M, (int)N, (int)K, device_shape().xcds, debug_lds_nan() ? 1 : 0};
    const int64_t tiles = ((M + MX_BM - 1) / MX_BM) * ((N + MX_BN - 1) / MX_BN);
    const size_t shm = (size_t)2 * MX_XST * MX_STAGE + 2 * 4096;
    static std::atomic<bool> attr{false};
    if (!attr.load(std::memory_order_acquire)) {
        hipError_t e = hipFuncSetAttribute((const void*)qqmm_mx8_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
        attr.store(true, std::memory_order_release);
    }
    qqmm_mx8_kernel<<<(unsigned)tiles, MX_THREADS, shm, st>>>(a);
    return hipGetLastError();
}

}  // namespace qlin
