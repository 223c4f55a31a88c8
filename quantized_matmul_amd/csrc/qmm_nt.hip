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
//   * codes become fp32 and accumulate with one FMA each (fp32 throughout;
//     E2M1 / E4M3 codes by the gfx950 converts, two per instruction);
//   * a wave load covers 8 rows x 8 packed words (one activation row of
//     microscaled or 2-bit codes: 32 or 16 rows, each lane a 16- or 8-byte
//     piece of one group), so a workgroup spans few columns and the grid has
//     enough workgroups; its 16 waves split K and meet once in LDS; the
//     weight words stream through a prefetch ring;
//   * x for all of K is staged in LDS up front; each row's scale and bias
//     ride in the prefetch ring with its packed word (staging them up front
//     serialised thousands of scattered 2-byte loads before the weight
//     stream started: 27 -> 25 us at M1, 63 -> 53 us at M8).

#include "qlin_common.h"

namespace qlin {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

struct NtArgs {
    const uint16_t* x;   // bf16 [M, K]
    const uint32_t* wq;  // [K, N/PER]
    const void* scales;  // [K, N/G] bf16 or u8
    const uint16_t* biases;
    uint16_t* y;         // bf16 [M, N]
    int M, N, K;
    int xcds;            // XCDs of the device (block renumbering)
    OutBias ob;          // dense-layer bias
};

// The PER codes of packed word w as floats, code 0 (the low bits) first.
// Affine: the integer code; microscaled: the element value at unit scale
// (E2M1 / E4M3 by the gfx950 converts, two codes per instruction).
template <int MODE, int BITS>
__device__ __forceinline__ void decode_word(uint32_t w, float (&f)[32 / BITS]) {
    if constexpr (MODE == AFFINE && BITS == 4) {
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = (float)((lo >> (8 * q)) & 0xFFu);
            f[2 * q + 1] = (float)((hi >> (8 * q)) & 0xFFu);
        }
    } else if constexpr (MODE == AFFINE && BITS == 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) f[q] = (float)((w >> (8 * q)) & 0xFFu);
    } else if constexpr (MODE == AFFINE) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t mm = (w >> (2 * t)) & 0x03030303u;
#pragma unroll
            for (int q = 0; q < 4; ++q) f[4 * q + t] = (float)((mm >> (8 * q)) & 0xFFu);
        }
    } else if constexpr (MODE == MXFP8) {
        const auto lo2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
        const auto hi2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
        f[0] = lo2[0]; f[1] = lo2[1]; f[2] = hi2[0]; f[3] = hi2[1];
    } else {
        // byte q holds codes 2q (low nibble) and 2q + 1
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        f[0] = p0[0]; f[1] = p0[1]; f[2] = p1[0]; f[3] = p1[1];
        f[4] = p2[0]; f[5] = p2[1]; f[6] = p3[0]; f[7] = p3[1];
    }
}

// Lane (rr, cl) = (lane / LPR, lane % LPR) handles the VW packed words
// c0 + VW*cl .. c0 + VW*cl + VW-1 of row k = RPS * step + rr: one wave load
// covers RPS = 64 / LPR rows x WPB words (LPR = WPB / VW lanes per row). The
// VW words of a lane lie in one quantization group. The NW waves of a
// workgroup split K. Each lane keeps RING2 steps (words, scale, bias) in
// flight. MR = activation rows rounded up (<= 8).
template <int MODE, int BITS, int G, int MR, int WPB, int NW, int VW>
__global__ void __launch_bounds__(64 * NW) qmm_nt_kernel(NtArgs a) {
    constexpr int PER = 32 / BITS;
    static_assert(VW == 1 || VW == 2 || VW == 4, "words per lane");
    static_assert((G / PER) % VW == 0 && WPB % VW == 0, "a lane's words share one group");
    // steps in flight per lane (microscaled decoding needs more registers):
    // the kernel is bound by the bytes each lane keeps in flight. With one
    // word per lane, one activation row of 4- or 8-bit affine codes takes 32
    // (126 registers, no spills; 25 -> 22.8 us at M1), two rows 16. With
    // 16-byte lanes a step already carries four words.
    constexpr int RING2 = VW > 1 ? 8
                        : (MR == 1 && MODE == AFFINE && BITS >= 4) ? 32
                        : (MR <= 2 && MODE == AFFINE) ? 16 : (MR <= 4 ? 8 : 4);
    constexpr int NWAVES = NW;
    constexpr int LPR = WPB / VW;                     // lanes per row
    constexpr int RPS = 64 / LPR;                     // rows per step
    constexpr int CPL = VW * PER;                     // columns per lane
    constexpr bool AFF = MODE == AFFINE;
    constexpr int SBYTES = AFF ? 2 : 1;               // bytes per scale value
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rr = lane / LPR, cl = lane % LPR;
    const int K = a.K, N = a.N;
    const int wcols = N / PER;                        // packed words per W row
    // Workgroups are dealt to the XCDs round-robin. Neighbouring column
    // blocks share 128-byte lines of every weight row (a block uses WPB words
    // of a row), so renumber the blocks: each XCD walks a contiguous run of
    // them and the shared lines meet in that XCD's L2 instead of being
    // fetched once per XCD.
    const int cb = xcd_block(blockIdx.x, gridDim.x, a.xcds);
    const int c = cb * WPB + cl * VW;                 // first word column of the lane
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

    float acc[MR][CPL], zacc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        zacc[m] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[m][e] = 0.f;
    }

    const uint32_t* wp = a.wq + (active ? c : 0);
    uint32_t rw[RING2][VW], rs[RING2], rz[RING2];
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
        const uint32_t* src = wp + (size_t)kk * wcols;
        if constexpr (VW == 4) {
            const u32x4 v = *(const u32x4*)src;
            rw[slot][0] = v.x; rw[slot][1] = v.y; rw[slot][2] = v.z; rw[slot][3] = v.w;
        } else if constexpr (VW == 2) {
            const u32x2 v = *(const u32x2*)src;
            rw[slot][0] = v.x; rw[slot][1] = v.y;
        } else {
            rw[slot][0] = *src;
        }
        const uint32_t so = ((uint32_t)kk * (uint32_t)gpr + gcol) * (uint32_t)SBYTES;
        if constexpr (AFF) {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0);
            rz[slot] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0);
        } else {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b8(srs, (int)so, 0, 0);
        }
    };
    auto consume = [&](int slot, int st) {
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
        float av[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float xv = bf16_bits_to_f32(xs[m * K + k]);
            av[m] = xv * s;
            if constexpr (AFF) zacc[m] = __builtin_fmaf(xv, z, zacc[m]);
        }
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            const uint32_t w = rw[slot][j];
            float f[PER];
            decode_word<MODE, BITS>(w, f);
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    acc[m][j * PER + e] = __builtin_fmaf(av[m], f[e], acc[m][j * PER + e]);
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
        for (int e = 0; e < CPL; ++e) {
            float v = acc[m][e] + zacc[m];
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
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
            for (int e = 0; e < CPL; ++e) red[(wv * WPB + cl * VW) * PER + e] = acc[m][e];
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

constexpr int kNtWpb = 8;    // packed words of a weight row per workgroup
constexpr int kNtNw = 16;    // waves per workgroup (up to 4 activation rows)

// waves per workgroup: 16 for up to 4 activation rows, 8 for more (the
// register ring then holds more accumulators per lane)
inline int nt_waves(int M) { return nt_mr(M) == 8 ? 8 : kNtNw; }

inline size_t nt_shm(int M, int K, int per) {
    const int wpb = kNtWpb;
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
    a.xcds = device_shape().xcds;
    constexpr int PER = 32 / BITS;
    const int wcols = a.N / PER;
    constexpr int WPB = kNtWpb, NW = kNtNw;
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
    // One activation row of microscaled or 2-bit codes: each lane loads VW
    // words (16 or 8 bytes, one group) per row. Measured at M1, N 14336 /
    // 8192, K 4096 / 8192: mxfp4 35.8 -> 35.2 us, nvfp4 40.5 -> 36.9 us, mxfp8
    // 38.0 -> 34.4 us, int2 g32 26.2 -> 24.5 us; 4- and 8-bit affine codes and
    // two or more rows ran slower that way (int4 M1 22.7 -> 25.2 us, M2 27.0
    // -> 31.3 us) and keep one word per lane.
    // (at most 32 columns per lane: 2-bit codes take two words)
    constexpr int VCAP = BITS < 4 ? BITS : 4;
    constexpr int VWIDE = (G / PER) < VCAP ? (G / PER) : VCAP;
    constexpr bool WIDE_FMT = VWIDE > 1 && (MODE != AFFINE || BITS == 2);
    if constexpr (WIDE_FMT) {
        const bool wide = a.M == 1 &&
                          ((uintptr_t)a.wq % (4 * VWIDE)) == 0 && (wcols % VWIDE) == 0;
        if (wide) return run(qmm_nt_kernel<MODE, BITS, G, 1, WPB, NW, VWIDE>, NW);
    }
    switch (nt_mr(a.M)) {
    case 1: return run(qmm_nt_kernel<MODE, BITS, G, 1, WPB, NW, 1>, NW);
    case 2: return run(qmm_nt_kernel<MODE, BITS, G, 2, WPB, NW, 1>, NW);
    case 4: return run(qmm_nt_kernel<MODE, BITS, G, 4, WPB, NW, 1>, NW);
    default: return run(qmm_nt_kernel<MODE, BITS, G, 8, WPB, 8, 1>, 8);
    }
}

// ---------------------------------------------------------------- K-split
// With a caller's workspace the rows of K are also split over workgroups:
// workgroup (superblock, slice) covers SBW packed words of every weight row
// (256 bytes: two whole cache lines, and one line of scales and of biases)
// for the rows of its K slice, and stores its fp32 partial sums. At one or
// two activation rows the slice that finishes last for a superblock adds
// the slices in order and writes y in the same launch (a separate summing
// kernel cost about 2 us of a 16.8 us call); at three or four rows a second
// kernel adds them. Each workgroup asks the L2 for a few hundred rows
// instead of all K, four requests per 256 bytes instead of three per 32.
constexpr int SPLIT_SBW = 64;   // packed words per superblock row
// The workspace starts with one completion counter per superblock (the
// caller zeroes them once; every call leaves them zero), then the partial
// sums [S][M][N] in fp32.
constexpr size_t kSplitCounterBytes = 4096;
// waves per workgroup (16 for one or two activation rows measured slower:
// 15.0 against 14.5 us at one row)
__host__ __device__ constexpr int split_nw(int) { return 8; }
// the last slice adds the slices in the same kernel at one or two rows
__host__ __device__ constexpr bool split_fuse(int mr) { return mr <= 2; }

template <int MODE, int BITS, int G, int MR, int VW>
__global__ void __launch_bounds__(64 * split_nw(MR)) qmm_nt_split_kernel(NtArgs a, float* part, uint32_t* cnt,
                                                                     int ks, int S, int nsb,
                                                                     int nreal) {
    constexpr int PER = 32 / BITS;
    constexpr int SBW = SPLIT_SBW, NWAVES = split_nw(MR);
    constexpr bool FUSE = split_fuse(MR);
    static_assert((G / PER) % VW == 0, "a lane's words share one group");
    constexpr int LPR = SBW / VW;        // lanes per row
    constexpr int RPS = 64 / LPR;        // rows per wave load
    constexpr int CPL = VW * PER;        // columns per lane
    constexpr int RING = 8;   // wave loads in flight per lane
    constexpr bool AFF = MODE == AFFINE;
    constexpr int SBYTES = AFF ? 2 : 1;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int rr = lane / LPR, cl = lane % LPR;
    const int K = a.K, N = a.N, M = a.M;
    const int wcols = N / PER, gpr = N / G;
    // Workgroups are dealt to the XCDs round-robin. A 128-byte line of a
    // row's scales (and biases) covers 64 groups, i.e. several neighbouring
    // superblocks, so renumber the blocks XCD-major: each XCD walks a
    // contiguous run of (slice, superblock) pairs and fetches each scale line
    // once instead of once per XCD. The grid is padded to a multiple of the
    // XCD count; the padding blocks leave at once.
    const int L = xcd_block(blockIdx.x, gridDim.x, a.xcds);
    if (L >= nreal) return;
    const int sb = L % nsb, sl = L / nsb;
    const int k0 = sl * ks;
    const int kn = (K - k0) < ks ? (K - k0) : ks;      // rows of this slice (>= 1)
    const int c = sb * SBW + cl * VW;                  // first word column of the lane
    const bool active = c < wcols;
    const uint32_t gcol = active ? (uint32_t)((c * PER) / G) : 0u;

    // x of the slice in LDS: [MR][ks] bf16, zero past M and past the slice
    uint16_t* xs = (uint16_t*)smem;
    for (int idx = tid; idx < MR * ks; idx += 64 * NWAVES) {
        const int m = idx / ks, kk = idx - m * ks;
        xs[idx] = (m < M && kk < kn) ? a.x[(size_t)m * K + k0 + kk] : (uint16_t)0;
    }
    __syncthreads();

    // wave load t of wave wv covers rows k0 + RPS * (wv + NWAVES * t) + rr
    const int steps = (kn + RPS * NWAVES - 1) / (RPS * NWAVES);
    const int T = (steps + RING - 1) / RING * RING;
    float acc[MR][CPL], zacc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        zacc[m] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) acc[m][e] = 0.f;
    }
    const uint32_t* wp = a.wq + (active ? c : 0);
    const uint32_t sbytes_all = (uint32_t)K * (uint32_t)gpr * SBYTES;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.scales), (short)0, (int)sbytes_all, 0x00020000);
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(AFF ? a.biases : (const uint16_t*)a.scales), (short)0,
        (int)(AFF ? sbytes_all : 0u), 0x00020000);
    uint32_t rw[RING][VW], rs[RING], rz[RING];
    auto row_of = [&](int t) { return RPS * (wv + NWAVES * t) + rr; };   // within the slice
    auto fetch = [&](int slot, int t) {
        const int kr = row_of(t);
        const int k = k0 + ((active && kr < kn) ? kr : 0);
        const uint32_t* src = wp + (size_t)k * wcols;
        if constexpr (VW == 4) {
            const u32x4 v = *(const u32x4*)src;
            rw[slot][0] = v.x; rw[slot][1] = v.y; rw[slot][2] = v.z; rw[slot][3] = v.w;
        } else if constexpr (VW == 2) {
            const u32x2 v = *(const u32x2*)src;
            rw[slot][0] = v.x; rw[slot][1] = v.y;
        } else {
            rw[slot][0] = *src;
        }
        const uint32_t so = ((uint32_t)k * (uint32_t)gpr + gcol) * (uint32_t)SBYTES;
        if constexpr (AFF) {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, (int)so, 0, 0);
            rz[slot] = __builtin_amdgcn_raw_buffer_load_b16(zrs, (int)so, 0, 0);
        } else {
            rs[slot] = __builtin_amdgcn_raw_buffer_load_b8(srs, (int)so, 0, 0);
        }
    };
    auto consume = [&](int slot, int t) {
        const int kr = row_of(t);
        const bool ok = active && kr < kn;
        const int kk = ok ? kr : 0;
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
        float av[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float xv = bf16_bits_to_f32(xs[m * ks + kk]);
            av[m] = xv * s;
            if constexpr (AFF) zacc[m] = __builtin_fmaf(xv, z, zacc[m]);
        }
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            float f[PER];
            decode_word<MODE, BITS>(rw[slot][j], f);
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    acc[m][j * PER + e] = __builtin_fmaf(av[m], f[e], acc[m][j * PER + e]);
        }
    };
    // 4-bit affine codes, two rows k0, k1 of a lane at a time: each column's
    // pair of codes becomes the exact bf16 pair (128 + q0, 128 + q1) by byte
    // permutes, and one v_dot2_f32_bf16 per column and activation row adds
    // a0 * (128 + q0) + a1 * (128 + q1) with a = x * s rounded to bf16; the
    // offset comes back out through the per-row term, which uses the same
    // rounded a: zacc += x0 z0 + x1 z1 - 128 (a0 + a1).
    auto consume2 = [&](int slot, int t) {
        float av[2][MR];
        uint32_t ab[MR];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kr = row_of(t + h);
            const bool ok = active && kr < kn;
            const int kk = ok ? kr : 0;
            const float s = ok ? bf16_bits_to_f32(rs[slot + h] & 0xFFFFu) : 0.f;
            const float z = ok ? bf16_bits_to_f32(rz[slot + h] & 0xFFFFu) : 0.f;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float xv = bf16_bits_to_f32(xs[m * ks + kk]);
                av[h][m] = xv * s;
                zacc[m] = __builtin_fmaf(xv, z, zacc[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const bf16x2 p = {(__bf16)av[0][m], (__bf16)av[1][m]};
            ab[m] = __builtin_bit_cast(uint32_t, p);
            zacc[m] = __builtin_fmaf(-128.f, __uint_as_float(ab[m] << 16), zacc[m]);
            zacc[m] = __builtin_fmaf(-128.f, __uint_as_float(ab[m] & 0xFFFF0000u), zacc[m]);
        }
        const uint32_t C = 0x43434343u;
#pragma unroll
        for (int j = 0; j < VW; ++j) {
            const uint32_t w0 = rw[slot][j], w1 = rw[slot + 1][j];
            // nibble bytes: lo = codes 0, 2, 4, 6 and hi = codes 1, 3, 5, 7
            const uint32_t lo[2] = {w0 & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu};
            const uint32_t hi[2] = {(w0 >> 4) & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const uint32_t l0 = par ? hi[0] : lo[0], l1 = par ? hi[1] : lo[1];
                // bytes (row 0, row 1) of code bytes 0, 1 and of 2, 3
                const uint32_t t01 = __builtin_amdgcn_perm(l1, l0, 0x05010400u);
                const uint32_t t23 = __builtin_amdgcn_perm(l1, l0, 0x07030602u);
                const uint32_t pr[4] = {__builtin_amdgcn_perm(C, t01, 0x04010400u),
                                        __builtin_amdgcn_perm(C, t01, 0x04030402u),
                                        __builtin_amdgcn_perm(C, t23, 0x04010400u),
                                        __builtin_amdgcn_perm(C, t23, 0x04030402u)};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = j * PER + 2 * q + par;
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        acc[m][col] = __builtin_amdgcn_fdot2_f32_bf16(
                            __builtin_bit_cast(bf16x2, ab[m]), __builtin_bit_cast(bf16x2, pr[q]),
                            acc[m][col], false);
                }
            }
        }
    };
    // (four rows keep the fp32 form: measured 23.2 against 23.9 us)
    constexpr bool DOT2 = AFF && BITS == 4 && MR <= 2;
#pragma unroll
    for (int r = 0; r < RING; ++r) fetch(r, r);
    for (int b = 0; b < T - RING; b += RING) {
        if constexpr (DOT2) {
#pragma unroll
            for (int r = 0; r < RING; r += 2) {
                consume2(r, b + r);
                fetch(r, b + r + RING);
                fetch(r + 1, b + r + 1 + RING);
            }
        } else {
#pragma unroll
            for (int r = 0; r < RING; ++r) {
                consume(r, b + r);
                fetch(r, b + r + RING);
            }
        }
    }
    if constexpr (DOT2) {
#pragma unroll
        for (int r = 0; r < RING; r += 2) consume2(r, T - RING + r);
    } else {
#pragma unroll
        for (int r = 0; r < RING; ++r) consume(r, T - RING + r);
    }

    // sum the RPS row-lanes of each column, then the waves in LDS, and store
    // the slice's partial sums part[sl][m][n]
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float v = acc[m][e] + zacc[m];
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            acc[m][e] = v;
        }
    __syncthreads();
    float* red = (float*)smem;  // [NWAVES][SBW * PER]
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        if (m >= M) break;
        if (rr == 0) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) red[wv * SBW * PER + cl * CPL + e] = acc[m][e];
        }
        __syncthreads();
        for (int o = tid; o < SBW * PER; o += 64 * NWAVES) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NWAVES; ++w) v += red[w * SBW * PER + o];
            const int n = sb * SBW * PER + o;
            if (n < N) {
                if constexpr (FUSE)
                    __hip_atomic_store(part + ((size_t)sl * M + m) * N + n, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                else
                    part[((size_t)sl * M + m) * N + n] = v;
            }
        }
        __syncthreads();
    }

    // Completion: the slice that finishes last for this superblock adds the
    // S slices' partial sums in slice order (the result does not depend on
    // which slice that is), adds the dense bias, rounds once to bf16 and
    // writes y, then puts the superblock's counter back to zero for the next
    // call. The partial sums are written and read as agent-scope atomics,
    // which are coherent across the XCDs' L2s without writing back or
    // invalidating whole caches (an agent-scope fence per workgroup does
    // that, and cost 45 us); every store has completed (the barrier waits
    // for its vector memory counter) before one lane counts the slice in.
    if constexpr (!FUSE) return;   // qmm_nt_split_reduce adds the slices
    __shared__ int is_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // A count of S or more can only come from counters that were not zero
    // when the call began (a workspace the caller did not zero): the slice
    // takes its count back out and fills its columns of y with NaN, so such
    // a call fails visibly, and so does every later call on that workspace.
    if (tid == 0) {
        const uint32_t old =
            __hip_atomic_fetch_add(&cnt[sb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = old == (uint32_t)(S - 1) ? 1 : (old >= (uint32_t)S ? -1 : 0);
        if (is_last < 0) __hip_atomic_fetch_sub(&cnt[sb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (is_last < 0) {
        for (int o = tid; o < M * SBW * PER; o += 64 * NWAVES) {
            const int m = o / (SBW * PER), n = sb * SBW * PER + o % (SBW * PER);
            if (n < N) a.y[(size_t)m * N + n] = (uint16_t)0x7FC0u;   // bf16 quiet NaN
        }
        return;
    }
    if (!is_last) return;
    // each thread takes one column at a time and has the loads of up to 16
    // slices of every activation row in flight at once
    const size_t stride = (size_t)M * N;
    for (int o = tid; o < SBW * PER; o += 64 * NWAVES) {
        const int n = sb * SBW * PER + o;
        if (n >= N) break;
        float v[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) v[m] = 0.f;
        for (int s0 = 0; s0 < S; s0 += 16) {
            float t[16][MR];
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    t[e][m] = (s0 + e < S && m < M)
                                  ? __hip_atomic_load(part + (size_t)(s0 + e) * stride + (size_t)m * N + n,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                  : 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e)
#pragma unroll
                for (int m = 0; m < MR; ++m)
                    if (s0 + e < S) v[m] += t[e][m];
        }
#pragma unroll
        for (int m = 0; m < MR; ++m)
            if (m < M) a.y[(size_t)m * N + n] = (uint16_t)f32_to_bf16_rne(add_out_bias(a.ob, n, v[m]));
    }
    if (tid == 0) __hip_atomic_store(&cnt[sb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Three or four activation rows: y[m, n] = sum over the slices (in order) of
// part[s][m][n], plus the dense bias, rounded once to bf16, in a second
// kernel (the in-kernel completion measured slower there: 25.3 against
// 23.2 us at four rows). A thread takes 4 adjacent outputs (N % 4 == 0)
// and has 8 slices' loads in flight at a time.
__global__ void __launch_bounds__(256) qmm_nt_split_reduce(const float* part, int S, int M, int N,
                                                           uint16_t* y, OutBias ob) {
    typedef __attribute__((ext_vector_type(4))) float f32x4;
    const int64_t mn = (int64_t)M * N;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    const f32x4* p = (const f32x4*)(part + i);
    const int64_t stride = mn / 4;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= S; s += 8) {
        f32x4 t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = p[(s + j) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) v += t[j];
    }
    for (; s < S; ++s) v += p[s * stride];
    const int64_t n = i % N;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        y[i + e] = (uint16_t)f32_to_bf16_rne(add_out_bias(ob, n + e, v[e]));
}

// Slices and superblocks of the K-split form for q (S = 0: not taken).
struct SplitPlan {
    int S, ks, nsb, vw, rps;
};

inline SplitPlan split_plan(const QmmArgs& q) {
    SplitPlan p{0, 0, 0, 0, 0};
    const int per = 32 / q.bits;
    const int mr = nt_mr((int)q.M);
    int vw = mr <= 2 ? 4 : 2;
    const int gw = q.group_size / per;               // words per group
    if (vw > gw) vw = gw;
    if (q.bits < 4 && vw > q.bits) vw = q.bits;      // at most 32 columns per lane
    if (vw < 1) vw = 1;
    const int64_t wcols = q.N / per;
    p.vw = vw;
    p.rps = 64 / (SPLIT_SBW / vw);
    p.nsb = (int)((wcols + SPLIT_SBW - 1) / SPLIT_SBW);
    const int rows_step = p.rps * split_nw(mr);
    // at most one workgroup per CU (a second round of a few workgroups, or
    // two per CU, measured slower), slices of whole wave-load steps, x slice
    // at most 32 KB of LDS
    int S = device_shape().cus / p.nsb;
    if (S < 1) S = 1;
    int64_t ks = (q.K + S - 1) / S;
    ks = (ks + rows_step - 1) / rows_step * rows_step;
    const int64_t ks_max = (32 * 1024) / (2 * mr) / rows_step * rows_step;
    if (ks > ks_max) ks = ks_max;
    p.ks = (int)ks;
    p.S = (int)((q.K + ks - 1) / ks);
    return p;
}

template <int MODE, int BITS, int G, int MR, int VW>
hipError_t launch_split_kernel(const NtArgs& a, float* part, uint32_t* cnt, const SplitPlan& p,
                               hipStream_t st) {
    constexpr int PER = 32 / BITS;
    const size_t red = (size_t)split_nw(MR) * SPLIT_SBW * PER * 4;
    const size_t stage = (size_t)MR * p.ks * 2;
    const size_t shm = stage > red ? stage : red;
    const int nreal = p.nsb * p.S;
    const int xc = a.xcds > 1 ? a.xcds : 1;
    const int grid = (nreal + xc - 1) / xc * xc;
    qmm_nt_split_kernel<MODE, BITS, G, MR, VW><<<grid, 64 * split_nw(MR), shm, st>>>(
        a, part, cnt, p.ks, p.S, p.nsb, nreal);
    if constexpr (split_fuse(MR)) return hipGetLastError();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t quads = (int64_t)a.M * a.N / 4;
    qmm_nt_split_reduce<<<(unsigned)((quads + 255) / 256), 256, 0, st>>>(part, p.S, a.M, a.N, a.y, a.ob);
    return hipGetLastError();
}

template <int MODE, int BITS, int G>
hipError_t launch_split_fmt(const QmmArgs& q, float* part, uint32_t* cnt, const SplitPlan& p,
                            hipStream_t st) {
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
    a.xcds = device_shape().xcds;
    constexpr int PER = 32 / BITS;
    constexpr int GW = G / PER;
    constexpr int V4 = GW < 4 ? GW : (BITS < 4 ? BITS : 4);
    constexpr int V2 = GW < 2 ? GW : 2;
    if (nt_mr(a.M) == 1)
        return p.vw == V4 ? launch_split_kernel<MODE, BITS, G, 1, V4>(a, part, cnt, p, st) : hipErrorInvalidValue;
    if (nt_mr(a.M) == 2)
        return p.vw == V4 ? launch_split_kernel<MODE, BITS, G, 2, V4>(a, part, cnt, p, st) : hipErrorInvalidValue;
    if constexpr (BITS == 2) {
        return hipErrorNotSupported;   // 2-bit codes: one or two rows only (registers)
    } else {
        if (nt_mr(a.M) == 4)
            return p.vw == V2 ? launch_split_kernel<MODE, BITS, G, 4, V2>(a, part, cnt, p, st) : hipErrorInvalidValue;
        return hipErrorNotSupported;   // 5..8 rows: the one-pass kernel
    }
}

}  // namespace

bool qmm_nt_supports(const QmmArgs& q) {
    if (q.transpose || q.x_dtype != QLIN_BF16 || q.R != 0) return false;
    if (q.M < 1 || q.M > 8) return false;
    if (q.K > (1 << 20) || q.N > (1 << 28)) return false;
    if (q.K % 8 != 0 || ((uintptr_t)q.x & 15) != 0) return false;
    // scale and bias offsets are 32-bit buffer offsets
    if (q.K * (q.N / q.group_size) * 2 >= (1LL << 31)) return false;
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

size_t qmm_nt_split_workspace_bytes(const QmmArgs& q) {
    if (!qmm_nt_supports(q)) return 0;
    // 5..8 rows measured no faster split (34.4 against 33.8 us at M8, int4);
    // 2-bit codes' accumulators fit the registers at one or two rows only
    if (q.M > 4 || (q.bits == 2 && q.M > 2)) return 0;
    const SplitPlan p = split_plan(q);
    // 16-byte words per lane need 16-byte aligned weight rows
    if (p.vw > 1 && ((uintptr_t)q.wq % (4 * p.vw)) != 0) return 0;
    if (p.S < 2 || p.nsb > kSplitCounterBytes / 4) return 0;
    if (q.N % 4 != 0) return 0;               // the sum kernel takes 4 outputs per thread
    return kSplitCounterBytes + (size_t)p.S * (size_t)q.M * (size_t)q.N * 4u;
}

hipError_t launch_qmm_nt_split(const QmmArgs& q, void* workspace, hipStream_t st) {
    if (qmm_nt_split_workspace_bytes(q) == 0) return hipErrorNotSupported;
    const SplitPlan p = split_plan(q);
    uint32_t* cnt = (uint32_t*)workspace;
    float* part = (float*)((char*)workspace + kSplitCounterBytes);
    switch (q.mode) {
    case MXFP4: return launch_split_fmt<MXFP4, 4, 32>(q, part, cnt, p, st);
    case NVFP4: return launch_split_fmt<NVFP4, 4, 16>(q, part, cnt, p, st);
    case MXFP8: return launch_split_fmt<MXFP8, 8, 32>(q, part, cnt, p, st);
    default: break;
    }
    if (q.bits == 4) {
        if (q.group_size == 32) return launch_split_fmt<AFFINE, 4, 32>(q, part, cnt, p, st);
        if (q.group_size == 64) return launch_split_fmt<AFFINE, 4, 64>(q, part, cnt, p, st);
        return launch_split_fmt<AFFINE, 4, 128>(q, part, cnt, p, st);
    }
    if (q.bits == 8) {
        if (q.group_size == 32) return launch_split_fmt<AFFINE, 8, 32>(q, part, cnt, p, st);
        if (q.group_size == 64) return launch_split_fmt<AFFINE, 8, 64>(q, part, cnt, p, st);
        return launch_split_fmt<AFFINE, 8, 128>(q, part, cnt, p, st);
    }
    if (q.group_size == 32) return launch_split_fmt<AFFINE, 2, 32>(q, part, cnt, p, st);
    if (q.group_size == 64) return launch_split_fmt<AFFINE, 2, 64>(q, part, cnt, p, st);
    return launch_split_fmt<AFFINE, 2, 128>(q, part, cnt, p, st);
}

}  // namespace qlin
