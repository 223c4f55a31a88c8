// gather_index.hip -- index handling of the mixture-of-experts matmul
// ("EMLX.Quantization", gather_quantized_matmul: rhs_indices names the expert
// of each row, lhs_indices the activation batch entry it reads; mlx-rs
// gather_qmm and its sorted_indices hint).
//
//  * bucket_kernel groups the index rows by expert on the device (counts,
//    scans, placement), so each expert's weight is read once for all of its
//    rows and never copied per row.
//  * check_indices_kernel is the opt-in range check (QLIN_CHECK_INDICES=1):
//    it finds the first index row whose expert is >= E or whose batch entry
//    is >= B and reports it to the host before any gather kernel runs.

#include "qlin_common.h"

namespace qlin {
namespace {

// One workgroup: per-expert counts, exclusive scan into offsets and row-tile
// prefix, then rows placed into expert order (or the identity when the
// caller's indices are verified non-decreasing). Index rows whose expert is
// not below E are left out of every bucket (their output rows are never
// written), so a bad index cannot move an LDS or global access out of range.
// Eight waves; each thread keeps the experts of its first BCACHE rows in
// registers, so rhs is read once (the kernel is latency-bound: a few
// barriers and memory round trips).
constexpr int BUCKET_THREADS = 512;   // 8 waves: MoE 4096 rows ~1.8 us faster than 4
// a single wave for few index rows (decode-sized batches): its barriers cost
// nothing and the one workgroup is all there is to launch
constexpr int64_t BUCKET_SMALL_R = 512;

template <int NTH>
__global__ void __launch_bounds__(NTH) bucket_kernel(const uint32_t* __restrict__ rhs, int R,
                                                                int E, int M, int BMrows, int sorted,
                                                                uint32_t* __restrict__ offsets,
                                                                uint32_t* __restrict__ tiles,
                                                                uint32_t* __restrict__ perm) {
    constexpr int NT = NTH;
    constexpr int BCACHE = NT >= 512 ? 4096 / NT : 8;   // rows per thread kept in registers
    extern __shared__ uint32_t sh[];
    uint32_t* cnt = sh;          // [E]
    uint32_t* cur = sh + E;      // [E]
    __shared__ int unsorted;
    __shared__ uint32_t carry[2];
    __shared__ uint32_t wsum[NT / 64][2];
    const int tid = threadIdx.x;
    if (tid == 0) {
        unsorted = 0;
        carry[0] = carry[1] = 0;
    }
    for (int e = tid; e < E; e += NT) cnt[e] = 0;
    // rows tid + c * NT, c < BCACHE: experts kept in registers
    uint32_t rv[BCACHE];
#pragma unroll
    for (int c = 0; c < BCACHE; ++c) {
        const int r = tid + c * NT;
        rv[c] = r < R ? rhs[r] : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < BCACHE; ++c) {
        const int r = tid + c * NT;
        if (r < R) {
            if (rv[c] < (uint32_t)E) atomicAdd(&cnt[rv[c]], 1u);
            else unsorted = 1;
            if (sorted && r + 1 < R && rv[c] > rhs[r + 1]) unsorted = 1;
        }
    }
    for (int r = tid + BCACHE * NT; r < R; r += NT) {
        const uint32_t v = rhs[r];
        if (v < (uint32_t)E) atomicAdd(&cnt[v], 1u);
        else unsorted = 1;
        if (sorted && r + 1 < R && v > rhs[r + 1]) unsorted = 1;
    }
    __syncthreads();
    // exclusive scans of counts and of row tiles, in chunks of NT experts
    for (int base = 0; base < E; base += NT) {
        const int e = base + tid;
        const uint32_t c = e < E ? cnt[e] : 0u;
        const uint32_t t = (uint32_t)(((uint64_t)c * M + BMrows - 1) / BMrows);
        uint32_t vc = c, vt = t;
        // inclusive wave scans, then across waves through shared memory
        for (int off = 1; off < 64; off <<= 1) {
            uint32_t uc = __shfl_up(vc, off, 64), ut = __shfl_up(vt, off, 64);
            if ((tid & 63) >= off) {
                vc += uc;
                vt += ut;
            }
        }
        if ((tid & 63) == 63) {
            wsum[tid >> 6][0] = vc;
            wsum[tid >> 6][1] = vt;
        }
        __syncthreads();
        uint32_t pc = carry[0], pt = carry[1];
        for (int w = 0; w < (tid >> 6); ++w) {
            pc += wsum[w][0];
            pt += wsum[w][1];
        }
        if (e < E) {
            offsets[e] = pc + vc - c;
            tiles[e] = pt + vt - t;
            cur[e] = pc + vc - c;
        }
        __syncthreads();
        if (tid == NT - 1) {
            carry[0] = pc + vc;
            carry[1] = pt + vt;
        }
        __syncthreads();
    }
    if (tid == 0) {
        offsets[E] = carry[0];
        tiles[E] = carry[1];
    }
    if (sorted && !unsorted) {
        for (int r = tid; r < R; r += NT) perm[r] = (uint32_t)r;
    } else {
#pragma unroll
        for (int c = 0; c < BCACHE; ++c) {
            const int r = tid + c * NT;
            if (r < R && rv[c] < (uint32_t)E) perm[atomicAdd(&cur[rv[c]], 1u)] = (uint32_t)r;
        }
        for (int r = tid + BCACHE * NT; r < R; r += NT) {
            const uint32_t v = rhs[r];
            if (v < (uint32_t)E) perm[atomicAdd(&cur[v], 1u)] = (uint32_t)r;
        }
    }
}

constexpr int CHECK_THREADS = 1024;

// One workgroup: every thread scans index rows tid, tid + 1024, ...; the
// smallest bad row wins. res[0] = that row (0xFFFFFFFF when every index is in
// range), res[1] = its rhs value, res[2] = its lhs value (or the row itself
// without lhs).
__global__ void __launch_bounds__(CHECK_THREADS) check_indices_kernel(
    const uint32_t* __restrict__ rhs, const uint32_t* __restrict__ lhs, uint32_t R, uint32_t E,
    uint32_t B, uint32_t* __restrict__ res) {
    __shared__ uint32_t wmin[CHECK_THREADS / 64];
    uint32_t bad = 0xFFFFFFFFu;
    for (uint32_t r = threadIdx.x; r < R; r += CHECK_THREADS) {
        const bool ok = rhs[r] < E && (lhs ? lhs[r] < B : r < B);
        if (!ok) {
            bad = r;
            break;   // rows grow along the loop: the first bad one is this thread's least
        }
    }
    for (int off = 32; off >= 1; off >>= 1) bad = min(bad, (uint32_t)__shfl_xor((int)bad, off, 64));
    if ((threadIdx.x & 63) == 0) wmin[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t b = 0xFFFFFFFFu;
        for (int w = 0; w < CHECK_THREADS / 64; ++w) b = min(b, wmin[w]);
        res[0] = b;
        res[1] = b != 0xFFFFFFFFu ? rhs[b] : 0u;
        res[2] = b != 0xFFFFFFFFu ? (lhs ? lhs[b] : b) : 0u;
    }
}

}  // namespace

size_t bucket_workspace_bytes(int64_t R, int64_t E) {
    // offsets [E+1], tiles [E+1], perm [R], then 256 bytes of which the
    // first 16 (16-byte aligned) hold the index check's result
    return (size_t)(2 * (E + 1) + R) * sizeof(uint32_t) + 256;
}

uint32_t* index_check_result(void* workspace, int64_t R, int64_t E) {
    const uintptr_t p = (uintptr_t)workspace + (size_t)(2 * (E + 1) + R) * sizeof(uint32_t);
    return (uint32_t*)((p + 15) & ~(uintptr_t)15);
}

hipError_t launch_check_indices(const uint32_t* rhs, const uint32_t* lhs, int64_t R, int64_t E,
                                int64_t B, uint32_t* result, hipStream_t st) {
    if (R <= 0 || R >= (1LL << 32) - 1 || E >= (1LL << 32) || B >= (1LL << 32))
        return hipErrorInvalidValue;
    check_indices_kernel<<<1, CHECK_THREADS, 0, st>>>(rhs, lhs, (uint32_t)R, (uint32_t)E,
                                                      (uint32_t)B, result);
    return hipGetLastError();
}

hipError_t launch_bucket(const uint32_t* rhs, int64_t R, int64_t E, int64_t M, int sorted,
                         int rows_per_tile, void* workspace, uint32_t** perm, uint32_t** offsets,
                         hipStream_t st) {
    uint32_t* ws = (uint32_t*)workspace;
    *offsets = ws;                   // [E+1] then tiles [E+1]
    *perm = ws + 2 * (E + 1);
    const size_t shm = (size_t)2 * E * sizeof(uint32_t);
    if (shm > 64 * 1024) return hipErrorInvalidValue;
    if (rows_per_tile < 1) return hipErrorInvalidValue;
    if (R <= BUCKET_SMALL_R)
        bucket_kernel<64><<<1, 64, shm, st>>>(rhs, (int)R, (int)E, (int)M, rows_per_tile, sorted,
                                              *offsets, *offsets + (E + 1), *perm);
    else
        bucket_kernel<BUCKET_THREADS><<<1, BUCKET_THREADS, shm, st>>>(rhs, (int)R, (int)E, (int)M,
                                                                      rows_per_tile, sorted, *offsets,
                                                                      *offsets + (E + 1), *perm);
    return hipGetLastError();
}

}  // namespace qlin
