/*
 * qlin.h -- C ABI of the MI355X (gfx950) group-wise quantization library.
 *
 * The library implements the operations described on these pages:
 *   "EMLX.Quantization" (emlx 0.4.2): quantize, dequantize,
 *       quantized_matmul, gather_quantized_matmul sections;
 *   "Emily.QuantizedWeight" (emily 0.7.2): Layout section and the
 *       Microscaled modes table;
 *   "Emily.Quantization.Layers" (emily 1.0.0): quantized_dense (the two
 *       weight layouts selected by `transpose`);
 *   mlx-rs "ops/quantization.rs" source: the quantize, quantized_matmul,
 *       dequantize and gather_qmm functions and their argument lists.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor is dense and row-major; every data pointer is a DEVICE
 *   pointer (memory from hipMalloc or a PyTorch CUDA/HIP tensor) on the
 *   current HIP device. Sizes are element counts.
 * - Ownership: the caller allocates and frees every buffer (inputs, outputs,
 *   workspace). The library never allocates, frees or keeps a pointer after
 *   the call returns.
 * - Asynchrony: all work is enqueued on `stream` (a hipStream_t; NULL means
 *   the default stream). The library never synchronises the host; buffers
 *   must stay alive until the stream has run the work.
 * - Errors: every argument is checked on the host before anything is
 *   launched; a rejected call launches nothing and leaves outputs untouched.
 *   The return value is a qlin_status; qlin_last_error() gives a message for
 *   the calling thread's last failure.
 * - Packing ("Emily.QuantizedWeight", Layout): codes of `bits` bits are
 *   packed 32/bits per uint32 word along the last axis, the element with the
 *   lowest index in the least significant bits.
 * - Modes ("Emily.QuantizedWeight", Microscaled modes table):
 *     "affine": bits in {2,4,8}, group_size in {32,64,128}; per group one
 *               scale and one bias, stored in the weight's float dtype;
 *     "mxfp4":  group 32, 4-bit E2M1 codes, one E8M0 scale byte per group;
 *     "mxfp8":  group 32, 8-bit E4M3 codes, one E8M0 scale byte per group;
 *     "nvfp4":  group 16, 4-bit E2M1 codes, one E4M3 scale byte per group.
 *   Microscaled modes have no biases (pass NULL). A (mode, group_size, bits)
 *   mismatch is QLIN_ERR_INVALID_ARGUMENT.
 * - Thread safety: no global mutable state besides the per-thread error
 *   text and last-path record; concurrent calls on different streams are
 *   independent.
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qlin_dtype {
    QLIN_F32 = 0,
    QLIN_F16 = 1,
    QLIN_BF16 = 2,
    QLIN_U8 = 3
} qlin_dtype;

typedef enum qlin_status {
    QLIN_OK = 0,
    QLIN_ERR_INVALID_ARGUMENT = 1, /* bad shape, dtype, mode, pairing, pointer */
    QLIN_ERR_UNSUPPORTED = 2,      /* valid combination the library does not run */
    QLIN_ERR_DEVICE = 3            /* a HIP launch or runtime call failed */
} qlin_status;

/*
 * qlin_quantize -- group-wise quantization of w [rows, cols] along cols.
 * ("EMLX.Quantization" quantize: rank >= 2, quantized along the last axis,
 * leading axes flattened into `rows`; mlx-rs quantize returns (wq, scales,
 * biases).)
 *   w        [rows, cols] of w_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16).
 *   wq       out, uint32 [rows, cols*bits/32].
 *   scales   out, [rows, cols/group_size]: w_dtype for "affine", uint8 bytes
 *            (E8M0 for mxfp4/mxfp8, E4M3 for nvfp4) otherwise.
 *   biases   out, like scales for "affine"; must be NULL otherwise.
 * Affine rule (the pages give only w ~ scale*q + bias): bias = group minimum
 * rounded down into w_dtype, scale = (max - bias)/(2^bits - 1) computed in
 * fp32 and rounded up into w_dtype, q = nearest-even of (w - bias)/scale in
 * fp32, clamped to [0, 2^bits-1]; a constant group has scale 0, codes 0.
 * Microscaled rule: OCP MX shared exponent floor(log2 amax) - emax_elem for
 * mxfp4/mxfp8; E4M3(amax/6) for nvfp4; elements nearest-even, saturating.
 * Requires cols % group_size == 0 and rows >= 1.
 */
qlin_status qlin_quantize(const void* w, qlin_dtype w_dtype, int64_t rows, int64_t cols,
                          int group_size, int bits, const char* mode, uint32_t* wq,
                          void* scales, void* biases, void* stream);

/*
 * qlin_dequantize -- dense weight from its quantized form
 * ("EMLX.Quantization" dequantize: the output has the logical shape; mlx-rs
 * dequantize takes an optional output dtype).
 *   wq [rows, cols*bits/32], scales/biases [rows, cols/group_size] as
 *   produced by qlin_quantize; scale_dtype is the float dtype of scales and
 *   biases for "affine" and must be QLIN_U8 otherwise.
 *   out [rows, cols] in out_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16).
 * Affine: out = round(fmaf(scale, q, bias)) -- one fp32 rounding, then
 * nearest-even into out_dtype. Microscaled: decode(q) * decode(scale byte).
 */
qlin_status qlin_dequantize(const uint32_t* wq, const void* scales, const void* biases,
                            qlin_dtype scale_dtype, int64_t rows, int64_t cols, int group_size,
                            int bits, const char* mode, void* out, qlin_dtype out_dtype,
                            void* stream);

/*
 * qlin_quantized_matmul -- fused y = x . W^T (transpose != 0) or y = x . W
 * (transpose == 0) on the quantized weight, without writing a dense W
 * ("EMLX.Quantization" quantized_matmul; "Emily.Quantization.Layers"
 * quantized_dense: transpose true is the [out, in] layout, false the
 * [in, out] layout).
 *   x   [M, K] of x_dtype (QLIN_F32, QLIN_F16 or QLIN_BF16); leading batch
 *       dims flattened into M; M == 0 is a no-op.
 *   wq  transpose: [N, K*bits/32], groups along K;
 *       else:      [K, N*bits/32], groups along N.
 *   scales/biases  transpose: [N, K/group_size]; else [K, N/group_size].
 *   y   out, [M, N] of x_dtype. For "affine" the output follows the scales
 *       dtype, so scale_dtype must equal x_dtype; microscaled output
 *       follows x.
 * Products accumulate in fp32.
 */
qlin_status qlin_quantized_matmul(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                  const uint32_t* wq, const void* scales, const void* biases,
                                  qlin_dtype scale_dtype, int64_t N, int transpose,
                                  int group_size, int bits, const char* mode, void* y,
                                  void* stream);

/*
 * qlin_quantized_matmul_workspace_bytes -- device workspace that lets
 * qlin_quantized_matmul_ws split K over workgroups for this shape: the
 * [in, out] layout (transpose == 0) with 1..4 rows of bf16 x (1..2 for
 * 2-bit codes) and K longer than one slice. 0 when the shape takes no
 * workspace (then qlin_quantized_matmul_ws is qlin_quantized_matmul). The
 * size assumes a 16-byte aligned wq; with another wq the call also falls
 * back to qlin_quantized_matmul.
 */
size_t qlin_quantized_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N, int transpose,
                                             int group_size, int bits, const char* mode);

/*
 * qlin_quantized_matmul_ws -- qlin_quantized_matmul with a caller's
 * workspace ("EMLX.Quantization" quantized_matmul, the same operation).
 * With at least qlin_quantized_matmul_workspace_bytes(...) bytes the
 * [in, out] layout at few rows splits K over workgroups: each stores fp32
 * partial sums of its slice of K in the workspace, and the workgroup that
 * finishes a column block last adds its slices in a fixed order (results do
 * not depend on scheduling) and writes y, all in one launch. With
 * workspace NULL, a smaller workspace or any other shape the call is
 * qlin_quantized_matmul's. The workspace is device memory the caller owns,
 * 16-byte aligned. Its first 4096 bytes hold completion counters: they must
 * be zero before the workspace's first use (e.g. hipMemset once after
 * allocating it) and every call leaves them zero; the rest is overwritten.
 * Calls that share one workspace must not overlap, and a workspace that
 * served another purpose must be zeroed again. A workspace whose counters
 * hold a value at or past the number of K slices (memory that was never
 * zeroed, typically) makes the call write NaN to the affected outputs, and
 * every later call on it does the same, until it is zeroed. Arguments and errors as for
 * qlin_quantized_matmul, plus QLIN_ERR_INVALID_ARGUMENT for a misaligned
 * workspace.
 */
qlin_status qlin_quantized_matmul_ws(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                     const uint32_t* wq, const void* scales, const void* biases,
                                     qlin_dtype scale_dtype, int64_t N, int transpose,
                                     int group_size, int bits, const char* mode, void* workspace,
                                     size_t workspace_bytes, void* y, void* stream);

/*
 * qlin_quantized_dense -- the dense layer on a quantized weight: y = x . W^T
 * (or x . W) plus a bias, fused into the matmul's output stage
 * ("Emily.Quantization.Layers" quantized_dense: x @ W (+ bias), the bias a
 * tensor or a number, 0 by default).
 *   x, wq, scales, biases, transpose, group_size, bits, mode, y: as for
 *       qlin_quantized_matmul.
 *   bias        device pointer to N values of bias_dtype (QLIN_F32, QLIN_F16
 *               or QLIN_BF16), one per output column, added to every row;
 *               or NULL, and then the number bias_value is added to every
 *               output (0 gives qlin_quantized_matmul's result).
 * The bias is added in fp32 to the fp32 accumulation of each output before
 * its one rounding into y's dtype. bias must be 4-byte aligned for QLIN_F32
 * and 2-byte aligned otherwise. Errors as for qlin_quantized_matmul, plus
 * QLIN_ERR_INVALID_ARGUMENT for a bias dtype outside those three or a
 * bias_value that is not finite once rounded to fp32 (the number is taken
 * in fp32).
 */
qlin_status qlin_quantized_dense(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K,
                                 const uint32_t* wq, const void* scales, const void* biases,
                                 qlin_dtype scale_dtype, int64_t N, int transpose,
                                 int group_size, int bits, const char* mode, const void* bias,
                                 qlin_dtype bias_dtype, double bias_value, void* y,
                                 void* stream);

/*
 * qlin_qqmm_workspace_bytes -- device workspace qlin_qqmm needs for x [M, K]:
 * the decoded activation, M*K bf16 values.
 */
size_t qlin_qqmm_workspace_bytes(int64_t M, int64_t K);

/*
 * qlin_qqmm -- matmul with both operands quantized: x is quantized on the
 * fly, W arrives quantized (mlx-rs qqmm: the nvfp4 and mxfp8 modes; the
 * optional global scales are not taken -- one level of scales).
 *   x        bf16 [M, K]; quantized along K with W's mode, group size and
 *            bits by the same rule as qlin_quantize. mxfp8 with M >= 32
 *            ([out, in] layout, K a multiple of 512): the workspace receives x's E4M3 codes
 *            [M, K] and then its E8M0 scales [M, K/32], which the CDNA4
 *            scaled fp8 MFMA multiplies against W's directly. Otherwise x is
 *            decoded back into the workspace as bf16 [M, K] (every decoded
 *            value is exact in bf16) for the bf16 MFMA kernels.
 *   wq, scales  W as for qlin_quantized_matmul in mode "nvfp4" (16, 4) or
 *            "mxfp8" (32, 8); no biases. transpose as there.
 *   workspace   device memory of at least qlin_qqmm_workspace_bytes(M, K)
 *            bytes, 16-byte aligned; the caller owns it; overwritten.
 *   y        out, bf16 [M, N] = dequant(quantize(x)) . dequant(W)^T (or . W),
 *            fp32 accumulation.
 * Errors: QLIN_ERR_INVALID_ARGUMENT for another mode, a mode/group/bits
 * mismatch, K not a multiple of the group, a short or misaligned workspace,
 * NULL pointers; QLIN_ERR_UNSUPPORTED for x other than bf16. M == 0 is a
 * no-op.
 */
qlin_status qlin_qqmm(const void* x, qlin_dtype x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                      const void* scales, int64_t N, int transpose, int group_size, int bits,
                      const char* mode, void* workspace, size_t workspace_bytes, void* y,
                      void* stream);

/*
 * qlin_gather_qmm_workspace_bytes -- device workspace qlin_gather_qmm needs
 * for R index rows over E experts (bucket offsets, counts and the row
 * permutation). Always > 0.
 */
size_t qlin_gather_qmm_workspace_bytes(int64_t R, int64_t E);

/*
 * qlin_gather_qmm -- mixture-of-experts quantized matmul
 * ("EMLX.Quantization" gather_quantized_matmul; mlx-rs gather_qmm):
 *   y[r] = x[lhs[r]] . W[rhs[r]]^T   (transpose != 0), or with W[rhs[r]]
 * for r in [0, R). The expert gather happens inside the op: expert weights
 * are read in place and never copied per row.
 *   x    [B, M, K] of x_dtype.
 *   wq   experts stacked on the leading axis: [E, N, K*bits/32] (transpose)
 *        or [E, K, N*bits/32]; scales/biases [E, N, K/g] or [E, K, N/g].
 *   lhs_indices  uint32 [R] in [0, B), or NULL meaning lhs[r] = r (then
 *        B must equal R). Reorders / selects activation rows.
 *   rhs_indices  uint32 [R] in [0, E): the expert of each row.
 *   sorted_indices  nonzero promises rhs is non-decreasing, so the library
 *        skips its own bucketing; results never depend on it.
 *   workspace  device buffer of at least
 *        qlin_gather_qmm_workspace_bytes(R, E) bytes, owned by the caller.
 *   y    out, [R, M, N] of x_dtype (same dtype rule as quantized_matmul).
 * Index values are a precondition. The kernels keep their own memory
 * accesses inside the buffers whatever the indices hold, but the output row
 * of an index row with rhs >= E or lhs >= B is unspecified (the grouped
 * kernels leave it unwritten). With the environment variable
 * QLIN_CHECK_INDICES=1 a small kernel checks every index first, the call
 * waits for it on the host and returns QLIN_ERR_INVALID_ARGUMENT naming the
 * first bad row, launching nothing else; under HIP graph capture that check
 * cannot wait and the call returns QLIN_ERR_UNSUPPORTED.
 */
qlin_status qlin_gather_qmm(const void* x, qlin_dtype x_dtype, int64_t B, int64_t M, int64_t K,
                            const uint32_t* wq, const void* scales, const void* biases,
                            qlin_dtype scale_dtype, int64_t E, int64_t N,
                            const uint32_t* lhs_indices, const uint32_t* rhs_indices, int64_t R,
                            int transpose, int group_size, int bits, const char* mode,
                            int sorted_indices, void* workspace, size_t workspace_bytes, void* y,
                            void* stream);

/*
 * qlin_gather_qmm_noalloc -- qlin_gather_qmm without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The call
 * allocates nothing; the bucketing scratch is a fixed device array inside
 * the library (about 295 KB per GPU, held until the process ends), which
 * limits the problem to R <= qlin_gather_qmm_noalloc_max_rows() (65536)
 * index rows and E <= qlin_gather_qmm_noalloc_max_experts() (4096) experts;
 * larger ones return QLIN_ERR_INVALID_ARGUMENT before anything runs (use
 * qlin_gather_qmm with a workspace). Every call on one GPU uses that GPU's
 * array: calls that overlap in time on the same GPU (other streams or
 * threads) race on it and must be serialised by the caller. Arguments,
 * results and errors are otherwise those of qlin_gather_qmm.
 */
qlin_status qlin_gather_qmm_noalloc(const void* x, qlin_dtype x_dtype, int64_t B, int64_t M,
                                    int64_t K, const uint32_t* wq, const void* scales,
                                    const void* biases, qlin_dtype scale_dtype, int64_t E,
                                    int64_t N, const uint32_t* lhs_indices,
                                    const uint32_t* rhs_indices, int64_t R, int transpose,
                                    int group_size, int bits, const char* mode, int sorted_indices,
                                    void* y, void* stream);
size_t qlin_gather_qmm_noalloc_max_rows(void);
size_t qlin_gather_qmm_noalloc_max_experts(void);

/* Message describing the calling thread's last failed call ("" if none). */
const char* qlin_last_error(void);

/*
 * Kernel path of the calling thread's last matmul-type call that reached a
 * launch (a static string: "decode", "in_out", "in_out_split",
 * "in_out_row_blocks", "prefill", "tiled", "generic", "gather_decode",
 * "gather_prefill", "qqmm_scaled_mfma"; "" before any). "generic" is the fp32 VALU fallback for
 * shapes the fast kernels do not take, typically an order of magnitude
 * slower; QLIN_WARN_FALLBACK=1 also prints a line to stderr when it runs.
 */
const char* qlin_last_path(void);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
