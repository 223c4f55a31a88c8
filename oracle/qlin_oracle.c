/*
 * qlin_oracle.c -- plain, slow CPU oracle for group-wise quantization and the
 * quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the independent reference that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. The product path never calls it,
 * and it shares no source, header, table or helper with the HIP library.
 *
 * Sources (the pages describe the operations; rounding details they leave
 * open are fixed here and each is marked READING):
 *   [EMLX]  "EMLX.Quantization" (emlx 0.4.2) -- module doc, quantize,
 *           dequantize, quantized_matmul, gather_quantized_matmul sections.
 *   [QW]    "Emily.QuantizedWeight" (emily 0.7.2) -- Layout section,
 *           Microscaled modes table, from_dense options.
 *   [LAY]   "Emily.Quantization.Layers" (emily 1.0.0) -- quantized_dense.
 *   [RS]    "mlx_rs/ops/quantization.rs" source page -- the quantize,
 *           quantized_matmul, dequantize and gather_qmm doc comments, and the
 *           unit tests test_quantize_dequantize, test_quantized_matmul,
 *           test_gather_qmm.
 *   [OCP]   OCP Microscaling Formats (MX) v1.0 -- element/scale encodings
 *           E2M1, E4M3 and E8M0 (not on the pages; the pages only name the
 *           modes).
 *
 * Style: every value is produced by the arithmetic its definition states, in
 * the order it states it. Floating-point formats other than fp32/fp64 are
 * handled by one generic rounding routine (oracle_round) working on exact
 * double values, never by bit tricks. Built with -O2 -ffp-contract=off and no
 * fast-math, so every float expression below is one IEEE operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype codes (this file's own numbering; the Python wrapper maps names) */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_U8 = 3 };
/* status codes */
enum { OR_OK = 0, OR_EINVAL = 1, OR_EUNSUP = 2 };
/* rounding modes */
enum { RND_NEAREST_EVEN = 0, RND_DOWN = 1, RND_UP = 2 };
/* number formats */
enum { FMT_F32 = 0, FMT_F16 = 1, FMT_BF16 = 2, FMT_E4M3 = 3, FMT_E2M1 = 4, FMT_E8M0 = 5 };
/* modes */
enum { MODE_AFFINE = 0, MODE_MXFP4 = 1, MODE_MXFP8 = 2, MODE_NVFP4 = 3, MODE_BAD = -1 };

/* ------------------------------------------------------------------------ */
/* Generic binary floating-point formats                                     */
/* ------------------------------------------------------------------------ */

/* Parameters of a binary format: p significand bits (implicit bit included),
 * emin the exponent of the smallest normal, maxval the largest finite value. */
typedef struct { int p; int emin; double maxval; } fmt_t;

static fmt_t fmt_params(int fmt) {
    fmt_t f;
    switch (fmt) {
    case FMT_F32:  f.p = 24; f.emin = -126; f.maxval = ldexp(2.0 - ldexp(1.0, -23), 127); break;
    case FMT_F16:  f.p = 11; f.emin = -14;  f.maxval = 65504.0; break;
    case FMT_BF16: f.p = 8;  f.emin = -126; f.maxval = ldexp(2.0 - ldexp(1.0, -7), 127); break;
    /* [OCP] E4M3: bias 7, 3 mantissa bits, S.1111.111 is NaN, largest 448. */
    case FMT_E4M3: f.p = 4;  f.emin = -6;   f.maxval = 448.0; break;
    /* [OCP] E2M1: bias 1, 1 mantissa bit, no inf/NaN, largest 6. */
    case FMT_E2M1: f.p = 2;  f.emin = 0;    f.maxval = 6.0; break;
    default:       f.p = 0;  f.emin = 0;    f.maxval = 0.0; break;
    }
    return f;
}

/* Nearest integer to t, ties to the even integer. */
static double rne_int(double t) {
    double fl = floor(t), diff = t - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Round the exact real v to format `fmt` with rounding `rnd`, exponent range
 * unbounded above (the caller decides overflow) and gradual underflow below.
 * The spacing of representable values at v is 2^(E-p+1) with
 * E = max(floor(log2|v|), emin); v divided by that spacing is an exact double
 * (power-of-two scaling), and is rounded to an integer by the chosen mode. */
double oracle_round(double v, int fmt, int rnd) {
    fmt_t f = fmt_params(fmt);
    if (v == 0.0 || !isfinite(v)) return v;
    int ex;
    frexp(v, &ex);              /* |v| = m * 2^ex, m in [0.5, 1) */
    int E = ex - 1;             /* floor(log2 |v|) */
    if (E < f.emin) E = f.emin;
    double ulp = ldexp(1.0, E - f.p + 1);
    double t = v / ulp;         /* exact */
    double r = (rnd == RND_DOWN) ? floor(t) : (rnd == RND_UP) ? ceil(t) : rne_int(t);
    double out = r * ulp;
    if (out == 0.0) out = copysign(0.0, v);
    return out;
}

/* Round to nearest-even into a storage float format; overflow gives inf. */
static double round_store(double v, int fmt) {
    fmt_t f = fmt_params(fmt);
    double r = oracle_round(v, fmt, RND_NEAREST_EVEN);
    if (fabs(r) > f.maxval) r = copysign(INFINITY, v);
    return r;
}

/* Decode one element / scale code of a small format from its definition.
 * [OCP] E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * [OCP] E4M3: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 *       S.1111.111 is NaN.
 * [OCP] E8M0: value 2^(code-127); code 255 is NaN. */
double oracle_decode(int fmt, unsigned code) {
    if (fmt == FMT_E2M1) {
        int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
        double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m / 2.0, e - 1);
        return s ? -mag : mag;
    }
    if (fmt == FMT_E4M3) {
        int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
        if (e == 15 && m == 7) return NAN;
        double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
        return s ? -mag : mag;
    }
    if (fmt == FMT_E8M0) {
        if (code == 255) return NAN;
        return ldexp(1.0, (int)code - 127);
    }
    return NAN;
}

/* Encode v into a small element format: round to nearest-even, saturate to the
 * largest finite magnitude, keep the sign (a negative value that rounds to
 * zero gives the -0 code). The code is found by searching the decode table,
 * so encode is by construction the inverse of oracle_decode. */
unsigned oracle_encode(int fmt, double v) {
    fmt_t f = fmt_params(fmt);
    int nbits = (fmt == FMT_E2M1) ? 4 : 8;
    unsigned sign_bit = 1u << (nbits - 1);
    double r = oracle_round(v, fmt, RND_NEAREST_EVEN);
    if (fabs(r) > f.maxval) r = copysign(f.maxval, v);
    double mag = fabs(r);
    for (unsigned c = 0; c < sign_bit; ++c) {
        double d = oracle_decode(fmt, c);
        if (d == mag) return signbit(v) ? (c | sign_bit) : c;
    }
    return 0xFFFFFFFFu; /* unreachable for finite v */
}

/* ------------------------------------------------------------------------ */
/* Storage dtypes                                                            */
/* ------------------------------------------------------------------------ */

static int dtype_fmt(int dtype) {
    return dtype == OR_F32 ? FMT_F32 : dtype == OR_F16 ? FMT_F16 : dtype == OR_BF16 ? FMT_BF16 : -1;
}

/* Widen one stored value to double (exact). bf16 is the top half of an fp32;
 * f16 is decoded from its fields. */
static double load_val(const void* p, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float*)p)[i];
    if (dtype == OR_BF16) {
        uint32_t b = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &b, 4);
        return (double)f;
    }
    if (dtype == OR_F16) {
        uint16_t h = ((const uint16_t*)p)[i];
        int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
        double mag;
        if (e == 31) mag = m ? NAN : INFINITY;
        else if (e == 0) mag = ldexp((double)m, -24);
        else mag = ldexp(1.0 + m / 1024.0, e - 15);
        return s ? -mag : mag;
    }
    return NAN;
}

/* Store v (already representable in dtype, or rounded here to nearest-even). */
static void store_val(void* p, int dtype, int64_t i, double v) {
    if (dtype == OR_F32) { ((float*)p)[i] = (float)round_store(v, FMT_F32); return; }
    double r = round_store(v, dtype_fmt(dtype));
    if (dtype == OR_BF16) {
        float f = (float)r; /* exact: a bf16 value is an fp32 value */
        uint32_t b;
        memcpy(&b, &f, 4);
        ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
        return;
    }
    if (dtype == OR_F16) {
        uint16_t s = signbit(r) ? 0x8000 : 0;
        double a = fabs(r);
        uint16_t bits;
        if (isinf(a)) bits = 0x7C00;
        else if (a == 0.0) bits = 0;
        else {
            int ex;
            frexp(a, &ex);
            int E = ex - 1;
            if (E < -14) bits = (uint16_t)(a / ldexp(1.0, -24)); /* subnormal */
            else bits = (uint16_t)(((E + 15) << 10) | (uint16_t)((a / ldexp(1.0, E) - 1.0) * 1024.0));
        }
        ((uint16_t*)p)[i] = s | bits;
    }
}

/* ------------------------------------------------------------------------ */
/* Modes and validation                                                      */
/* ------------------------------------------------------------------------ */

static int parse_mode(const char* mode) {
    if (!mode) return MODE_BAD;
    if (!strcmp(mode, "affine")) return MODE_AFFINE;
    if (!strcmp(mode, "mxfp4")) return MODE_MXFP4;
    if (!strcmp(mode, "mxfp8")) return MODE_MXFP8;
    if (!strcmp(mode, "nvfp4")) return MODE_NVFP4;
    return MODE_BAD;
}

/* [QW] Microscaled modes table: mxfp4 = (32, 4), mxfp8 = (32, 8),
 * nvfp4 = (16, 4); a mismatch is an error. [EMLX] quantize options: affine
 * group_size in {32, 64, 128}, bits in {2, 4, 8}; the group size must divide
 * the last dimension. READING: 3- and 6-bit affine (listed only by [QW]
 * from_dense) are rejected: 32/bits is not a whole number of codes per word. */
static int check_params(int mode, int group_size, int bits, int64_t last_dim) {
    if (mode == MODE_BAD) return OR_EINVAL;
    if (mode == MODE_AFFINE) {
        if (bits != 2 && bits != 4 && bits != 8) return OR_EINVAL;
        if (group_size != 32 && group_size != 64 && group_size != 128) return OR_EINVAL;
    } else {
        int g = (mode == MODE_NVFP4) ? 16 : 32;
        int b = (mode == MODE_MXFP8) ? 8 : 4;
        if (group_size != g || bits != b) return OR_EINVAL;
    }
    if (last_dim <= 0 || last_dim % group_size != 0) return OR_EINVAL;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Packing                                                                   */
/* ------------------------------------------------------------------------ */

/* [QW] Layout: codes are packed 32/bits to a uint32 along the last axis
 * (e.g. 8 nibbles per word for 4 bits). READING: element k of a row sits in
 * word k/(32/bits) at bit (k mod (32/bits))*bits, least significant first. */
static unsigned get_code(const uint32_t* row_words, int64_t k, int bits) {
    int per = 32 / bits;
    uint32_t w = row_words[k / per];
    return (w >> ((k % per) * bits)) & ((1u << bits) - 1u);
}

static void put_code(uint32_t* row_words, int64_t k, int bits, unsigned q) {
    int per = 32 / bits;
    row_words[k / per] |= (uint32_t)q << ((k % per) * bits);
}

/* ------------------------------------------------------------------------ */
/* Quantize                                                                  */
/* ------------------------------------------------------------------------ */

/* Affine quantization of one group ([RS] quantize doc: every group_size
 * elements of a row share one scale and one bias; w ~ scale*q + bias).
 * READING (min-max): bias = min, scale = (max - min)/(2^bits - 1), stored in
 * the weight's dtype ([QW] Layout: scales take the source weight's dtype) with
 * the bias rounded down and the scale rounded up, so the stored grid still
 * covers [min, max] and |w - dequant| <= scale/2. Codes are the nearest-even
 * integer of (w - bias)/scale, each step one fp32 operation, clamped to
 * [0, 2^bits - 1]; a constant group has scale 0 and all codes 0. */
static void quantize_affine_group(const void* w, int dtype, int64_t base, int g, int bits,
                                  uint32_t* row_words, int64_t k0, double* s_out, double* z_out) {
    int fmt = dtype_fmt(dtype);
    int n = (1 << bits) - 1;
    float lo = (float)load_val(w, dtype, base), hi = lo;
    for (int i = 1; i < g; ++i) {
        float v = (float)load_val(w, dtype, base + i);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
    }
    float z = (float)oracle_round((double)lo, fmt, RND_DOWN);
    float range = hi - z;
    float s32 = range / (float)n;
    float s = (float)oracle_round((double)s32, fmt, RND_UP);
    for (int i = 0; i < g; ++i) {
        unsigned q = 0;
        if (s != 0.0f) {
            float v = (float)load_val(w, dtype, base + i);
            float d = v - z;
            float t = d / s;
            double r = rne_int((double)t);
            if (r < 0.0) r = 0.0;
            if (r > (double)n) r = (double)n;
            q = (unsigned)r;
        }
        put_code(row_words, k0 + i, bits, q);
    }
    *s_out = (double)s;
    *z_out = (double)z;
}

/* Microscaled quantization of one group (no bias; [EMLX] module doc and [QW]
 * Layout: one scale byte per group, e8m0 for mxfp4/mxfp8, e4m3 for nvfp4).
 * READING for mxfp4/mxfp8 ([OCP] conversion rule): shared exponent
 * e = floor(log2 amax) - emax_elem (emax_elem 2 for E2M1, 8 for E4M3),
 * clamped to [-127, 127]; scale byte e + 127; amax = 0 gives byte 0.
 * Elements are w / 2^e rounded nearest-even, saturating.
 * READING for nvfp4: scale = E4M3(amax / 6) (nearest-even, saturating), no
 * second-level scale; a zero scale gives zero codes; elements are
 * fl32(w / scale) rounded nearest-even into E2M1, saturating. */
static unsigned quantize_micro_group(const void* w, int dtype, int64_t base, int g, int mode,
                                     uint32_t* row_words, int64_t k0, int bits) {
    double amax = 0.0;
    for (int i = 0; i < g; ++i) {
        double a = fabs(load_val(w, dtype, base + i));
        if (a > amax) amax = a;
    }
    int efmt = (mode == MODE_MXFP8) ? FMT_E4M3 : FMT_E2M1;
    if (mode == MODE_NVFP4) {
        float a32 = (float)amax;
        float ratio = a32 / 6.0f;
        unsigned sbyte = oracle_encode(FMT_E4M3, (double)ratio);
        float sc = (float)oracle_decode(FMT_E4M3, sbyte);
        for (int i = 0; i < g; ++i) {
            double v = load_val(w, dtype, base + i);
            unsigned c;
            if (sc == 0.0f) c = signbit(v) ? 0x8u : 0x0u;
            else {
                float t = (float)v / sc;
                c = oracle_encode(FMT_E2M1, (double)t);
            }
            put_code(row_words, k0 + i, bits, c);
        }
        return sbyte;
    }
    int emax_elem = (efmt == FMT_E2M1) ? 2 : 8;
    int e;
    if (amax == 0.0) e = -127;
    else {
        int ex;
        frexp(amax, &ex);
        e = (ex - 1) - emax_elem;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
    }
    for (int i = 0; i < g; ++i) {
        double v = load_val(w, dtype, base + i);
        unsigned c = oracle_encode(efmt, ldexp(v, -e));
        put_code(row_words, k0 + i, bits, c);
    }
    return (unsigned)(e + 127);
}

/* quantize(w [rows, cols]) -> wq u32 [rows, cols*bits/32], scales/biases
 * [rows, cols/group_size] ([RS] quantize returns three arrays; [EMLX] quantize:
 * along the last axis, leading axes flattened into rows). Microscaled scales
 * are one byte each and biases must be NULL. */
int oracle_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int group_size,
                    int bits, const char* mode_str, uint32_t* wq, void* scales, void* biases) {
    int mode = parse_mode(mode_str);
    if (check_params(mode, group_size, bits, cols) != OR_OK) return OR_EINVAL;
    if (dtype_fmt(w_dtype) < 0 || rows <= 0 || !w || !wq || !scales) return OR_EINVAL;
    if ((mode == MODE_AFFINE) != (biases != NULL)) return OR_EINVAL;
    int64_t words = cols * bits / 32, groups = cols / group_size;
    memset(wq, 0, (size_t)(rows * words) * sizeof(uint32_t));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t j = 0; j < groups; ++j) {
            int64_t base = r * cols + j * group_size;
            if (mode == MODE_AFFINE) {
                double s, z;
                quantize_affine_group(w, w_dtype, base, group_size, bits, wq + r * words,
                                      j * group_size, &s, &z);
                store_val(scales, w_dtype, r * groups + j, s);
                store_val(biases, w_dtype, r * groups + j, z);
            } else {
                unsigned b = quantize_micro_group(w, w_dtype, base, group_size, mode,
                                                  wq + r * words, j * group_size, bits);
                ((uint8_t*)scales)[r * groups + j] = (uint8_t)b;
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Dequantize                                                                */
/* ------------------------------------------------------------------------ */

/* One dequantized weight in fp32.
 * Affine: scale*q + bias with a single rounding (fmaf) -- READING of the
 * pages' "w ~ scale*q + bias" ([RS] quantized_matmul doc).
 * Microscaled: decode(code) * decode(scale byte), exact in fp32. */
static float dq_elem(const uint32_t* row_words, int64_t k, const void* scales,
                     const void* biases, int sdtype, int64_t gidx, int bits, int mode) {
    unsigned q = get_code(row_words, k, bits);
    if (mode == MODE_AFFINE) {
        float s = (float)load_val(scales, sdtype, gidx);
        float z = (float)load_val(biases, sdtype, gidx);
        return fmaf(s, (float)q, z);
    }
    uint8_t sb = ((const uint8_t*)scales)[gidx];
    double sc = (mode == MODE_NVFP4) ? oracle_decode(FMT_E4M3, sb) : oracle_decode(FMT_E8M0, sb);
    double el = oracle_decode(mode == MODE_MXFP8 ? FMT_E4M3 : FMT_E2M1, q);
    return (float)(el * sc);
}

/* dequantize -> out [rows, cols] in out_dtype ([EMLX] dequantize: same logical
 * shape; [RS] dequantize takes an optional output dtype). The fp32 value is
 * rounded nearest-even into out_dtype. */
int oracle_dequantize(const uint32_t* wq, const void* scales, const void* biases, int scale_dtype,
                      int64_t rows, int64_t cols, int group_size, int bits, const char* mode_str,
                      void* out, int out_dtype) {
    int mode = parse_mode(mode_str);
    if (check_params(mode, group_size, bits, cols) != OR_OK) return OR_EINVAL;
    if (!wq || !scales || !out || rows <= 0 || dtype_fmt(out_dtype) < 0) return OR_EINVAL;
    if (mode == MODE_AFFINE && (dtype_fmt(scale_dtype) < 0 || !biases)) return OR_EINVAL;
    if (mode != MODE_AFFINE && (scale_dtype != OR_U8 || biases)) return OR_EINVAL;
    int64_t words = cols * bits / 32, groups = cols / group_size;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k) {
            float v = dq_elem(wq + r * words, k, scales, biases, scale_dtype,
                              r * groups + k / group_size, bits, mode);
            store_val(out, out_dtype, r * cols + k, (double)v);
        }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Quantized matmul                                                          */
/* ------------------------------------------------------------------------ */

/* Dense fp32 dequantized weight of one [rows, cols] matrix (helper for qmm). */
static float* dense_weight(const uint32_t* wq, const void* scales, const void* biases,
                           int sdtype, int64_t rows, int64_t cols, int g, int bits, int mode) {
    float* d = (float*)malloc((size_t)(rows * cols) * sizeof(float));
    if (!d) return NULL;
    int64_t words = cols * bits / 32, groups = cols / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < cols; ++k)
            d[r * cols + k] = dq_elem(wq + r * words, k, scales, biases, sdtype,
                                      r * groups + k / g, bits, mode);
    return d;
}

/* y = x . dequant(W)^T  (transpose=1, W stored [N, K]) or
 * y = x . dequant(W)    (transpose=0, W stored [K, N], groups along N)
 * ([EMLX] quantized_matmul; [LAY] quantized_dense: transpose true is the
 * [out, in] layout, false the [in, out] layout; [RS] test_quantized_matmul
 * compares against x.matmul(dequantize(w))). The sum runs over k in order in
 * fp64 with fp64 products of the fp32 dequantized weights; y is fp64. */
static int qmm_dense(const void* x, int x_dtype, int64_t M, int64_t K, const float* wd, int64_t N,
                     int transpose, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double wv = transpose ? (double)wd[n * K + k] : (double)wd[k * N + n];
                acc += load_val(x, x_dtype, m * K + k) * wv;
            }
            y[m * N + n] = acc;
        }
    return OR_OK;
}

/* Shared argument checks of quantized_matmul and gather_qmm ([EMLX]
 * quantized_matmul: affine output follows the scales dtype, microscaled the
 * activation's). READING: affine requires x's dtype to equal the scales'. */
static int check_qmm_args(int mode, int x_dtype, int sdtype, const void* biases) {
    if (dtype_fmt(x_dtype) < 0) return OR_EINVAL;
    if (mode == MODE_AFFINE) {
        if (dtype_fmt(sdtype) < 0 || !biases || sdtype != x_dtype) return OR_EINVAL;
    } else if (sdtype != OR_U8 || biases) {
        return OR_EINVAL;
    }
    return OR_OK;
}

int oracle_quantized_matmul(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                            const void* scales, const void* biases, int scale_dtype, int64_t N,
                            int transpose, int group_size, int bits, const char* mode_str,
                            double* y) {
    int mode = parse_mode(mode_str);
    int64_t qrows = transpose ? N : K, qcols = transpose ? K : N;
    if (check_params(mode, group_size, bits, qcols) != OR_OK) return OR_EINVAL;
    if (check_qmm_args(mode, x_dtype, scale_dtype, biases) != OR_OK) return OR_EINVAL;
    if (!x || !wq || !scales || !y || M < 0 || N <= 0 || K <= 0) return OR_EINVAL;
    if (M == 0) return OR_OK;
    float* wd = dense_weight(wq, scales, biases, scale_dtype, qrows, qcols, group_size, bits, mode);
    if (!wd) return OR_EUNSUP;
    qmm_dense(x, x_dtype, M, K, wd, N, transpose, y);
    free(wd);
    return OR_OK;
}

/* quantized_dense ([LAY] quantized_dense: x times the quantized W, plus a
 * bias that is a tensor or a number, 0 when omitted): the quantized_matmul
 * above, then the bias added to every output.
 * READING: a tensor bias holds one value per output column (N values, the
 * dense layer's bias) and is broadcast over the rows of y; a number is taken
 * in fp32 (rounded to nearest even), the precision of the accumulation it
 * joins. y stays fp64, before any rounding to the output dtype. */
int oracle_quantized_dense(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                           const void* scales, const void* biases, int scale_dtype, int64_t N,
                           int transpose, int group_size, int bits, const char* mode_str,
                           const void* bias, int bias_dtype, double bias_value, double* y) {
    if (bias && dtype_fmt(bias_dtype) < 0) return OR_EINVAL;
    if (!bias && !isfinite(bias_value)) return OR_EINVAL;
    int rc = oracle_quantized_matmul(x, x_dtype, M, K, wq, scales, biases, scale_dtype, N,
                                     transpose, group_size, bits, mode_str, y);
    if (rc != OR_OK) return rc;
    double number = round_store(bias_value, FMT_F32);
    if (!bias && !isfinite(number)) return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] += bias ? load_val(bias, bias_dtype, n) : number;
    return OR_OK;
}

/* qqmm ([RS] qqmm doc comment: x is quantized on the fly, W arrives already
 * quantized; the modes are nvfp4 and mxfp8): y = dequant(quantize(x)) .
 * dequant(W)^T (transpose) or dequant(quantize(x)) . dequant(W).
 * READINGS: x is quantized along its last axis by this file's microscaled
 * rule (the one that quantizes weights) with W's mode, group size and bits;
 * the optional global scales the page passes empty are absent (one level of
 * scales). xhat, if not NULL, receives dequant(quantize(x)) in fp32 (every
 * value is exact there); y is fp64. */
int oracle_qqmm(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                const void* scales, int64_t N, int transpose, int group_size, int bits,
                const char* mode_str, float* xhat, double* y) {
    int mode = parse_mode(mode_str);
    if (mode != MODE_NVFP4 && mode != MODE_MXFP8) return OR_EINVAL;
    if (check_params(mode, group_size, bits, K) != OR_OK) return OR_EINVAL;
    if (check_params(mode, group_size, bits, transpose ? K : N) != OR_OK) return OR_EINVAL;
    if (!x || !wq || !scales || !y || M < 0 || N <= 0 || K <= 0) return OR_EINVAL;
    if (dtype_fmt(x_dtype) < 0) return OR_EINVAL;
    if (M == 0) return OR_OK;
    uint32_t* xq = (uint32_t*)malloc((size_t)(M * K * bits / 32) * sizeof(uint32_t));
    uint8_t* xs = (uint8_t*)malloc((size_t)(M * K / group_size));
    float* xd = (float*)malloc((size_t)(M * K) * sizeof(float));
    int rc = (xq && xs && xd) ? OR_OK : OR_EUNSUP;
    if (rc == OR_OK) rc = oracle_quantize(x, x_dtype, M, K, group_size, bits, mode_str, xq, xs, NULL);
    if (rc == OR_OK) rc = oracle_dequantize(xq, xs, NULL, OR_U8, M, K, group_size, bits, mode_str,
                                            xd, OR_F32);
    if (rc == OR_OK) rc = oracle_quantized_matmul(xd, OR_F32, M, K, wq, scales, NULL, OR_U8, N,
                                                  transpose, group_size, bits, mode_str, y);
    if (rc == OR_OK && xhat) memcpy(xhat, xd, (size_t)(M * K) * sizeof(float));
    free(xq);
    free(xs);
    free(xd);
    return rc;
}

/* gather_qmm ([EMLX] gather_quantized_matmul; [RS] gather_qmm doc and
 * test_gather_qmm): x [B, M, K], W stacked [E, N, K] (transpose) or
 * [E, K, N]; for each r, y[r] = x[lhs[r]] . dequant(W[rhs[r]])^T, with
 * lhs NULL meaning lhs[r] = r. A plain loop in input order, no sorting. */
int oracle_gather_qmm(const void* x, int x_dtype, int64_t B, int64_t M, int64_t K,
                      const uint32_t* wq, const void* scales, const void* biases, int scale_dtype,
                      int64_t E, int64_t N, const uint32_t* lhs, const uint32_t* rhs, int64_t R,
                      int transpose, int group_size, int bits, const char* mode_str, double* y) {
    int mode = parse_mode(mode_str);
    int64_t qrows = transpose ? N : K, qcols = transpose ? K : N;
    if (check_params(mode, group_size, bits, qcols) != OR_OK) return OR_EINVAL;
    if (check_qmm_args(mode, x_dtype, scale_dtype, biases) != OR_OK) return OR_EINVAL;
    if (!x || !wq || !scales || !y || !rhs || B <= 0 || M < 0 || E <= 0 || R < 0) return OR_EINVAL;
    if (!lhs && B != R) return OR_EINVAL;
    for (int64_t r = 0; r < R; ++r) {
        if (rhs[r] >= (uint64_t)E) return OR_EINVAL;
        if (lhs && lhs[r] >= (uint64_t)B) return OR_EINVAL;
    }
    int64_t wwords = qrows * qcols * bits / 32, sgroups = qrows * qcols / group_size;
    int ssz = (mode == MODE_AFFINE) ? (scale_dtype == OR_F32 ? 4 : 2) : 1;
    int xsz = (x_dtype == OR_F32) ? 4 : 2;
    /* each expert's dense weight is built once, on first use */
    float** dense = (float**)calloc((size_t)E, sizeof(float*));
    if (!dense) return OR_EUNSUP;
    int rc = OR_OK;
    for (int64_t r = 0; r < R && rc == OR_OK; ++r) {
        int64_t b = lhs ? (int64_t)lhs[r] : r;
        int64_t e = (int64_t)rhs[r];
        if (!dense[e]) {
            const char* sc = (const char*)scales + e * sgroups * ssz;
            const char* bi = biases ? (const char*)biases + e * sgroups * ssz : NULL;
            dense[e] = dense_weight(wq + e * wwords, sc, bi, scale_dtype, qrows, qcols,
                                    group_size, bits, mode);
            if (!dense[e]) { rc = OR_EUNSUP; break; }
        }
        const char* xb = (const char*)x + b * M * K * xsz;
        qmm_dense(xb, x_dtype, M, K, dense[e], N, transpose, y + r * M * N);
    }
    for (int64_t e = 0; e < E; ++e) free(dense[e]);
    free(dense);
    return rc;
}
