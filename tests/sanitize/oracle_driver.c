/* oracle_driver.c -- runs every entry point of the CPU oracle
 * (oracle/qlin_oracle.c) on small inputs, each buffer allocated at exactly
 * the size the call may touch, so that a build with
 * -fsanitize=address,undefined reports any out-of-bounds access or undefined
 * behaviour. It checks return codes only; the values are checked by the
 * oracle pins. Test infrastructure, like the oracle itself. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int group_size,
                    int bits, const char* mode, uint32_t* wq, void* scales, void* biases);
int oracle_dequantize(const uint32_t* wq, const void* scales, const void* biases, int scale_dtype,
                      int64_t rows, int64_t cols, int group_size, int bits, const char* mode,
                      void* out, int out_dtype);
int oracle_quantized_matmul(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                            const void* scales, const void* biases, int scale_dtype, int64_t N,
                            int transpose, int group_size, int bits, const char* mode, double* y);
int oracle_quantized_dense(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                           const void* scales, const void* biases, int scale_dtype, int64_t N,
                           int transpose, int group_size, int bits, const char* mode,
                           const void* bias, int bias_dtype, double bias_value, double* y);
int oracle_qqmm(const void* x, int x_dtype, int64_t M, int64_t K, const uint32_t* wq,
                const void* scales, int64_t N, int transpose, int group_size, int bits,
                const char* mode, float* xhat, double* y);
int oracle_gather_qmm(const void* x, int x_dtype, int64_t B, int64_t M, int64_t K,
                      const uint32_t* wq, const void* scales, const void* biases, int scale_dtype,
                      int64_t E, int64_t N, const uint32_t* lhs, const uint32_t* rhs, int64_t R,
                      int transpose, int group_size, int bits, const char* mode, double* y);

enum { F32 = 0, F16 = 1, BF16 = 2, U8 = 3 };

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform(void) {   /* xorshift64*, in [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static int fails = 0;
static void expect(int rc, int want, const char* what) {
    if (rc != want) {
        fprintf(stderr, "%s: rc %d, expected %d\n", what, rc, want);
        ++fails;
    }
}

/* a [n] array of dtype dt with values ~ scale * U(-1, 1); bf16 by truncation */
static void* make(int64_t n, int dt, double scale) {
    if (dt == F32) {
        float* p = malloc((size_t)n * sizeof *p);
        for (int64_t i = 0; i < n; ++i) p[i] = (float)(scale * uniform());
        return p;
    }
    uint16_t* p = malloc((size_t)n * sizeof *p);
    for (int64_t i = 0; i < n; ++i) {
        float f = (float)(scale * uniform());
        uint32_t u;
        memcpy(&u, &f, 4);
        p[i] = (uint16_t)(u >> 16);   /* bf16 bit pattern */
    }
    return p;
}

static size_t dt_size(int dt) { return dt == F32 ? 4 : (dt == U8 ? 1 : 2); }

static void run_mode(const char* mode, int bits, int g, int wdt) {
    const int affine = strcmp(mode, "affine") == 0;
    const int sdt = affine ? wdt : U8;
    const int64_t N = 5, K = 256, M = 3, G = K / g, words = K * bits / 32;
    char what[96];
    snprintf(what, sizeof what, "%s b%d g%d dtype %d", mode, bits, g, wdt);

    /* quantize W [N, K], dequantize it */
    void* w = make(N * K, wdt, 0.05);
    uint32_t* wq = malloc((size_t)(N * words) * sizeof *wq);
    void* sc = malloc((size_t)(N * G) * dt_size(sdt));
    void* bi = affine ? malloc((size_t)(N * G) * dt_size(sdt)) : NULL;
    expect(oracle_quantize(w, wdt, N, K, g, bits, mode, wq, sc, bi), 0, what);
    float* deq = malloc((size_t)(N * K) * sizeof *deq);
    expect(oracle_dequantize(wq, sc, bi, sdt, N, K, g, bits, mode, deq, F32), 0, what);
    uint16_t* deqb = malloc((size_t)(N * K) * sizeof *deqb);
    expect(oracle_dequantize(wq, sc, bi, sdt, N, K, g, bits, mode, deqb, BF16), 0, what);

    /* y = x . W^T and the dense layer (bias vector, then a number) */
    void* x = make(M * K, wdt == F32 ? F32 : BF16, 1.0);
    const int xdt = wdt == F32 ? F32 : BF16;
    double* y = malloc((size_t)(M * N) * sizeof *y);
    expect(oracle_quantized_matmul(x, xdt, M, K, wq, sc, bi, sdt, N, 1, g, bits, mode, y), 0, what);
    void* bias = make(N, F32, 1.0);
    expect(oracle_quantized_dense(x, xdt, M, K, wq, sc, bi, sdt, N, 1, g, bits, mode, bias, F32, 0.0, y),
           0, what);
    expect(oracle_quantized_dense(x, xdt, M, K, wq, sc, bi, sdt, N, 1, g, bits, mode, NULL, F32, -0.5, y),
           0, what);

    /* [in, out] layout: W2 [K2 = 8, N2 = 256], y2 = x2 [M, 8] . W2 */
    const int64_t K2 = 8, N2 = 256, G2 = N2 / g, words2 = N2 * bits / 32;
    void* w2 = make(K2 * N2, wdt, 0.05);
    uint32_t* wq2 = malloc((size_t)(K2 * words2) * sizeof *wq2);
    void* sc2 = malloc((size_t)(K2 * G2) * dt_size(sdt));
    void* bi2 = affine ? malloc((size_t)(K2 * G2) * dt_size(sdt)) : NULL;
    expect(oracle_quantize(w2, wdt, K2, N2, g, bits, mode, wq2, sc2, bi2), 0, what);
    void* x2 = make(M * K2, xdt, 1.0);
    double* y2 = malloc((size_t)(M * N2) * sizeof *y2);
    expect(oracle_quantized_matmul(x2, xdt, M, K2, wq2, sc2, bi2, sdt, N2, 0, g, bits, mode, y2), 0, what);

    /* gather: E = 3 experts [3, N, K], x [B = 2, Mg = 2, K], R = 4 index rows */
    const int64_t E = 3, B = 2, Mg = 2, R = 4;
    void* we = make(E * N * K, wdt, 0.05);
    uint32_t* wqe = malloc((size_t)(E * N * words) * sizeof *wqe);
    void* sce = malloc((size_t)(E * N * G) * dt_size(sdt));
    void* bie = affine ? malloc((size_t)(E * N * G) * dt_size(sdt)) : NULL;
    expect(oracle_quantize(we, wdt, E * N, K, g, bits, mode, wqe, sce, bie), 0, what);
    void* xg = make(B * Mg * K, xdt, 1.0);
    uint32_t lhs[4] = {1, 0, 1, 1}, rhs[4] = {2, 0, 1, 2};
    double* yg = malloc((size_t)(R * Mg * N) * sizeof *yg);
    expect(oracle_gather_qmm(xg, xdt, B, Mg, K, wqe, sce, bie, sdt, E, N, lhs, rhs, R, 1, g, bits, mode, yg),
           0, what);
    expect(oracle_gather_qmm(xg, xdt, B, Mg, K, wqe, sce, bie, sdt, E, N, NULL, rhs, R, 1, g, bits, mode, yg),
           1, "gather without lhs and B != R");

    /* qqmm (x quantized on the fly) for the modes that have it */
    if (!strcmp(mode, "mxfp8") || !strcmp(mode, "nvfp4")) {
        float* xhat = malloc((size_t)(M * K) * sizeof *xhat);
        expect(oracle_qqmm(x, xdt, M, K, wq, sc, N, 1, g, bits, mode, xhat, y), 0, what);
        free(xhat);
    }

    /* rejected arguments touch nothing */
    expect(oracle_quantize(w, wdt, N, K, g, bits, "bogus", wq, sc, bi), 1, "bad mode");
    expect(oracle_quantize(w, wdt, N, K - 1, g, bits, mode, wq, sc, bi), 1, "K not a multiple of the group");

    free(w); free(wq); free(sc); free(bi); free(deq); free(deqb); free(x); free(y); free(bias);
    free(w2); free(wq2); free(sc2); free(bi2); free(x2); free(y2);
    free(we); free(wqe); free(sce); free(bie); free(xg); free(yg);
}

int main(void) {
    const int dts[2] = {F32, BF16};
    for (int d = 0; d < 2; ++d) {
        run_mode("affine", 2, 32, dts[d]);
        run_mode("affine", 4, 64, dts[d]);
        run_mode("affine", 8, 128, dts[d]);
        run_mode("mxfp4", 4, 32, dts[d]);
        run_mode("mxfp8", 8, 32, dts[d]);
        run_mode("nvfp4", 4, 16, dts[d]);
    }
    if (fails) {
        fprintf(stderr, "%d unexpected return codes\n", fails);
        return 1;
    }
    printf("oracle driver: all entry points ran\n");
    return 0;
}
