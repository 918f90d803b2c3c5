/*
 * ConvRot W8A8 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct host C for what the ConvRot INT8 linear layer
 * computes.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does, and the
 * product shares no code, header, table or constant with it.
 *
 * Sources (cited by page title and section):
 *   [G71]  "LoRA Training Guide for MOSS-Image", section 7.1 "VRAM Usage
 *          Optimization", subsection "ConvRot INT8": a block-diagonal Hadamard
 *          rotation smooths activation outliers, weights are then quantized
 *          per channel to int8; the forward rotates activations online,
 *          quantizes them row-wise on the fly and dequantizes after the int8
 *          matmul; the opt-in int8 backward routes grad_x through the int8
 *          GEMM, the default dequantizes transiently to bf16.
 *   [PRK]  sd-scripts pull request 2461 (MOSS-Image ConvRot INT8), Summary,
 *          kernels bullet: block-diagonal Hadamard rotation, row-wise int8
 *          quantization, fused int8 GEMM with online activation rotation,
 *          dynamic per-row quantization and a dequantization epilogue.
 *   [PRU]  same pull request, Summary, utils bullet: frozen base, backward
 *          returns grad_x only (bf16 transient dequant or int8 GEMM);
 *          row-chunked quantization of the token embedding; the quantized
 *          embedding stores rows in the rotated basis and its lookup
 *          dequantizes and applies the inverse rotation.
 *   [PRW]  same pull request, Summary, wiring bullet: int8 weight and
 *          per-row scale are split along the rows.
 *   [PRV]  same pull request, Verification: dynamic quantization matches the
 *          published int8 files up to rounding ties, so tie handling matters.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   block = 128, scale = absmax / 127 as an IEEE fp32 division, codes by
 *   round-half-to-even of the IEEE fp32 quotient r / s, clamped to [-127,127];
 *   Sylvester natural-order Hadamard, normalised by 1/sqrt(block) applied to
 *   the rotated values; the rotation sum is carried out exactly (fp64) and the
 *   product with the constant is rounded to fp64 then to fp32; a row whose
 *   scale is 0 (all zero, or a maximum so small that a / 127 underflows) has
 *   codes 0; a row with a NaN or infinite value r (a non-finite input, or an
 *   fp32 overflow of the rotated value) has scale NaN (the canonical quiet NaN,
 *   bits 0x7fc00000) and codes 0, so that it dequantizes to NaN.
 *
 * Floating-point environment: built with -O2 -fno-fast-math -ffp-contract=off,
 * so every expression below rounds exactly as written.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* ------------------------------------------------------------------ */
/* bf16 <-> binary64                                                   */
/* ------------------------------------------------------------------ */

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round-half-to-even of a finite double to an integer-valued double.  The
 * explicit tie rule (not the library's rint) keeps the rule readable. */
static double rne_integer(double t) {
    double f = floor(t);
    double d = t - f; /* exact: f and t are within 1 of each other */
    if (d > 0.5) return f + 1.0;
    if (d < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Single rounding of a double to the nearest bfloat16, ties to even
 * (bf16: 8 significant bits, minimum normal 2^-126, subnormal step 2^-133). */
static uint16_t double_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    (void)frexp(x, &e);                 /* |x| = f * 2^e, f in [0.5, 1) */
    int qexp = e - 8;                   /* quantum 2^(e-8): 8 significant bits */
    if (qexp < -133) qexp = -133;       /* subnormal range */
    double q = ldexp(1.0, qexp);
    double r = rne_integer(x / q) * q;  /* x / q is exact (power-of-two scale) */
    float rf = (float)r;                /* exact unless overflow */
    if (isinf(rf) || fabs(r) > 3.3895313892515355e38) {
        return signbit(x) ? 0xff80 : 0x7f80;
    }
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* O1: Sylvester Hadamard matrix and the normalisation constant        */
/* ------------------------------------------------------------------ */

static int is_pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

/* H_1 = [1];  H_2n = [[H_n, H_n], [H_n, -H_n]]  (natural order). */
int oracle_hadamard(int n, int8_t* H) {
    if (!H || !is_pow2(n) || n > 4096) return ORACLE_EINVAL;
    H[0] = 1;
    for (int m = 1; m < n; m *= 2) {
        for (int i = 0; i < m; ++i) {
            for (int j = 0; j < m; ++j) {
                int8_t h = H[i * n + j];
                H[i * n + (j + m)] = h;
                H[(i + m) * n + j] = h;
                H[(i + m) * n + (j + m)] = (int8_t)(-h);
            }
        }
    }
    return ORACLE_OK;
}

/* 1/sqrt(block) as a binary64 constant.  For block = 4^k it is 2^-k exactly;
 * for block = 2 * 4^k it is fl64(sqrt 2) * 2^-(k+1) (sqrt is correctly rounded
 * and the power-of-two scale is exact).  Block 128 gives 0x1.6a09e667f3bcdp-4;
 * evaluating 1.0 / sqrt(128.0) instead would round twice and land one ulp low. */
double oracle_norm_const(int block) {
    if (!is_pow2(block)) return 0.0;
    int lg = 0;
    while ((1 << lg) < block) ++lg;
    if (lg % 2 == 0) return ldexp(1.0, -lg / 2);
    return ldexp(sqrt(2.0), -(lg + 1) / 2);
}

/* ------------------------------------------------------------------ */
/* O2: rotation of rows by R = diag(H_b / sqrt(b)) along the columns   */
/* ------------------------------------------------------------------ */

/* Error of one binary64 addition s = fl(a + b) (Knuth's TwoSum); nonzero iff
 * the addition rounded.  Used only as the exactness witness. */
static double two_sum_err(double a, double b, double s) {
    double bb = s - a;
    return (a - (s - bb)) + (b - bb);
}

/* r[row][blk*B + j] = fl32( fl64( S_j * c ) ),  S_j = sum_i H[i][j] v[blk*B+i],
 * summed in index order in binary64.  *inexact_rows counts rows in which any
 * partial sum rounded (the exact-sum reading then does not hold for them). */
int oracle_rotate_rows(const uint16_t* x, int64_t rows, int64_t cols, int block,
                       float* r, int64_t* inexact_rows) {
    if (!x || !r || rows < 0 || cols <= 0 || !is_pow2(block) || block > 4096 ||
        cols % block != 0)
        return ORACLE_EINVAL;
    int8_t* H = (int8_t*)malloc((size_t)block * block);
    if (!H) return ORACLE_EINVAL;
    oracle_hadamard(block, H);
    const double c = oracle_norm_const(block);
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t m = 0; m < rows; ++m) {
        const uint16_t* v = x + m * cols;
        int row_inexact = 0;
        for (int64_t b0 = 0; b0 < cols; b0 += block) {
            for (int j = 0; j < block; ++j) {
                double S = 0.0;
                for (int i = 0; i < block; ++i) {
                    double term = (double)H[i * block + j] * bf16_to_double(v[b0 + i]);
                    double s2 = S + term;
                    if (two_sum_err(S, term, s2) != 0.0) row_inexact = 1;
                    S = s2;
                }
                double P = S * c;
                r[m * cols + b0 + j] = (float)P;
            }
        }
        bad += row_inexact;
    }
    free(H);
    if (inexact_rows) *inexact_rows = bad;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O3, O4: symmetric per-row int8 quantization of fp32 rows            */
/* ------------------------------------------------------------------ */

static void quantize_one_row(const float* r, int64_t cols, int8_t* q, float* s_out) {
    float a = 0.0f;
    int finite = 1;
    for (int64_t j = 0; j < cols; ++j) {
        float v = fabsf(r[j]);
        if (!isfinite(v)) finite = 0;
        else if (v > a) a = v;
    }
    /* A NaN or infinite r has no finite scale: the row gets the canonical quiet
     * NaN as its scale and codes 0, and dequantizes to NaN. */
    if (!finite) {
        const uint32_t nan_bits = 0x7fc00000u;
        memcpy(s_out, &nan_bits, sizeof nan_bits);
        for (int64_t j = 0; j < cols; ++j) q[j] = 0;
        return;
    }
    float s = a / 127.0f; /* IEEE binary32 division */
    /* A zero scale dequantizes every code to 0 and leaves r / s undefined: the
     * all-zero row, and a row whose maximum is so small (below 127 * 2^-150)
     * that a / 127 underflows to 0, both get scale 0 and codes 0. */
    if (s == 0.0f) {
        *s_out = 0.0f;
        for (int64_t j = 0; j < cols; ++j) q[j] = 0;
        return;
    }
    *s_out = s;
    for (int64_t j = 0; j < cols; ++j) {
        float t = r[j] / s; /* IEEE binary32 division */
        double k = rne_integer((double)t);
        if (k > 127.0) k = 127.0;
        if (k < -127.0) k = -127.0;
        q[j] = (int8_t)k;
    }
}

int oracle_quantize_rows(const float* r, int64_t rows, int64_t cols, int8_t* q, float* s) {
    if (!r || !q || !s || rows < 0 || cols <= 0) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; ++m) quantize_one_row(r + m * cols, cols, q + m * cols, s + m);
    return ORACLE_OK;
}

/* O5 / O6: rotate then quantize every row; rows are processed chunk by chunk
 * when chunk_rows > 0 (the embedding is quantized that way).  The chunking
 * only bounds the fp32 staging buffer: rows are independent. */
int oracle_rotate_quantize(const uint16_t* x, int64_t rows, int64_t cols, int block,
                           int64_t chunk_rows, int8_t* q, float* s, int64_t* inexact_rows) {
    if (!x || !q || !s || rows < 0 || cols <= 0) return ORACLE_EINVAL;
    if (chunk_rows <= 0 || chunk_rows > rows) chunk_rows = rows > 0 ? rows : 1;
    float* rbuf = (float*)malloc((size_t)chunk_rows * (size_t)cols * sizeof(float));
    if (!rbuf) return ORACLE_EINVAL;
    int64_t bad_total = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += chunk_rows) {
        int64_t n = rows - r0 < chunk_rows ? rows - r0 : chunk_rows;
        int64_t bad = 0;
        int rc = oracle_rotate_rows(x + r0 * cols, n, cols, block, rbuf, &bad);
        if (rc) { free(rbuf); return rc; }
        bad_total += bad;
        oracle_quantize_rows(rbuf, n, cols, q + r0 * cols, s + r0);
    }
    free(rbuf);
    if (inexact_rows) *inexact_rows = bad_total;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O7: int8 x int8 -> int32 contraction along K (both operands K-major) */
/* ------------------------------------------------------------------ */

/* acc[i][n] = sum_k a[rows[i]][k] * b[n][k] for the listed rows of a
 * (rows == NULL: all M rows in order). */
int oracle_gemm_i8_i32(const int8_t* a, const int8_t* b, int64_t M, int64_t N, int64_t K,
                       const int64_t* rows, int64_t nrows, int32_t* acc) {
    if (!a || !b || !acc || M < 0 || N < 0 || K <= 0) return ORACLE_EINVAL;
    if (!rows) nrows = M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        const int8_t* ar = a + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* br = b + n * K;
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int32_t)ar[k] * (int32_t)br[k];
            acc[i * N + n] = s;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O8: dequantization epilogue                                          */
/* ------------------------------------------------------------------ */

/* y[i][n] = bf16( acc[i][n] * s_x[rows[i]] * s_w[n] + bias[n] ), evaluated in
 * binary64 and rounded once to bf16.  bias may be NULL. */
int oracle_dequant_epilogue(const int32_t* acc, int64_t nrows, int64_t N, const float* sx,
                            const int64_t* rows, const float* sw, const uint16_t* bias,
                            uint16_t* y) {
    if (!acc || !sx || !sw || !y || nrows < 0 || N < 0) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[i * N + n] * (double)sx[m] * (double)sw[n];
            if (bias) v = v + bf16_to_double(bias[n]);
            y[i * N + n] = double_to_bf16(v);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Inverse rotation of fp64 rows (R is symmetric and orthogonal, so the */
/* inverse is R itself): out_i = c * sum_j H[j][i] u_j per block.       */
/* ------------------------------------------------------------------ */

static void inverse_rotate_row_to_bf16(const double* u, int64_t cols, int block, const int8_t* H,
                                       double c, uint16_t* out) {
    for (int64_t b0 = 0; b0 < cols; b0 += block) {
        for (int i = 0; i < block; ++i) {
            double S = 0.0;
            for (int j = 0; j < block; ++j) S += (double)H[j * block + i] * u[b0 + j];
            out[b0 + i] = double_to_bf16(c * S);
        }
    }
}

/* ------------------------------------------------------------------ */
/* O9: int8 input gradient                                              */
/* ------------------------------------------------------------------ */

/* Step 1: g[m][n] = fl32( fl32(dY[m][n]) * s_w[n] ), then O3-O4 on each row of
 * g without rotation -> q_g, s_g.  (s_w lies on the contraction axis of
 * dY * W, so it is folded into dY's columns before the per-row quantization.) */
int oracle_bwd_quant_dy(const uint16_t* dy, int64_t M, int64_t N, const float* sw, int8_t* qg,
                        float* sg) {
    if (!dy || !sw || !qg || !sg || M < 0 || N <= 0) return ORACLE_EINVAL;
#pragma omp parallel
    {
        float* g = (float*)malloc((size_t)N * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t n = 0; n < N; ++n) {
                float d = (float)bf16_to_double(dy[m * N + n]);
                g[n] = d * sw[n];
            }
            quantize_one_row(g, N, qg + m * N, sg + m);
        }
        free(g);
    }
    return ORACLE_OK;
}

/* Step 2: acc2[i][k] = sum_n q_g[rows[i]][n] * q_w[n][k]  (contraction along
 * the rows of q_w). */
int oracle_gemm_i8_i32_rows_of_b(const int8_t* qg, const int8_t* qw, int64_t M, int64_t N,
                                 int64_t K, const int64_t* rows, int64_t nrows, int32_t* acc2) {
    if (!qg || !qw || !acc2 || M < 0 || N <= 0 || K <= 0) return ORACLE_EINVAL;
    if (!rows) nrows = M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) {
            int32_t s = 0;
            for (int64_t n = 0; n < N; ++n) s += (int32_t)qg[m * N + n] * (int32_t)qw[n * K + k];
            acc2[i * K + k] = s;
        }
    }
    return ORACLE_OK;
}

/* Step 3: dX[i][blk] = bf16( c * sum_j H[j][.] * (acc2[i][j] * s_g[rows[i]]) ). */
int oracle_bwd_int8_epilogue(const int32_t* acc2, int64_t nrows, int64_t K, const float* sg,
                             const int64_t* rows, int block, uint16_t* dx) {
    if (!acc2 || !sg || !dx || nrows < 0 || K <= 0 || !is_pow2(block) || K % block)
        return ORACLE_EINVAL;
    int8_t* H = (int8_t*)malloc((size_t)block * block);
    oracle_hadamard(block, H);
    double c = oracle_norm_const(block);
#pragma omp parallel
    {
        double* u = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t m = rows ? rows[i] : i;
            for (int64_t k = 0; k < K; ++k) u[k] = (double)acc2[i * K + k] * (double)sg[m];
            inverse_rotate_row_to_bf16(u, K, block, H, c, dx + i * K);
        }
        free(u);
    }
    free(H);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O10: bf16 transient-dequant input gradient                           */
/* ------------------------------------------------------------------ */

/* W_hat[n][blk] = bf16( c * sum_j H[j][.] * (q_w[n][j] * s_w[n]) ): the
 * dequantized weight brought back to the unrotated basis, rounded to bf16. */
int oracle_dequant_weight(const int8_t* qw, const float* sw, int64_t N, int64_t K, int block,
                          uint16_t* what) {
    if (!qw || !sw || !what || N < 0 || K <= 0 || !is_pow2(block) || K % block)
        return ORACLE_EINVAL;
    int8_t* H = (int8_t*)malloc((size_t)block * block);
    oracle_hadamard(block, H);
    double c = oracle_norm_const(block);
#pragma omp parallel
    {
        double* u = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) u[k] = (double)qw[n * K + k] * (double)sw[n];
            inverse_rotate_row_to_bf16(u, K, block, H, c, what + n * K);
        }
        free(u);
    }
    free(H);
    return ORACLE_OK;
}

/* dX[i][k] = bf16( sum_n dY[rows[i]][n] * W_hat[n][k] ), summed in binary64. */
int oracle_bf16_gemm_dx(const uint16_t* dy, const uint16_t* what, int64_t M, int64_t N, int64_t K,
                        const int64_t* rows, int64_t nrows, uint16_t* dx) {
    if (!dy || !what || !dx || M < 0 || N <= 0 || K <= 0) return ORACLE_EINVAL;
    if (!rows) nrows = M;
#pragma omp parallel
    {
        double* acc = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t m = rows ? rows[i] : i;
            for (int64_t k = 0; k < K; ++k) acc[k] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double d = bf16_to_double(dy[m * N + n]);
                const uint16_t* wr = what + n * K;
                for (int64_t k = 0; k < K; ++k) acc[k] += d * bf16_to_double(wr[k]);
            }
            for (int64_t k = 0; k < K; ++k) dx[i * K + k] = double_to_bf16(acc[k]);
        }
        free(acc);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O11: quantized embedding lookup                                      */
/* ------------------------------------------------------------------ */

/* out[t] = bf16( (s_E[id] * q_E[id]) * R ) -- rows are stored in the rotated
 * basis, so the lookup dequantizes and applies the inverse rotation.  An id
 * outside [0, V) yields a zero row and is counted. */
int oracle_embedding_lookup(const int32_t* ids, int64_t T, const int8_t* qe, const float* se,
                            int64_t V, int64_t D, int block, uint16_t* out, int64_t* oob) {
    if (!ids || !qe || !se || !out || T < 0 || V <= 0 || D <= 0 || !is_pow2(block) || D % block)
        return ORACLE_EINVAL;
    int8_t* H = (int8_t*)malloc((size_t)block * block);
    oracle_hadamard(block, H);
    double c = oracle_norm_const(block);
    int64_t bad = 0;
#pragma omp parallel reduction(+ : bad)
    {
        double* u = (double*)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            int64_t id = ids[t];
            if (id < 0 || id >= V) {
                for (int64_t k = 0; k < D; ++k) out[t * D + k] = 0;
                bad += 1;
                continue;
            }
            for (int64_t k = 0; k < D; ++k) u[k] = (double)qe[id * D + k] * (double)se[id];
            inverse_rotate_row_to_bf16(u, D, block, H, c, out + t * D);
        }
        free(u);
    }
    free(H);
    if (oob) *oob = bad;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* O13: LoRA branch of the forward ([G71]: the quantized layers stay    */
/* LoRA-trainable and the LoRA branch receives the unrotated input)     */
/* ------------------------------------------------------------------ */

/* Down projection, as a bf16 Linear: xa[i][r] = bf16( sum_k x[m][k] * A[r][k] )
 * for the listed rows m = rows[i] (rows == NULL: all M rows), the sum taken in
 * index order in binary64.  A is [R, K]. */
int oracle_lora_down(const uint16_t* x, int64_t M, int64_t K, const uint16_t* A, int64_t R,
                     const int64_t* rows, int64_t nrows, uint16_t* xa) {
    if (!x || !A || !xa || M < 0 || K <= 0 || R <= 0) return ORACLE_EINVAL;
    if (!rows) nrows = M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t r = 0; r < R; ++r) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += bf16_to_double(x[m * K + k]) * bf16_to_double(A[r * K + k]);
            xa[i * R + r] = double_to_bf16(s);
        }
    }
    return ORACLE_OK;
}

/* Forward output with the LoRA branch:
 *   y[i][n] = bf16( acc[i][n] * s_x[m] * s_w[n] + bias[n]
 *                   + scale * sum_r xa[i][r] * B[n][r] ),   m = rows[i],
 * evaluated in binary64 and rounded once.  B is [N, R]; bias may be NULL. */
int oracle_lora_epilogue(const int32_t* acc, int64_t nrows, int64_t N, const float* sx,
                         const int64_t* rows, const float* sw, const uint16_t* bias,
                         const uint16_t* xa, const uint16_t* B, int64_t R, double scale,
                         uint16_t* y) {
    if (!acc || !sx || !sw || !xa || !B || !y || nrows < 0 || N < 0 || R <= 0)
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t n = 0; n < N; ++n) {
            double l = 0.0;
            for (int64_t r = 0; r < R; ++r)
                l += bf16_to_double(xa[i * R + r]) * bf16_to_double(B[n * R + r]);
            double v = (double)acc[i * N + n] * (double)sx[m] * (double)sw[n];
            if (bias) v = v + bf16_to_double(bias[n]);
            y[i * N + n] = double_to_bf16(v + scale * l);
        }
    }
    return ORACLE_OK;
}

/* Threads the OpenMP loops above use (reported with oracle timings), and a
 * setter so that a timing can run single-threaded; results do not depend on it. */
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* Rounding helpers exported for the oracle's own pins. */
uint16_t oracle_double_to_bf16(double x) { return double_to_bf16(x); }
double oracle_rne_integer(double t) { return rne_integer(t); }
