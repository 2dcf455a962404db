/*
 * hkg_oracle.c -- CPU oracle for the dense BF16 GEMM  C = A * B^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or helper with the
 * HIP library: it is built by gcc from this one file.
 *
 * What it computes (the plain definition, written out):
 *   The operation is the NT-layout projection GEMM described on the FlyDSL
 *   "prebuilt_kernels_guide" page (section 3.1, Preshuffle GEMM:
 *   C[M,N] = A[M,K] @ B[N,K]^T) and on the "FlyDSL in PyTorch" blog page
 *   (section "Dense GEMM": BF16 NT shapes, projection and feed-forward
 *   layers).  A is M x K row-major, B is N x K row-major (K contiguous in
 *   both), C is M x N row-major.
 *
 *     S[i][j]    = sum over k = 0..K-1 (ascending) of  a(i,k) * b(j,k)   in fp64
 *     absS[i][j] = sum over k of |a(i,k) * b(j,k)|                        in fp64
 *     C[i][j]    = bf16 nearest-even rounding of S[i][j], applied once, f64 -> bf16
 *
 *   A bf16 x bf16 product has at most 16 significant bits, so every product
 *   is exact in fp64; the only fp64 roundings are in the running sums.
 *   Round-to-nearest-even as the bf16 output rounding follows the same
 *   FlyDSL guide (section 1.1, LayerNorm, "bf16 handling": RNE pack in
 *   software on gfx942, the hardware cvt_pk_bf16_f32 instruction on gfx950).
 *
 * Build:  gcc -O2 -fopenmp -shared -fPIC hkg_oracle.c -o libhkg_oracle.so -lm
 * (no -ffast-math, no -ffp-contract games: the k order is the loop order).
 *
 * Pins (checked by the CPU test suite, independent of this code):
 *   bf16 conversion: all 65536 bit patterns round-trip; nearest-even ties;
 *   agreement with an integer float32->bf16 rounding on float32 inputs and
 *   with torch's float32->bfloat16 conversion.
 *   GEMM: all-ones (C = K), identity on either side (C = B^T, C = A),
 *   small-integer inputs against exact int64 products, exact-rational brute
 *   force on tiny shapes, and the fp64 summation error bound.
 *   MXFP8: every E4M3 and E8M0 code against torch's float8_e4m3fn and
 *   float8_e8m0fnu conversions; all-ones with unit scales (C = K); scale
 *   changes multiply exactly by powers of two; exact rationals on tiny shapes.
 *   MXFP4: the eight E2M1 magnitudes of the format definition; every E2M1
 *   code through its E4M3 equivalent and torch's float8_e4m3fn conversion;
 *   the MXFP4 product equal to the MXFP8 product of the same values (an
 *   independent decoder); all-ones with unit scales (C = K); scale changes
 *   multiply exactly by powers of two; exact rationals on tiny shapes.
 *   Layouts: every (A, B) layout with padded leading dimensions equals the
 *   dense oracle on the logical matrices, and padding (filled with NaN
 *   patterns) is never read.
 *   Grouped GEMM: one expert equals the dense oracle; all-ones activations
 *   against expert weights filled with (g + 1) give C = K (g + 1) exactly in
 *   each expert's rows (boundaries, empty experts); permuting the experts
 *   permutes the rows; exact rationals on tiny shapes.
 *   Epilogue: bias through all-ones products (C = K + b, exact), ReLU's
 *   definition, the odd parts SiLU(x) - SiLU(-x) = x and GELU(x) - GELU(-x) = x,
 *   the closed form sigmoid(ln 3) = 3/4, the normal quantile Phi(1.959963985)
 *   = 0.975, and slopes 1/2 at 0.
 */
#define _DEFAULT_SOURCE  /* M_SQRT1_2 under -std=c11 */
#include <stdint.h>
#include <math.h>
#include <string.h>
#include <stdlib.h>
#include <omp.h>

/* ---- bf16 <-> f64 from the format's definition ------------------------- */
/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.          */

double hkg_oracle_bf16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int f = bits & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = f ? NAN : INFINITY;
    else if (e == 0)                     /* subnormal: 0.f * 2^-126 */
        mag = ldexp((double)f / 128.0, -126);
    else                                 /* normal: 1.f * 2^(e-127) */
        mag = ldexp(1.0 + (double)f / 128.0, e - 127);
    return sign ? -mag : mag;
}

/* Round a finite or infinite double to the nearest bf16, ties to even. */
uint16_t hkg_oracle_bf16_rne(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (isinf(ax))
        return sign | 0x7F80;
    if (ax == 0.0)
        return sign;
    int e;
    frexp(ax, &e);                  /* ax = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                  /* ax = (2m) * 2^E, 2m in [1, 2) */
    if (E < -126)
        E = -126;                   /* bf16 subnormal range: fixed quantum */
    double q = ldexp(1.0, E - 7);   /* spacing of bf16 values near ax */
    double n = rint(ax / q);        /* ax/q is exact (power-of-two scale); rint = nearest, ties to even */
    double y = n * q;               /* exact */
    if (y >= ldexp(1.0, 128))       /* past the largest finite bf16 */
        return sign | 0x7F80;
    /* y is a bf16 value, hence exactly a float32 whose low 16 bits are 0 */
    float yf = (float)y;
    uint32_t u;
    memcpy(&u, &yf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* Table of the 65536 bf16 values, built from the definition above. */
static double g_val[65536];
static int g_val_ready = 0;

static void build_table(void)
{
    if (g_val_ready)
        return;
#pragma omp critical(hkg_oracle_table)
    {
        if (!g_val_ready) {
            for (int b = 0; b < 65536; ++b)
                g_val[b] = hkg_oracle_bf16_value((uint16_t)b);
            __atomic_store_n(&g_val_ready, 1, __ATOMIC_RELEASE);
        }
    }
}

/* One output element: the fp64 sum over k ascending, and the sum of |products|. */
static void dot_one(const uint16_t* a_row, const uint16_t* b_row, int64_t K,
                    double* s_out, double* abs_out)
{
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = g_val[a_row[k]] * g_val[b_row[k]];
        s += p;
        sa += fabs(p);
    }
    *s_out = s;
    *abs_out = sa;
}

/*
 * Rows [row_begin, row_end) of C = A * B^T.  Outputs are (row_end-row_begin) x N,
 * row-major.  S and absS may be NULL.  nthreads <= 0 uses the OpenMP default.
 */
void hkg_oracle_gemm_rows(const uint16_t* A, const uint16_t* B,
                          int64_t M, int64_t N, int64_t K,
                          int64_t row_begin, int64_t row_end,
                          uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    build_table();
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s, sa;
            dot_one(A + i * K, B + j * K, K, &s, &sa);
            int64_t o = (i - row_begin) * N + j;
            C[o] = hkg_oracle_bf16_rne(s);
            if (S)
                S[o] = s;
            if (absS)
                absS[o] = sa;
        }
    }
}

/* Selected elements (ii[t], jj[t]), t < count, of C = A * B^T. */
void hkg_oracle_gemm_entries(const uint16_t* A, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K,
                             const int64_t* ii, const int64_t* jj, int64_t count,
                             uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    (void)N;
    build_table();
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t t = 0; t < count; ++t) {
        double s, sa;
        dot_one(A + ii[t] * K, B + jj[t] * K, K, &s, &sa);
        C[t] = hkg_oracle_bf16_rne(s);
        if (S)
            S[t] = s;
        if (absS)
            absS[t] = sa;
    }
}

int hkg_oracle_max_threads(void) { return omp_get_max_threads(); }

/* ---- operand layouts and leading dimensions --------------------------------
 * The FlyDSL-in-PyTorch blog (section "Dense GEMM") measures all four
 * operand layouts; the FlyDSL "Prebuilt kernels guide" works with strided
 * operands.  Read plainly: the logical operands stay A (M x K) and B (N x K)
 * and C = A * B^T as above; only where element (i, k) lives changes:
 *   A row layout (a_col = 0): a(i,k) = A[i * lda + k]   (K contiguous, lda >= K)
 *   A column layout (a_col = 1): a(i,k) = A[k * lda + i] (stored K x M, lda >= M)
 *   B row layout (b_col = 0): b(j,k) = B[j * ldb + k]   (stored N x K, ldb >= K)
 *   B column layout (b_col = 1): b(j,k) = B[k * ldb + j] (stored K x N, ldb >= N)
 *   C[i * ldc + j] for 0 <= j < N, ldc >= N (elements in between untouched).
 * Sums and rounding exactly as hkg_oracle_gemm_rows; C is written here as a
 * dense (row_end - row_begin) x N block like the other row functions.
 */
void hkg_oracle_gemm_layout_rows(const uint16_t* A, int64_t lda, int a_col, const uint16_t* B, int64_t ldb,
                                 int b_col, int64_t M, int64_t N, int64_t K, int64_t row_begin, int64_t row_end,
                                 uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    build_table();
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint16_t a = a_col ? A[k * lda + i] : A[i * lda + k];
                const uint16_t b = b_col ? B[k * ldb + j] : B[j * ldb + k];
                double p = g_val[a] * g_val[b];
                s = s + p;
                sa = sa + fabs(p);
            }
            int64_t o = (i - row_begin) * N + j;
            C[o] = hkg_oracle_bf16_rne(s);
            if (S)
                S[o] = s;
            if (absS)
                absS[o] = sa;
        }
    }
}

/* ---- grouped GEMM ----------------------------------------------------------
 * The FlyDSL-in-PyTorch blog (grouped GEMM section, mixture of experts): the
 * activations of all experts concatenated as A[sum of M_g, K], one weight per
 * expert, and offsets marking where each expert's rows end.  Read with this
 * library's NT convention (each expert's weight N x K, K contiguous, stacked
 * as B[G][N][K]) and offs[g] the end (exclusive) of expert g's rows, expert g
 * owns rows [offs[g-1], offs[g]) (offs[-1] = 0), and
 *     C[i][j] = bf16( sum over k of A[i][k] * B[g][j][k] )   for i in group g,
 * i.e. the dense definition above with the row's own expert weight.  Offsets
 * are non-decreasing; rows at or past offs[G-1] belong to no expert.
 */
static int64_t group_of_row(const int32_t* offs, int64_t G, int64_t i)
{
    /* first g with offs[g] > i; G if none */
    int64_t lo = 0, hi = G;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if ((int64_t)offs[mid] > i)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

/* Rows [row_begin, row_end) of the grouped product; outputs as in
 * hkg_oracle_gemm_rows.  Rows of no expert give C = 0, S = absS = 0 and
 * return value 0 for the caller to know; 1 otherwise (all rows grouped). */
int hkg_oracle_grouped_gemm_rows(const uint16_t* A, const uint16_t* B, const int32_t* offs, int64_t G,
                                 int64_t M, int64_t N, int64_t K, int64_t row_begin, int64_t row_end,
                                 uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    build_table();
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int all_grouped = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(&& : all_grouped)
    for (int64_t i = row_begin; i < row_end; ++i) {
        const int64_t g = group_of_row(offs, G, i);
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0, sa = 0.0;
            if (g < G)
                dot_one(A + i * K, B + (g * N + j) * K, K, &s, &sa);
            int64_t o = (i - row_begin) * N + j;
            C[o] = hkg_oracle_bf16_rne(s);
            if (S)
                S[o] = s;
            if (absS)
                absS[o] = sa;
        }
        if (g >= G)
            all_grouped = 0;
    }
    return all_grouped;
}

/* ---- fused epilogue ------------------------------------------------------
 * The FlyDSL "prebuilt_kernels_guide" page (section 3.1, Preshuffle GEMM,
 * parameter `epilogue`) lists the fused epilogues "none", "bias",
 * "bias_relu", "bias_silu" and "bias_gelu", with the bias one value per
 * output column in the output dtype.  Read plainly, on the unrounded sum S:
 *
 *   x = S[i][j] + bias[j]                   (bf16 bias, widened exactly)
 *   y = x                                   bias
 *       x if x > 0, else +0                 bias_relu
 *       x * sigmoid(x) = x / (1 + e^-x)     bias_silu
 *       x * Phi(x) = x * erfc(-x/sqrt 2)/2  bias_gelu (Phi: standard normal
 *                                            CDF; erfc keeps the left tail
 *                                            accurate)
 *   C[i][j] = bf16 nearest-even rounding of y, once.
 *
 * "none" is the plain GEMM: y = S, bias unused.  All in fp64.
 */
enum { HKG_ORACLE_EPI_NONE = 0, HKG_ORACLE_EPI_BIAS = 1, HKG_ORACLE_EPI_BIAS_RELU = 2,
       HKG_ORACLE_EPI_BIAS_SILU = 3, HKG_ORACLE_EPI_BIAS_GELU = 4 };

double hkg_oracle_activation(double x, int epi)
{
    switch (epi) {
    case HKG_ORACLE_EPI_BIAS_RELU:
        return x > 0.0 ? x : 0.0;
    case HKG_ORACLE_EPI_BIAS_SILU:
        return x / (1.0 + exp(-x));
    case HKG_ORACLE_EPI_BIAS_GELU:
        return 0.5 * x * erfc(-x * M_SQRT1_2);
    default:
        return x;
    }
}

/*
 * count results with sums S[t]; element t belongs to output column cols[t]
 * (cols NULL: column t mod N, i.e. whole rows of an N-column C).  Writes the
 * unrounded epilogue value Y[t] (may be NULL) and its bf16 rounding C[t].
 * Returns -1 for an unknown epilogue, else 0.
 */
int hkg_oracle_epilogue(const double* S, const uint16_t* bias, int64_t count, int64_t N,
                        const int64_t* cols, int epi, double* Y, uint16_t* C)
{
    if (epi < HKG_ORACLE_EPI_NONE || epi > HKG_ORACLE_EPI_BIAS_GELU)
        return -1;
    for (int64_t t = 0; t < count; ++t) {
        double y = S[t];
        if (epi != HKG_ORACLE_EPI_NONE) {
            const int64_t j = cols ? cols[t] : t % N;
            y = hkg_oracle_activation(S[t] + hkg_oracle_bf16_value(bias[j]), epi);
        }
        if (Y)
            Y[t] = y;
        C[t] = hkg_oracle_bf16_rne(y);
    }
    return 0;
}


/* ---- MXFP8 GEMM ----------------------------------------------------------
 * The "FlyDSL in PyTorch" blog page (section on MXFP) describes the block-
 * scaled GEMM: operands FP8 E4M3, one E8M0 scale per 32 values along the
 * reduction axis (BlockWise1x32), fp32 accumulation, bf16 output, K a
 * multiple of 128.  Written out:
 *
 *   a(i,k) = e4m3(A[i][k]) * e8m0(SA[i][k / 32]),  b(j,k) likewise with SB
 *   S[i][j] = sum over k ascending of a(i,k) * b(j,k)   (fp64)
 *   C[i][j] = bf16 nearest-even rounding of S[i][j], once
 *
 * Layouts: A is M x K bytes and B N x K bytes (K contiguous), SA is M x K/32
 * and SB N x K/32 bytes (one row of scales per operand row).
 * E4M3 (OCP "e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 fraction bits;
 * exponent field 0 holds subnormals 0.f * 2^-6; no infinities; S.1111.111
 * is NaN; the largest finite value is 448.  E8M0: an unsigned exponent,
 * value 2^(e - 127); 0xFF is NaN.
 * A product of two E4M3 values has at most 8 significant bits and the
 * scales are powers of two in [2^-127, 2^127], so every scaled product is
 * exact in fp64; only the running sums round.
 */
double hkg_oracle_e4m3_value(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int f = bits & 0x7;
    double mag;
    if (e == 0xF && f == 0x7)
        mag = NAN;
    else if (e == 0)                     /* subnormal: 0.f * 2^-6 */
        mag = ldexp((double)f / 8.0, -6);
    else                                 /* normal: 1.f * 2^(e-7) */
        mag = ldexp(1.0 + (double)f / 8.0, e - 7);
    return sign ? -mag : mag;
}

double hkg_oracle_e8m0_value(uint8_t bits)
{
    return bits == 0xFF ? NAN : ldexp(1.0, (int)bits - 127);
}

static double g_e4m3[256];
static int g_e4m3_ready = 0;

static void build_e4m3_table(void)
{
    if (g_e4m3_ready)
        return;
#pragma omp critical(hkg_oracle_e4m3_table)
    {
        if (!g_e4m3_ready) {
            for (int b = 0; b < 256; ++b)
                g_e4m3[b] = hkg_oracle_e4m3_value((uint8_t)b);
            __atomic_store_n(&g_e4m3_ready, 1, __ATOMIC_RELEASE);
        }
    }
}

static void mx_dot_one(const uint8_t* a_row, const uint8_t* sa_row, const uint8_t* b_row,
                       const uint8_t* sb_row, int64_t K, double* s_out, double* abs_out)
{
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = (g_e4m3[a_row[k]] * hkg_oracle_e8m0_value(sa_row[k / 32])) *
                   (g_e4m3[b_row[k]] * hkg_oracle_e8m0_value(sb_row[k / 32]));
        s += p;
        sa += fabs(p);
    }
    *s_out = s;
    *abs_out = sa;
}

/* Rows [row_begin, row_end) of the MXFP8 product; outputs as in
 * hkg_oracle_gemm_rows.  K must be a multiple of 32. */
void hkg_oracle_mx_gemm_rows(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                             int64_t M, int64_t N, int64_t K, int64_t row_begin, int64_t row_end,
                             uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    build_e4m3_table();
    const int64_t KB = K / 32;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s, sa;
            mx_dot_one(A + i * K, SA + i * KB, B + j * K, SB + j * KB, K, &s, &sa);
            int64_t o = (i - row_begin) * N + j;
            C[o] = hkg_oracle_bf16_rne(s);
            if (S)
                S[o] = s;
            if (absS)
                absS[o] = sa;
        }
    }
}

/* Selected elements (ii[t], jj[t]) of the MXFP8 product. */
void hkg_oracle_mx_gemm_entries(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                                int64_t M, int64_t N, int64_t K, const int64_t* ii, const int64_t* jj,
                                int64_t count, uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    (void)N;
    build_e4m3_table();
    const int64_t KB = K / 32;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t t = 0; t < count; ++t) {
        double s, sa;
        mx_dot_one(A + ii[t] * K, SA + ii[t] * KB, B + jj[t] * K, SB + jj[t] * KB, K, &s, &sa);
        C[t] = hkg_oracle_bf16_rne(s);
        if (S)
            S[t] = s;
        if (absS)
            absS[t] = sa;
    }
}


/* ---- MXFP4 GEMM ----------------------------------------------------------
 * The same MXFP section of the "FlyDSL in PyTorch" blog page names the
 * packed-FP4 form: E2M1 operands stored two per byte, one E8M0 scale per 32
 * values along the reduction axis, fp32 accumulation, bf16 output.  Written
 * out as for MXFP8:
 *
 *   a(i,k) = e2m1(nibble k of row i of A) * e8m0(SA[i][k / 32]),  b likewise
 *   S[i][j] = sum over k ascending of a(i,k) * b(j,k)   (fp64)
 *   C[i][j] = bf16 nearest-even rounding of S[i][j], once
 *
 * Layouts: A is M x K/2 bytes and B N x K/2 bytes; byte c of a row holds
 * element 2c in its low nibble and element 2c + 1 in its high nibble.  SA is
 * M x K/32 and SB N x K/32 bytes.
 * E2M1 (OCP MX): 1 sign bit, 2 exponent bits (bias 1), 1 fraction bit;
 * exponent field 0 holds the subnormals 0.f * 2^0 (0 and 0.5), otherwise
 * 1.f * 2^(e - 1); no infinities or NaNs; the largest value is 6.
 * Every scaled product is exact in fp64; only the running sums round.
 */
double hkg_oracle_e2m1_value(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int f = code & 1;
    double mag = e == 0 ? (double)f / 2.0                        /* subnormal: 0.f * 2^0 */
                        : ldexp(1.0 + (double)f / 2.0, e - 1);    /* normal: 1.f * 2^(e-1) */
    return sign ? -mag : mag;
}

static double mx4_element(const uint8_t* row, int64_t k)
{
    const uint8_t byte = row[k / 2];
    return hkg_oracle_e2m1_value((uint8_t)((k & 1) ? byte >> 4 : byte & 0xF));
}

static void mx4_dot_one(const uint8_t* a_row, const uint8_t* sa_row, const uint8_t* b_row,
                        const uint8_t* sb_row, int64_t K, double* s_out, double* abs_out)
{
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = (mx4_element(a_row, k) * hkg_oracle_e8m0_value(sa_row[k / 32])) *
                   (mx4_element(b_row, k) * hkg_oracle_e8m0_value(sb_row[k / 32]));
        s += p;
        sa += fabs(p);
    }
    *s_out = s;
    *abs_out = sa;
}

/* Rows [row_begin, row_end) of the MXFP4 product; outputs as in
 * hkg_oracle_gemm_rows.  K must be a multiple of 32. */
void hkg_oracle_mx4_gemm_rows(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                              int64_t M, int64_t N, int64_t K, int64_t row_begin, int64_t row_end,
                              uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    const int64_t KB = K / 32, KH = K / 2;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t i = row_begin; i < row_end; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s, sa;
            mx4_dot_one(A + i * KH, SA + i * KB, B + j * KH, SB + j * KB, K, &s, &sa);
            int64_t o = (i - row_begin) * N + j;
            C[o] = hkg_oracle_bf16_rne(s);
            if (S)
                S[o] = s;
            if (absS)
                absS[o] = sa;
        }
    }
}

/* Selected elements (ii[t], jj[t]) of the MXFP4 product. */
void hkg_oracle_mx4_gemm_entries(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                                 int64_t M, int64_t N, int64_t K, const int64_t* ii, const int64_t* jj,
                                 int64_t count, uint16_t* C, double* S, double* absS, int nthreads)
{
    (void)M;
    (void)N;
    const int64_t KB = K / 32, KH = K / 2;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
    for (int64_t t = 0; t < count; ++t) {
        double s, sa;
        mx4_dot_one(A + ii[t] * KH, SA + ii[t] * KB, B + jj[t] * KH, SB + jj[t] * KB, K, &s, &sa);
        C[t] = hkg_oracle_bf16_rne(s);
        if (S)
            S[t] = s;
        if (absS)
            absS[t] = sa;
    }
}
