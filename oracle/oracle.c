/*
 * CPU oracle for the tiled GEMM  C = A * B^T  (TEST INFRASTRUCTURE ONLY).
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  The product path never calls it, and it shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes (FlyDSL "Kernel authoring guide", section 11 "Complete
 * example: Preshuffle GEMM": a GEMM with fp32 accumulation whose output is
 * scaled by per-operand scales and converted to bf16; FlyDSL "Kernel Authoring"
 * skill, section 3 "Internal Types", for the scale order (value * scale_a) *
 * scale_b):
 *
 *     C_ref[i][j] = sigma * sum_{k=0}^{K-1} a(i,k) * b(j,k)
 *
 * with A stored M x K row-major and B stored N x K row-major (both
 * K-contiguous, so b(j,k) = B[j][k]), one fp64 accumulator per output and k
 * taken in increasing order, sigma = 1 for bf16 and s_a * s_b (formed in fp64)
 * for fp8.  It also returns S[i][j] = |sigma| * sum_k |a(i,k) * b(j,k)|, the
 * magnitude sum used by the element-wise tolerance.
 *
 * Element decoders are written from the format definitions:
 *   bf16      : the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent,
 *               7 fraction bits).
 *   e4m3fn    : OCP 8-bit float, 1 sign, 4 exponent bits (bias 7), 3 fraction
 *               bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is
 *               NaN; no infinities; largest finite value 448.
 *
 *   e2m1      : OCP MX 4-bit float, 1 sign, 2 exponent bits (bias 1), 1
 *               fraction bit; exponent field 0 is subnormal (m * 2^-1); all
 *               16 codes finite (largest 6).  Two per byte, element 2t in the
 *               low nibble of byte t.
 *   e8m0      : OCP MX block scale, 8 exponent bits (bias 127), value
 *               2^(e-127); 0xFF is NaN.
 *
 * MX block-scaled operands (the gfx950 scaled MFMA of FlyDSL "Kernel
 * authoring guide", section 4.3 "ROCm intrinsics", MFMA instructions; E8M0
 * block scales with block size 32, FlyDSL "Kernel Authoring" skill, section 6
 * "MFMA Integration", gfx1250 WMMA entry; formats as the OCP Microscaling
 * specification defines them): element k of row i counts as
 * elem(i,k) * 2^(scale[i][k/32] - 127), the scales stored rows x K/32 bytes
 * row-major.
 *
 * Integer operands (int8 MFMA with int32 accumulation: FlyDSL "Kernel
 * authoring guide", section 4.3 "ROCm intrinsics", MFMA instructions, and
 * the "Kernel Authoring" skill, section 6 "MFMA Integration"; W4A8: the same
 * skill, section 10 "Troubleshooting", item INT4, an int8 A with a B of
 * packed int4 values):
 *   int8      : two's complement byte, -128 .. 127.
 *   int4      : two's complement nibble, -8 .. 7; two per byte, element 2t
 *               in the low nibble of byte t (the order MX e2m1 uses).
 * The products are summed exactly in int64: acc[i][j] = sum_k a(i,k) b(j,k)
 * and S[i][j] = sum_k |a(i,k) b(j,k)|.
 *
 * The output rounding to bf16 is round-to-nearest, ties-to-even, done in
 * fp64 with nearbyint() under the default FE_TONEAREST mode.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math, so every fp64 sum
 * stays in program order).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_E4M3FN = 1, ORACLE_MXFP8 = 2, ORACLE_MXFP4 = 3 };

double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_e4m3fn_value(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int expo = (bits >> 3) & 0xF;
    int frac = bits & 0x7;
    double mag;
    if (expo == 0xF && frac == 0x7)
        return NAN;
    if (expo == 0)
        mag = ldexp((double)frac, -9);              /* subnormal: m * 2^(1-7-3) */
    else
        mag = ldexp(1.0 + frac / 8.0, expo - 7);    /* normal: 1.m * 2^(e-7)    */
    return sign ? -mag : mag;
}

double oracle_e2m1_value(uint8_t code)
{
    int sign = (code >> 3) & 1;
    int expo = (code >> 1) & 0x3;
    int frac = code & 0x1;
    double mag = expo == 0 ? 0.5 * frac                     /* subnormal: m * 2^(1-1-1) */
                           : ldexp(1.0 + frac / 2.0, expo - 1); /* normal: 1.m * 2^(e-1) */
    return sign ? -mag : mag;
}

double oracle_e8m0_value(uint8_t bits)
{
    if (bits == 0xFF)
        return NAN;
    return ldexp(1.0, (int)bits - 127);
}

/* Element k of row r of an MX operand (K elements per row). */
static double mx_element(int kind, const void *base, const uint8_t *scale, int64_t K, int64_t r, int64_t k)
{
    const int64_t idx = r * K + k;
    double v;
    if (kind == ORACLE_MXFP8) {
        v = oracle_e4m3fn_value(((const uint8_t *)base)[idx]);
    } else {
        const uint8_t byte = ((const uint8_t *)base)[idx / 2];
        v = oracle_e2m1_value((idx % 2) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF));
    }
    return v * oracle_e8m0_value(scale[r * (K / 32) + k / 32]);
}

static void dot_entry_mx(int64_t K, int kind, const void *A, const uint8_t *SA, const void *B,
                         const uint8_t *SB, int64_t i, int64_t j, double *c, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = mx_element(kind, A, SA, K, i, k) * mx_element(kind, B, SB, K, j, k);
        acc += p;
        mag += fabs(p);
    }
    *c = acc;
    *s = mag;
}

static double element(int kind, const void *base, int64_t idx)
{
    if (kind == ORACLE_BF16)
        return oracle_bf16_value(((const uint16_t *)base)[idx]);
    return oracle_e4m3fn_value(((const uint8_t *)base)[idx]);
}

/* One output element: the definition written out. */
static void dot_entry(int64_t K, int kind, const void *A, const void *B,
                      int64_t i, int64_t j, double sigma, double *c, double *s)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = element(kind, A, i * K + k) * element(kind, B, j * K + k);
        acc += p;
        mag += fabs(p);
    }
    *c = sigma * acc;
    *s = fabs(sigma) * mag;
}

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Full product.  C and S are M x N row-major fp64 (S may be NULL). */
void oracle_gemm_bt(int64_t M, int64_t N, int64_t K, int kind,
                    const void *A, const void *B, double sigma,
                    double *C, double *S)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double c, s;
            dot_entry(K, kind, A, B, i, j, sigma, &c, &s);
            C[i * N + j] = c;
            if (S)
                S[i * N + j] = s;
        }
    }
}

/* Selected entries (rows[t], cols[t]) for t < count, for checks at sizes
 * where the full product would take too long. */
void oracle_gemm_bt_entries(int64_t K, int kind, const void *A, const void *B,
                            double sigma, int64_t count, const int64_t *rows,
                            const int64_t *cols, double *C, double *S)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < count; ++t) {
        double c, s;
        dot_entry(K, kind, A, B, rows[t], cols[t], sigma, &c, &s);
        C[t] = c;
        if (S)
            S[t] = s;
    }
}

/* MX product (K % 32 == 0; for MXFP4 K even): full and selected entries. */
void oracle_gemm_bt_mx(int64_t M, int64_t N, int64_t K, int kind, const void *A, const uint8_t *SA,
                       const void *B, const uint8_t *SB, double *C, double *S)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double c, s;
            dot_entry_mx(K, kind, A, SA, B, SB, i, j, &c, &s);
            C[i * N + j] = c;
            if (S)
                S[i * N + j] = s;
        }
    }
}

void oracle_gemm_bt_mx_entries(int64_t K, int kind, const void *A, const uint8_t *SA, const void *B,
                               const uint8_t *SB, int64_t count, const int64_t *rows, const int64_t *cols,
                               double *C, double *S)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < count; ++t) {
        double c, s;
        dot_entry_mx(K, kind, A, SA, B, SB, rows[t], cols[t], &c, &s);
        C[t] = c;
        if (S)
            S[t] = s;
    }
}

int oracle_int8_value(uint8_t bits) { return bits < 128 ? (int)bits : (int)bits - 256; }

int oracle_int4_value(uint8_t nibble)
{
    nibble &= 0xF;
    return nibble < 8 ? (int)nibble : (int)nibble - 16;
}

/* Element k of row r of an integer operand with K elements per row:
 * bits 8 (one byte each) or 4 (two per byte, the even element low). */
static int64_t int_element(int bits, const uint8_t *base, int64_t K, int64_t r, int64_t k)
{
    const int64_t idx = r * K + k;
    if (bits == 8)
        return oracle_int8_value(base[idx]);
    const uint8_t byte = base[idx / 2];
    return oracle_int4_value((idx % 2) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF));
}

static void dot_entry_int(int64_t K, int b_bits, const uint8_t *A, const uint8_t *B, int64_t i, int64_t j,
                          int64_t *c, int64_t *s)
{
    int64_t acc = 0, mag = 0;
    for (int64_t k = 0; k < K; ++k) {
        const int64_t p = int_element(8, A, K, i, k) * int_element(b_bits, B, K, j, k);
        acc += p;
        mag += p < 0 ? -p : p;
    }
    *c = acc;
    *s = mag;
}

/* int8 A (M x K bytes) times B^T, B int8 (b_bits 8, N x K bytes) or packed
 * int4 (b_bits 4, N x K/2 bytes): exact sums, full and selected entries. */
void oracle_gemm_bt_int(int64_t M, int64_t N, int64_t K, int b_bits, const uint8_t *A, const uint8_t *B,
                        int64_t *C, int64_t *S)
{
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t c, s;
            dot_entry_int(K, b_bits, A, B, i, j, &c, &s);
            C[i * N + j] = c;
            if (S)
                S[i * N + j] = s;
        }
    }
}

void oracle_gemm_bt_int_entries(int64_t K, int b_bits, const uint8_t *A, const uint8_t *B, int64_t count,
                                const int64_t *rows, const int64_t *cols, int64_t *C, int64_t *S)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < count; ++t) {
        int64_t c, s;
        dot_entry_int(K, b_bits, A, B, rows[t], cols[t], &c, &s);
        C[t] = c;
        if (S)
            S[t] = s;
    }
}

/* Round-to-nearest-even of a finite double to bf16, returned as bits.
 * bf16 keeps 8 significant bits; below 2^-126 the spacing is fixed at
 * 2^-133 (subnormals).  Overflow past the largest finite bf16 gives inf. */
uint16_t oracle_round_bf16(double x)
{
    double r;
    float f;
    uint32_t u;
    if (isnan(x))
        return 0x7FC0;
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    if (fabs(x) < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(x, 133)), -133);
    } else {
        int e;
        double m = frexp(x, &e);                     /* x = m * 2^e, 0.5 <= |m| < 1 */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);    /* 8 significant bits */
    }
    f = (float)r;                                    /* exact: r has <= 8 bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_round_bf16_array(int64_t n, const double *x, uint16_t *out)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; ++t)
        out[t] = oracle_round_bf16(x[t]);
}
