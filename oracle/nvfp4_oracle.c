/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 skinny GEMM
 *     Y[M,N] = X[M,K] . dequant(W)[K,N]
 *
 * TEST INFRASTRUCTURE ONLY. It is loaded by the tests, by the smoke check and by the CPU-baseline
 * leg of the benchmark, and by nothing else. The HIP library shares no code, header, table or
 * constant with this file, and neither side includes or links the other.
 *
 * Sources of the definitions (the pages name the format but never define its bits):
 *   - "Qwen3.8-27B-NVFP4-RTX5090" model card, table "Recipe (NVIDIA ModelOpt)": the weights are
 *     NVFP4 with group size 16 and the checkpoint stores packed U8 tensors (section "Serving",
 *     SGLang note on modelopt_fp4).
 *   - "Qwen3.8-27B-NVFP4-RTX5090" model card, section "Why lm_head is NVFP4": decode reads every
 *     weight once per token, which is the operation computed here.
 *   - OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element type (textbook definition of the code).
 *   - OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding with one NaN per sign and
 *     maximum 448 (textbook definition of the block-scale byte).
 *   - The quantisation recipe of the single-GEMV workload: per-tensor scale g = amax/(6*448);
 *     per 16-element block along K an E4M3 scale s = round_e4m3(block_amax/(6g)); codes are the
 *     round-to-nearest E2M1 of w/(s*g).
 *
 * Readings taken where the sources are silent (each is listed with its reason in the design doc):
 *   R1 layout: Wq[n][k/2], low nibble = even k; Ws[n][k/16]; W fp32 is [K][N] row-major.
 *   R2 "round" means round-to-nearest, ties to the even code (even mantissa bit).
 *   R3 E2M1 saturates: magnitudes above 6 give the code for 6.
 *   R4 E4M3 saturates at 448 (finite maximum), it never produces the NaN byte.
 *   R5 every step of the recipe is one fp32 IEEE operation, round-to-nearest-even, in the order
 *      written: g = amax/2688; t = bmax/(6*g) with 6*g rounded first; d = s*g; q = w/d.
 *   R6 degenerate blocks: if g == 0 every byte is 0; if d == 0 (scale byte decodes to zero, or s*g
 *      underflows) the block's codes are all 0 and its scale byte is kept as rounded.
 *   R7 the sign of a code is the sign of q, so small negative q gives code 8 (-0).
 *   R8 the dequantised weight is e2m1(code)*e4m3(scale)*g, exact in double.
 *
 * Compile with gcc, no fast-math, no FMA contraction (fp32 steps must round one at a time).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------ */
/* Element decoders, written from the bit-field definitions.                                   */
/* ------------------------------------------------------------------------------------------ */

/* FP4 E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: value = mantissa * 0.5. No infinities, no NaN. */
double oracle_e2m1_value(int code)
{
    int sign = (code >> 3) & 1;
    int expo = (code >> 1) & 3;
    int mant = code & 1;
    double mag;
    if (expo == 0)
        mag = 0.5 * mant;
    else
        mag = ldexp(1.0 + 0.5 * mant, expo - 1);
    return sign ? -mag : mag;
}

/* FP8 E4M3 (OCP OFP8, the "FN" variant): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa. Exponent 15 with mantissa 7 is NaN; there are no infinities. Exponent 0 is
 * subnormal: value = mantissa * 2^-9. Largest finite value 0x7E = 448. */
double oracle_e4m3_value(int byte)
{
    int sign = (byte >> 7) & 1;
    int expo = (byte >> 3) & 15;
    int mant = byte & 7;
    double mag;
    if (expo == 15 && mant == 7)
        return NAN;
    if (expo == 0)
        mag = ldexp((double)mant, -9);
    else
        mag = ldexp(1.0 + mant / 8.0, expo - 7);
    return sign ? -mag : mag;
}

/* bf16 bits widened to double: bf16 is the upper half of an fp32, so this is exact. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------------------------ */
/* Rounding, written as the definition: the representable value nearest to the input, with a  */
/* tie going to the even code (R2). Candidates are enumerated; no bit tricks.                  */
/* ------------------------------------------------------------------------------------------ */

/* Nearest E2M1 code to q (R2, R3, R7). */
uint8_t oracle_e2m1_round(float q)
{
    int sign = signbit(q) ? 1 : 0;
    double a = fabs((double)q);
    int best = 0;
    double best_dist;
    /* R3: at or above the largest magnitude the answer is 6. (This also keeps every distance
     * below exact: for a < 6 the subtraction a - v is exact in double.) */
    if (a >= 6.0)
        return (uint8_t)((sign << 3) | 7);
    best_dist = a - oracle_e2m1_value(0);
    for (int code = 1; code <= 7; code++) {
        double dist = fabs(a - oracle_e2m1_value(code));
        if (dist < best_dist || (dist == best_dist && (code & 1) == 0)) {
            best = code;
            best_dist = dist;
        }
    }
    return (uint8_t)((sign << 3) | best);
}

/* Nearest finite E4M3 byte to t (R2, R4). Bytes 0x00..0x7E are the non-negative finite values
 * in increasing order; ties go to the byte with mantissa lsb 0. NaN input gives the NaN byte. */
uint8_t oracle_e4m3_round(float t)
{
    int sign = signbit(t) ? 1 : 0;
    double a = fabs((double)t);
    int best = 0;
    double best_dist;
    if (isnan(t))
        return 0x7F;
    /* R4: at or above 448 the answer is 448. (Below it, the distances to the two neighbours of
     * a are exact in double, which is all a nearest-with-ties decision needs.) */
    if (a >= 448.0)
        return (uint8_t)((sign << 7) | 0x7E);
    best_dist = a - oracle_e4m3_value(0);
    for (int byte = 1; byte <= 0x7E; byte++) {
        double dist = fabs(a - oracle_e4m3_value(byte));
        if (dist < best_dist || (dist == best_dist && (byte & 1) == 0)) {
            best = byte;
            best_dist = dist;
        }
    }
    return (uint8_t)((sign << 7) | best);
}

/* Array forms, used by the exhaustive rounding tests. */
void oracle_e2m1_round_array(const float *q, size_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < (long long)n; i++)
        out[i] = oracle_e2m1_round(q[i]);
}

void oracle_e4m3_round_array(const float *t, size_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (long long i = 0; i < (long long)n; i++)
        out[i] = oracle_e4m3_round(t[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Quantisation recipe (R1, R5, R6): fp32 W[K][N] -> codes Wq[N][K/2], scales Ws[N][K/16], g.   */
/* ------------------------------------------------------------------------------------------ */

void oracle_quantize(int K, int N, const float *W, uint8_t *Wq, uint8_t *Ws, float *g_out)
{
    const size_t total = (size_t)K * (size_t)N;
    const int nblocks = K / 16;
    float amax = 0.0f;
    float g;

    /* Step 1: amax = max |w| over the tensor (exact). */
    for (size_t i = 0; i < total; i++) {
        float a = fabsf(W[i]);
        if (a > amax)
            amax = a;
    }
    /* Step 2: the per-tensor scale, 6 * 448 = 2688 exactly. */
    g = amax / 2688.0f;
    *g_out = g;

    memset(Wq, 0, (size_t)N * (size_t)(K / 2));
    memset(Ws, 0, (size_t)N * (size_t)nblocks);
    if (g == 0.0f)
        return; /* R6 */

#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
        for (int b = 0; b < nblocks; b++) {
            float bmax = 0.0f;
            float sixg, t, d;
            uint8_t sbyte;
            /* Step 3: block amax, then the E4M3 block scale. */
            for (int i = 0; i < 16; i++) {
                float a = fabsf(W[(size_t)(16 * b + i) * N + n]);
                if (a > bmax)
                    bmax = a;
            }
            sixg = 6.0f * g;
            t = bmax / sixg;
            sbyte = oracle_e4m3_round(t);
            Ws[(size_t)n * nblocks + b] = sbyte;
            /* Step 4: codes of w / (s * g). */
            d = (float)oracle_e4m3_value(sbyte) * g;
            if (d == 0.0f)
                continue; /* R6: codes stay 0 */
            for (int i = 0; i < 16; i++) {
                int k = 16 * b + i;
                float q = W[(size_t)k * N + n] / d;
                uint8_t code = oracle_e2m1_round(q);
                /* Step 5: pack, low nibble = even k (R1). */
                uint8_t *byte = &Wq[(size_t)n * (K / 2) + k / 2];
                if ((k & 1) == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | code);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (code << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Dequantisation (R8): the exact weight w(k,n) in double, written to Wd[K][N].                */
/* ------------------------------------------------------------------------------------------ */

static double weight_at(int K, const uint8_t *Wq, const uint8_t *Ws, double g, int k, int n)
{
    uint8_t byte = Wq[(size_t)n * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 0x0F);
    double s = oracle_e4m3_value(Ws[(size_t)n * (K / 16) + k / 16]);
    return oracle_e2m1_value(code) * s * g;
}

void oracle_dequantize(int K, int N, const uint8_t *Wq, const uint8_t *Ws, float g, double *Wd)
{
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++)
            Wd[(size_t)k * N + n] = weight_at(K, Wq, Ws, (double)g, k, n);
}

/* ------------------------------------------------------------------------------------------ */
/* The GEMM in double.                                                                         */
/*   Y[m][n] = sum_k x[m][k] * w(k,n)       A[m][n] = sum_k |x[m][k] * w(k,n)|                 */
/* X is bf16 bits [M][K]; Y and A are double [M][ncols] for the listed columns (all if cols is  */
/* NULL, in which case ncols must equal N). Each weight is decoded from its code, its block    */
/* scale and g; x is widened exactly; products and sums are in double, k in increasing order. */
/* ------------------------------------------------------------------------------------------ */

int oracle_gemm(int M, int N, int K, const uint16_t *X, const uint8_t *Wq, const uint8_t *Ws,
                float g, const int *cols, int ncols, double *Y, double *A)
{
    int failed = 0;
    double *xd = (double *)malloc(sizeof(double) * (size_t)M * (size_t)K);
    (void)N;
    if (!xd)
        return 1;
    for (size_t i = 0; i < (size_t)M * (size_t)K; i++)
        xd[i] = oracle_bf16_value(X[i]);
#pragma omp parallel
    {
        /* One decoded column of W, reused for every row m of X. */
        double *wcol = (double *)malloc(sizeof(double) * (size_t)K);
        if (!wcol) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int j = 0; j < ncols; j++) {
            int n = cols ? cols[j] : j;
            if (!wcol)
                continue;
            for (int k = 0; k < K; k++)
                wcol[k] = weight_at(K, Wq, Ws, (double)g, k, n);
            for (int m = 0; m < M; m++) {
                const double *x = xd + (size_t)m * K;
                double sum = 0.0, asum = 0.0;
                for (int k = 0; k < K; k++) {
                    double p = x[k] * wcol[k];
                    sum += p;
                    asum += fabs(p);
                }
                Y[(size_t)m * ncols + j] = sum;
                A[(size_t)m * ncols + j] = asum;
            }
        }
        free(wcol);
    }
    free(xd);
    return failed;
}

/* Number of threads the parallel loops above use (for reporting CPU timings). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the OpenMP loops from now on (the benchmark times the oracle on all host cores and
 * on one); n < 1 is taken as 1. No effect without OpenMP. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n < 1 ? 1 : n);
#else
    (void)n;
#endif
}
