/*
 * TACO CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C implementation of what the TACO compression
 * operator computes, written in double precision from the paper's equations.
 * Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library.  The GPU library never links it, includes it or
 * calls it, and it shares no code, header or constant table with the GPU side.
 *
 * Source ([TACO] below): the page "TACO: Efficient Communication Compression of
 * Intermediate Tensors for Scalable Tensor-Parallel LLM Training", sections
 * 4.2.2 (ASH transform, Eq. 5-8), 4.3 (Dual-Scale FP8 quantization, Eq. 9-13)
 * and Algorithm 1 (sender side and receiver side), plus section 2.3 / Figure 3
 * / Eq. 4 for the E4M3 format.
 *
 * Readings of points the paper leaves open (all stated once here):
 *  - epsilon sits inside the square root of Eq. 6 (the text calls sigma an RMS
 *    amplitude); its value is a parameter (the library documents 1e-20).
 *  - Q_max is the largest finite value of OCP E4M3 ("E4M3FN"): bias 7, no
 *    infinities, NaN = S.1111.111, max 448.  The paper cites the FP8 formats
 *    paper of Micikevicius et al. (2022) for the format.
 *  - Cvt_FP8 of Eq. 10 takes a single-precision argument (the conversion the
 *    paper names takes a float) and rounds to nearest, ties to even,
 *    saturating to +-448.  Exact zeros of the rotated block carry no sign in the
 *    code: they encode as 0x00.
 *  - "max" in Eq. 9 is the maximum absolute value.  A block whose rotated
 *    values are all zero gets s = 0 and all-zero codes, and reconstructs to 0.
 *  - The Hadamard matrix of Eq. 8 / Eq. 12 is Sylvester's, in natural order:
 *    H[i][j] = (-1)^popcount(i & j), the matrix an in-place FWHT applies.
 *  - alpha and s travel as float32 (each rounded once from double), and the
 *    receiver uses exactly those float32 values.
 *  - The decompressed tensor is rounded once to bfloat16 (nearest, ties to
 *    even); the accumulate variant rounds G' once to float32 and adds it to
 *    the float32 accumulator with one float32 addition.
 *  - Code formats other than E4M3 (section 5.3.2 format ablation; section 6,
 *    the INT8 fallback for hardware without FP8): the pipeline is unchanged
 *    and only Cvt_FP8 / Cvt_FP32 and Q_max change.
 *      E5M2: OCP E5M2 (bias 15, S.11111.00 = infinity, S.11111.mm with
 *            mm != 0 = NaN), Q_max = 57344, nearest-even, saturating.
 *      INT8: the uniform quantiser of section 2.3 / Eq. 1 with the dual
 *            scale as its step (Delta = s = max|Z| / 127, Q_max = 127):
 *            q = round(Z / s), nearest with ties to even, clamped to
 *            [-127, 127], stored as a two's complement byte.
 *
 * Build:  gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 *         taco_oracle.c -o libtaco_oracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_QMAX 448.0          /* largest finite OCP E4M3 value */
#define ORACLE_E5M2_MAX 57344.0    /* largest finite OCP E5M2 value */
#define ORACLE_INT8_MAX 127.0      /* symmetric INT8 range */
#define ORACLE_MAX_BLOCK 4096

/* Code formats (argument `fmt` below). */
#define ORACLE_FMT_E4M3 0
#define ORACLE_FMT_E5M2 1
#define ORACLE_FMT_INT8 2

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> double                                                        */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round q to the nearest integer, ties to the even integer (q >= 0). */
static double round_half_even(double q)
{
    double fl = floor(q);
    double d = q - fl;               /* exact: q has few significant bits */
    if (d > 0.5) return fl + 1.0;
    if (d < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/*
 * double -> bfloat16, round to nearest, ties to even (one rounding from the
 * double value).  bfloat16 has 8 significant bits, exponents -126..127, and
 * subnormals with step 2^-133.
 */
uint16_t taco_oracle_double_to_bf16(double g)
{
    if (isnan(g)) return 0x7FC0;
    uint16_t sign = signbit(g) ? 0x8000 : 0;
    double a = fabs(g);
    double r;
    if (a == 0.0) {
        r = 0.0;
    } else {
        int e;
        frexp(a, &e);                /* a = f * 2^e, f in [0.5, 1) */
        int E = e - 1;               /* a in [2^E, 2^(E+1)) */
        if (E < -126) E = -126;      /* subnormal range: fixed step 2^-133 */
        double step = ldexp(1.0, E - 7);
        r = round_half_even(a / step) * step;
    }
    /* r is a bfloat16 value (or overflows): express it through binary32. */
    float f = (float)r;              /* exact when representable; inf beyond */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* E4M3 codec ([TACO] section 2.3, Eq. 4: 4 exponent bits, 3 mantissa bits)   */
/* ------------------------------------------------------------------------ */

/* Value of an E4M3 code: sign, 4-bit exponent with bias 7, 3-bit mantissa;
 * exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN. */
double taco_oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 0x7;
    if (e == 0xF && m == 0x7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest E4M3 code to v, ties to even mantissa, saturating to +-448. */
uint8_t taco_oracle_e4m3_encode(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= ORACLE_QMAX) return sign | 0x7E;
    int code;
    if (a < ldexp(1.0, -6)) {
        /* Subnormal range: values m * 2^-9.  m = 8 is the smallest normal,
         * which has code 0x08, so the code equals the rounded multiple. */
        code = (int)round_half_even(a / ldexp(1.0, -9));
    } else {
        int e;
        frexp(a, &e);
        int E = e - 1;                          /* a in [2^E, 2^(E+1)) */
        double q = a / ldexp(1.0, E - 3);       /* in [8, 16), exact */
        int mq = (int)round_half_even(q);       /* 8..16; 16 carries */
        code = ((E + 7) << 3) + (mq - 8);
    }
    if (code > 0x7E) code = 0x7E;               /* 480 would be the NaN slot */
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* E5M2 codec (section 2.3 / Figure 3: 5 exponent bits, 2 mantissa bits)      */
/* ------------------------------------------------------------------------ */

/* Value of an E5M2 code: bias 15, exponent field 0 is subnormal (m * 2^-16),
 * exponent field 31 is infinity (m = 0) or NaN. */
double taco_oracle_e5m2_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 2) & 0x1F, m = c & 0x3;
    double mag;
    if (e == 0x1F)
        mag = (m == 0) ? INFINITY : NAN;
    else
        mag = (e == 0) ? ldexp((double)m, -16) : ldexp(1.0 + m / 4.0, e - 15);
    return s ? -mag : mag;
}

/* Nearest E5M2 code to v, ties to even mantissa, saturating to +-57344. */
uint8_t taco_oracle_e5m2_encode(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a >= ORACLE_E5M2_MAX) return sign | 0x7B;
    int code;
    if (a < ldexp(1.0, -14)) {
        /* Subnormal range m * 2^-16; m = 4 is the smallest normal, code 0x04. */
        code = (int)round_half_even(a / ldexp(1.0, -16));
    } else {
        int e;
        frexp(a, &e);
        int E = e - 1;                          /* a in [2^E, 2^(E+1)) */
        double q = a / ldexp(1.0, E - 2);       /* in [4, 8), exact */
        int mq = (int)round_half_even(q);       /* 4..8; 8 carries */
        code = ((E + 15) << 2) + (mq - 4);
    }
    if (code > 0x7B) code = 0x7B;               /* 0x7C would be infinity */
    return sign | (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* INT8 codec (section 2.3 and Eq. 1: round(x / Delta))                      */
/* ------------------------------------------------------------------------ */

/* Value of an INT8 code: the byte as a two's complement integer. */
double taco_oracle_int8_decode(uint8_t c)
{
    return (double)(int8_t)c;
}

/* Nearest integer to v, ties to even, clamped to [-127, 127]. */
uint8_t taco_oracle_int8_encode(float v)
{
    if (isnan(v)) return 0x00;
    double a = fabs((double)v);
    double r = (a >= ORACLE_INT8_MAX) ? ORACLE_INT8_MAX : round_half_even(a);
    int q = (int)r;
    if (signbit(v)) q = -q;
    return (uint8_t)(int8_t)q;
}

/* Format dispatch: Q_max, Cvt (float -> code) and its inverse. */
double taco_oracle_qmax(int fmt)
{
    switch (fmt) {
    case ORACLE_FMT_E4M3: return ORACLE_QMAX;
    case ORACLE_FMT_E5M2: return ORACLE_E5M2_MAX;
    case ORACLE_FMT_INT8: return ORACLE_INT8_MAX;
    default: return -1.0;
    }
}

static uint8_t encode_fmt(float v, int fmt)
{
    switch (fmt) {
    case ORACLE_FMT_E5M2: return taco_oracle_e5m2_encode(v);
    case ORACLE_FMT_INT8: return taco_oracle_int8_encode(v);
    default: return taco_oracle_e4m3_encode(v);
    }
}

static double decode_fmt(uint8_t c, int fmt)
{
    switch (fmt) {
    case ORACLE_FMT_E5M2: return taco_oracle_e5m2_decode(c);
    case ORACLE_FMT_INT8: return taco_oracle_int8_decode(c);
    default: return taco_oracle_e4m3_decode(c);
    }
}

static int valid_fmt(int fmt)
{
    return fmt == ORACLE_FMT_E4M3 || fmt == ORACLE_FMT_E5M2 || fmt == ORACLE_FMT_INT8;
}

void taco_oracle_encode_array(int fmt, const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = encode_fmt(v[i], fmt);
}

void taco_oracle_decode_array(int fmt, const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = decode_fmt(c[i], fmt);
}

/* Element-wise array forms of the three conversions above. */
void taco_oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = taco_oracle_e4m3_encode(v[i]);
}

void taco_oracle_e4m3_decode_array(const uint8_t *c, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = taco_oracle_e4m3_decode(c[i]);
}

void taco_oracle_double_to_bf16_array(const double *g, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = taco_oracle_double_to_bf16(g[i]);
}

/* ------------------------------------------------------------------------ */
/* Hadamard ([TACO] Eq. 8, Eq. 12; section 4.2.2 "FWHT")                      */
/* ------------------------------------------------------------------------ */

/* In-place unnormalised Walsh-Hadamard transform, Sylvester natural order:
 * v <- H_n v with H_n[i][j] = (-1)^popcount(i & j).  n is a power of two. */
void taco_oracle_fwht(double *v, int n)
{
    for (int h = 1; h < n; h *= 2)
        for (int i = 0; i < n; i += 2 * h)
            for (int j = i; j < i + h; ++j) {
                double a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
}

static int valid_block(int B)
{
    if (B < 2 || B > ORACLE_MAX_BLOCK) return 0;
    return (B & (B - 1)) == 0;
}

/* ------------------------------------------------------------------------ */
/* Sender side ([TACO] Algorithm 1, Eq. 5-10)                                 */
/* ------------------------------------------------------------------------ */

/*
 * ASH transform of one block given as doubles: alpha_k (Eq. 6-7), the
 * rescaled block Gt (Eq. 7, element-wise product) and Z (Eq. 8).  Any of the
 * output pointers may be NULL.
 */
static void ash_block_f64(const double *G, int B, double tau, double eps,
                          double *alpha_out, double *gt_out, double *z_out)
{
    double Z[ORACLE_MAX_BLOCK];
    double energy = 0.0;
    for (int j = 0; j < B; ++j) energy += G[j] * G[j];
    double sigma = sqrt(energy / B + eps);         /* Eq. 6 */
    double alpha = tau / sigma;                    /* Eq. 7 */
    for (int j = 0; j < B; ++j) Z[j] = alpha * G[j];
    if (gt_out) memcpy(gt_out, Z, sizeof(double) * (size_t)B);
    taco_oracle_fwht(Z, B);                        /* Eq. 8 */
    double c = 1.0 / sqrt((double)B);
    for (int j = 0; j < B; ++j) Z[j] *= c;
    if (alpha_out) *alpha_out = alpha;
    if (z_out) memcpy(z_out, Z, sizeof(double) * (size_t)B);
}

/* The same for one block of bf16 values. */
int taco_oracle_ash_block(const uint16_t *x, int B, double tau, double eps,
                          double *alpha_out, double *gt_out, double *z_out)
{
    if (!valid_block(B)) return -1;
    double G[ORACLE_MAX_BLOCK];
    for (int j = 0; j < B; ++j) G[j] = bf16_to_double(x[j]);
    ash_block_f64(G, B, tau, eps, alpha_out, gt_out, z_out);
    return 0;
}

/* Eq. 9-10 for one block with its Z and alpha (Algorithm 1, sender side). */
static void quantise_block(const double *Z, double a, int B, int fmt, uint8_t *q,
                           float *alpha_out, float *scale_out)
{
    double zmax = 0.0;
    for (int j = 0; j < B; ++j) zmax = fmax(zmax, fabs(Z[j]));
    double s = zmax / taco_oracle_qmax(fmt);       /* Eq. 9 */
    for (int j = 0; j < B; ++j) {                  /* Eq. 10 */
        float v = (s > 0.0) ? (float)(Z[j] / s) : 0.0f;
        if (v == 0.0f) v = 0.0f;                   /* zero carries no sign */
        q[j] = encode_fmt(v, fmt);
    }
    *alpha_out = (float)a;
    *scale_out = (float)s;
}

/*
 * Compress a flattened tensor of n bf16 values (n a multiple of B) into
 * n codes of format fmt and n/B pairs (alpha_k, s_k), block by block.
 */
int taco_oracle_compress_fmt(const uint16_t *x, int64_t n, int B, double tau,
                             double eps, int fmt, uint8_t *codes, float *alpha,
                             float *scale)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    double Z[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        double a;
        taco_oracle_ash_block(x + k * B, B, tau, eps, &a, NULL, Z);
        quantise_block(Z, a, B, fmt, codes + k * B, alpha + k, scale + k);
    }
    return 0;
}

int taco_oracle_compress(const uint16_t *x, int64_t n, int B, double tau,
                         double eps, uint8_t *codes, float *alpha, float *scale)
{
    return taco_oracle_compress_fmt(x, n, B, tau, eps, ORACLE_FMT_E4M3, codes,
                                    alpha, scale);
}

/* The same for a tensor given as doubles. */
int taco_oracle_compress_f64(const double *x, int64_t n, int B, double tau,
                             double eps, int fmt, uint8_t *codes, float *alpha,
                             float *scale)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    double Z[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        double a;
        ash_block_f64(x + k * B, B, tau, eps, &a, NULL, Z);
        quantise_block(Z, a, B, fmt, codes + k * B, alpha + k, scale + k);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Receiver side ([TACO] Algorithm 1, Eq. 11-13)                              */
/* ------------------------------------------------------------------------ */

/* Reconstruct one block G'_k in double from its codes and float32 scalars. */
static void reconstruct_block(const uint8_t *q, float alpha, float s, int B,
                              int fmt, double *out)
{
    for (int j = 0; j < B; ++j)                    /* Eq. 11 */
        out[j] = decode_fmt(q[j], fmt) * (double)s;
    taco_oracle_fwht(out, B);                      /* Eq. 12 */
    double c = 1.0 / sqrt((double)B);
    for (int j = 0; j < B; ++j) out[j] = out[j] * c / (double)alpha; /* Eq. 13 */
}

/* G' in double precision (no output rounding), for error analysis. */
int taco_oracle_reconstruct_f64(const uint8_t *codes, const float *alpha,
                                const float *scale, int64_t n, int B, int fmt,
                                double *out)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    for (int64_t k = 0; k < n / B; ++k)
        reconstruct_block(codes + k * B, alpha[k], scale[k], B, fmt, out + k * B);
    return 0;
}

/* Decompress to bf16 (round to nearest even, once). */
int taco_oracle_decompress(const uint8_t *codes, const float *alpha,
                           const float *scale, int64_t n, int B, int fmt,
                           uint16_t *y)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    double g[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        reconstruct_block(codes + k * B, alpha[k], scale[k], B, fmt, g);
        for (int j = 0; j < B; ++j)
            y[k * B + j] = taco_oracle_double_to_bf16(g[j]);
    }
    return 0;
}

/* acc += G' in float32: G' rounded once to float32, then one float32 add. */
int taco_oracle_decompress_accumulate(const uint8_t *codes, const float *alpha,
                                      const float *scale, int64_t n, int B,
                                      int fmt, float *acc)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    double g[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        reconstruct_block(codes + k * B, alpha[k], scale[k], B, fmt, g);
        for (int j = 0; j < B; ++j) {
            float gf = (float)g[j];
            acc[k * B + j] = acc[k * B + j] + gf;
        }
    }
    return 0;
}

/*
 * Several payloads at once (the local reduction of section 4.4.2 over P
 * received payloads): acc += float32(sum_p G'_p), the payloads' exact
 * reconstructions summed in double, rounded once to float32 and added with
 * one float32 addition.  With one payload this is
 * taco_oracle_decompress_accumulate.
 */
int taco_oracle_decompress_accumulate_n(int npay, const uint8_t *const *codes_in,
                                        const float *const *alpha_in,
                                        const float *const *scale_in, int64_t n, int B,
                                        int fmt, float *acc)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B || npay < 0) return -1;
    double g[ORACLE_MAX_BLOCK], sum[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        for (int j = 0; j < B; ++j) sum[j] = 0.0;
        for (int p = 0; p < npay; ++p) {
            reconstruct_block(codes_in[p] + k * B, alpha_in[p][k], scale_in[p][k], B, fmt, g);
            for (int j = 0; j < B; ++j) sum[j] += g[j];
        }
        if (npay == 0) continue;
        for (int j = 0; j < B; ++j) {
            float gf = (float)sum[j];
            acc[k * B + j] = acc[k * B + j] + gf;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Owner step of the two-shot all-reduce ([TACO] section 4.4.2)              */
/* ------------------------------------------------------------------------ */

/*
 * The reduce-scatter phase ends in one local reduction of the received
 * payloads, and the reduced segment is compressed again for the all-gather:
 * X = own + sum_p G'_p (Eq. 11-13 per payload, summed in double; own may be
 * NULL for a pure sum), then (codes, alpha, s) of X by Eq. 5-10.  Payloads
 * and result share one code format.
 */
int taco_oracle_reduce_compress(const uint16_t *own, int npay,
                                const uint8_t *const *codes_in,
                                const float *const *alpha_in,
                                const float *const *scale_in, int64_t n, int B,
                                double tau, double eps, int fmt, uint8_t *codes,
                                float *alpha, float *scale)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B || npay < 0) return -1;
    double X[ORACLE_MAX_BLOCK], g[ORACLE_MAX_BLOCK], Z[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        for (int j = 0; j < B; ++j) X[j] = own ? bf16_to_double(own[k * B + j]) : 0.0;
        for (int p = 0; p < npay; ++p) {
            reconstruct_block(codes_in[p] + k * B, alpha_in[p][k], scale_in[p][k], B,
                              fmt, g);
            for (int j = 0; j < B; ++j) X[j] += g[j];
        }
        double a;
        ash_block_f64(X, B, tau, eps, &a, NULL, Z);
        quantise_block(Z, a, B, fmt, codes + k * B, alpha + k, scale + k);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Ablation variants and the fidelity metrics                                */
/* ------------------------------------------------------------------------ */

/*
 * The variants the TACO paper compares its operator with, each as a round
 * trip x -> codes -> x' (every variant keeps the code format's Q_max):
 *   0 TACO      ASH + DS: Eq. 5-13 (compress, then reconstruct).
 *   1 DIRECT    direct cast of x, no scaling (section 4.2.1 "direct FP8
 *               quantization"; the NVFP8 arm of section 5.2.2).
 *   2 DS        dual scale only: per block s = max|x| / Q_max, q = Cvt(x / s),
 *               x' = decode(q) s (section 5.2.2, DS in isolation).
 *   3 ASH       adaptive scale and rotation, no post-rotation scale:
 *               q = Cvt(Z) with Z of Eq. 8, x' = H decode(q) / sqrt(B) / alpha
 *               (section 5.2.2, ASH alone).
 *   4 HADAMARD  the standard rotation alone: Z = H x / sqrt(B), q = Cvt(Z),
 *               x' = H decode(q) / sqrt(B) (sections 4.2.1 and 5.3.1).
 *   5 TENSOR    one scale for the whole tensor: Delta = max|x| / Q_max,
 *               q = Cvt(x / Delta), x' = decode(q) Delta (the uniform
 *               quantiser of section 2.3 / Eq. 1 with INT8 codes; the same
 *               per-tensor scaling with the FP8 formats).
 * Cvt rounds the float32 value of its argument (saturating), as in Eq. 10;
 * scalars that a receiver would use (alpha, s, Delta) are float32.  The
 * output x' is in double (no output rounding).
 */
#define ORACLE_VARIANT_TACO 0
#define ORACLE_VARIANT_DIRECT 1
#define ORACLE_VARIANT_DS 2
#define ORACLE_VARIANT_ASH 3
#define ORACLE_VARIANT_HADAMARD 4
#define ORACLE_VARIANT_TENSOR 5

static uint8_t cvt_fmt(double v, int fmt)
{
    float f = (float)v;
    if (f == 0.0f) f = 0.0f;                       /* zero carries no sign */
    return encode_fmt(f, fmt);
}

int taco_oracle_roundtrip_variant(const uint16_t *x, int64_t n, int B, int variant,
                                  int fmt, double tau, double eps, double *out)
{
    if (!valid_block(B) || !valid_fmt(fmt) || n < 0 || n % B) return -1;
    if (variant < ORACLE_VARIANT_TACO || variant > ORACLE_VARIANT_TENSOR) return -1;
    const double qmax = taco_oracle_qmax(fmt);
    const double c = 1.0 / sqrt((double)B);
    double tensor_max = 0.0;
    for (int64_t i = 0; i < n; ++i) tensor_max = fmax(tensor_max, fabs(bf16_to_double(x[i])));
    const float delta = (float)(tensor_max / qmax);
    double G[ORACLE_MAX_BLOCK], Z[ORACLE_MAX_BLOCK];
    uint8_t q[ORACLE_MAX_BLOCK];
    for (int64_t k = 0; k < n / B; ++k) {
        const uint16_t *xb = x + k * B;
        double *ob = out + k * B;
        for (int j = 0; j < B; ++j) G[j] = bf16_to_double(xb[j]);
        switch (variant) {
        case ORACLE_VARIANT_TACO: {
            float a32, s32;
            double a;
            ash_block_f64(G, B, tau, eps, &a, NULL, Z);
            quantise_block(Z, a, B, fmt, q, &a32, &s32);
            reconstruct_block(q, a32, s32, B, fmt, ob);
            break;
        }
        case ORACLE_VARIANT_DIRECT:
            for (int j = 0; j < B; ++j) ob[j] = decode_fmt(cvt_fmt(G[j], fmt), fmt);
            break;
        case ORACLE_VARIANT_DS: {
            double m = 0.0;
            for (int j = 0; j < B; ++j) m = fmax(m, fabs(G[j]));
            const double s = m / qmax;
            const float s32 = (float)s;
            for (int j = 0; j < B; ++j) {
                double v = (s > 0.0) ? G[j] / s : 0.0;
                ob[j] = decode_fmt(cvt_fmt(v, fmt), fmt) * (double)s32;
            }
            break;
        }
        case ORACLE_VARIANT_ASH: {
            double a;
            ash_block_f64(G, B, tau, eps, &a, NULL, Z);
            const float a32 = (float)a;
            for (int j = 0; j < B; ++j) ob[j] = decode_fmt(cvt_fmt(Z[j], fmt), fmt);
            taco_oracle_fwht(ob, B);
            for (int j = 0; j < B; ++j) ob[j] = ob[j] * c / (double)a32;
            break;
        }
        case ORACLE_VARIANT_HADAMARD:
            memcpy(Z, G, sizeof(double) * (size_t)B);
            taco_oracle_fwht(Z, B);
            for (int j = 0; j < B; ++j) ob[j] = decode_fmt(cvt_fmt(Z[j] * c, fmt), fmt);
            taco_oracle_fwht(ob, B);
            for (int j = 0; j < B; ++j) ob[j] *= c;
            break;
        default: /* ORACLE_VARIANT_TENSOR */
            for (int j = 0; j < B; ++j) {
                double v = (tensor_max > 0.0) ? G[j] / (tensor_max / qmax) : 0.0;
                ob[j] = decode_fmt(cvt_fmt(v, fmt), fmt) * (double)delta;
            }
            break;
        }
    }
    return 0;
}

/*
 * Round-trip fidelity of x' against the reference x (n values), as the GIFT
 * page defines it (Eq. 21): out[0] = RelL2 = |x' - x|_2 / |x|_2,
 * out[1] = Cos = <x', x> / (|x'|_2 |x|_2), out[2] = MaxErr = |x' - x|_inf,
 * out[3] = MSE = |x' - x|_2^2 / n.  Sums in double, in element order.
 */
int taco_oracle_fidelity(const double *ref, const double *got, int64_t n, double *out)
{
    if (n <= 0) return -1;
    double se = 0.0, sr = 0.0, sg = 0.0, sd = 0.0, me = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double d = got[i] - ref[i];
        se += d * d;
        sr += ref[i] * ref[i];
        sg += got[i] * got[i];
        sd += got[i] * ref[i];
        me = fmax(me, fabs(d));
    }
    out[0] = (sr > 0.0) ? sqrt(se) / sqrt(sr) : sqrt(se);
    out[1] = (sr > 0.0 && sg > 0.0) ? sd / (sqrt(sg) * sqrt(sr)) : 0.0;
    out[2] = me;
    out[3] = se / (double)n;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Self-check mode: the ASH round trip with quantisation left out            */
/* ------------------------------------------------------------------------ */

/*
 * Z from Eq. 8 fed straight into Eq. 12-13 (Z-hat = Z): returns the
 * reconstructed block in double.  In exact arithmetic this is x itself.
 */
int taco_oracle_roundtrip_noquant(const uint16_t *x, int B, double tau,
                                  double eps, double *out)
{
    double a;
    if (taco_oracle_ash_block(x, B, tau, eps, &a, NULL, out)) return -1;
    taco_oracle_fwht(out, B);
    double c = 1.0 / sqrt((double)B);
    for (int j = 0; j < B; ++j) out[j] = out[j] * c / a;
    return 0;
}
