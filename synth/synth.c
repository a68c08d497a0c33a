/*
 * Seeded synthetic inputs for the TACO operator (shared by the GPU tests,
 * the oracle tests and the benchmark).  This file holds no arithmetic of the
 * compression method: it only draws bf16 tensors whose shape follows the
 * TP intermediate tensors the TACO paper describes (section 3.1 and Figure 4:
 * zero-centred, dense near zero, with a long tail and outlier channels).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: draw i of stream s under seed S is the SplitMix64 output
 * function applied to  key(S, s) + (i + 1) * GAMMA,  where key(S, s) is
 * itself a SplitMix64 output of S and s.  Every element is therefore a pure
 * function of (seed, stream, element index), independent of thread count.
 *
 * Element recipe, in this order (double precision, then one rounding):
 *   1. body draw (Laplace, normal, or a two-component normal mixture);
 *   2. with probability p_out the element is replaced by a Student-t(3)
 *      draw times out_scale  (t3 = Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3));
 *   3. the whole column is multiplied by chan_factor if it is one of the
 *      n_chan outlier columns (chosen by a seeded partial Fisher-Yates);
 *   4. with probability p_zero the element becomes exactly +0;
 *   5. round to bfloat16 (via binary32, nearest-even at each step).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -pthread synth.c -o libtaco_synth.so -lm
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream)
{
    return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ull) + stream * GAMMA);
}

/* Uniform in the open interval (0, 1), 53 random bits. */
static inline double u01(uint64_t key, uint64_t i)
{
    uint64_t r = mix64(key + (i + 1) * GAMMA);
    return ((double)(r >> 11) + 0.5) * 0x1.0p-53;
}

enum { BODY_LAPLACE = 0, BODY_NORMAL = 1, BODY_MIXTURE = 2 };

/* Streams: one per purpose, so that adding a feature never moves another. */
enum {
    S_BODY_A = 0, S_BODY_B = 1, S_BODY_C = 2,
    S_OUT_P = 3, S_OUT_Z = 4,      /* S_OUT_Z .. S_OUT_Z + 7: t3 normals */
    S_ZERO = 12, S_CHAN = 13
};

static inline double normal(uint64_t ka, uint64_t kb, uint64_t i)
{
    double u1 = u01(ka, i), u2 = u01(kb, i);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

typedef struct {
    uint64_t seed;
    int64_t rows, cols;
    int body;
    double p1, p2, p3;             /* Laplace b | normal std | mixture: w, std1, std2 */
    double p_out, out_scale;
    double p_zero;
    const uint8_t *chan_mask;      /* cols entries, 1 = outlier column */
    double chan_factor;
    uint16_t *out;
    int64_t row0, row1;
} job_t;

static uint16_t double_to_bf16_bits(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)(u >> 16);  /* inf */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static void *run(void *arg)
{
    job_t *J = (job_t *)arg;
    uint64_t ka = stream_key(J->seed, S_BODY_A), kb = stream_key(J->seed, S_BODY_B);
    uint64_t kc = stream_key(J->seed, S_BODY_C), kp = stream_key(J->seed, S_OUT_P);
    uint64_t kz = stream_key(J->seed, S_ZERO);
    uint64_t kt[8];
    for (int t = 0; t < 8; ++t) kt[t] = stream_key(J->seed, S_OUT_Z + t);
    for (int64_t r = J->row0; r < J->row1; ++r) {
        for (int64_t c = 0; c < J->cols; ++c) {
            uint64_t i = (uint64_t)(r * J->cols + c);
            double v;
            if (J->body == BODY_LAPLACE) {
                double u = u01(ka, i);
                v = (u < 0.5) ? J->p1 * log(2.0 * u) : -J->p1 * log(2.0 * (1.0 - u));
            } else if (J->body == BODY_NORMAL) {
                v = J->p1 * normal(ka, kb, i);
            } else {
                double sd = (u01(kc, i) < J->p1) ? J->p2 : J->p3;
                v = sd * normal(ka, kb, i);
            }
            if (J->p_out > 0.0 && u01(kp, i) < J->p_out) {
                double z0 = normal(kt[0], kt[1], i), z1 = normal(kt[2], kt[3], i);
                double z2 = normal(kt[4], kt[5], i), z3 = normal(kt[6], kt[7], i);
                v = J->out_scale * z0 / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
            }
            if (J->chan_mask && J->chan_mask[c]) v *= J->chan_factor;
            if (J->p_zero > 0.0 && u01(kz, i) < J->p_zero) v = 0.0;
            J->out[i] = double_to_bf16_bits(v);
        }
    }
    return NULL;
}

/* Seeded choice of k distinct columns out of cols (partial Fisher-Yates). */
int taco_synth_pick_columns(uint64_t seed, int64_t cols, int64_t k, int64_t *picked)
{
    if (k < 0 || k > cols) return -1;
    int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)cols);
    if (!perm) return -2;
    for (int64_t i = 0; i < cols; ++i) perm[i] = i;
    uint64_t key = stream_key(seed, S_CHAN);
    for (int64_t i = 0; i < k; ++i) {
        int64_t j = i + (int64_t)(u01(key, (uint64_t)i) * (double)(cols - i));
        if (j >= cols) j = cols - 1;
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
        picked[i] = perm[i];
    }
    free(perm);
    return 0;
}

int taco_synth_generate(uint64_t seed, int64_t rows, int64_t cols, int body,
                        double p1, double p2, double p3,
                        double p_out, double out_scale,
                        int64_t n_chan, double chan_factor, double p_zero,
                        uint16_t *out, int nthreads)
{
    if (rows < 0 || cols <= 0 || !out) return -1;
    uint8_t *mask = NULL;
    if (n_chan > 0) {
        int64_t *picked = (int64_t *)malloc(sizeof(int64_t) * (size_t)n_chan);
        mask = (uint8_t *)calloc((size_t)cols, 1);
        if (!picked || !mask) { free(picked); free(mask); return -2; }
        if (taco_synth_pick_columns(seed, cols, n_chan, picked)) {
            free(picked); free(mask); return -1;
        }
        for (int64_t i = 0; i < n_chan; ++i) mask[picked[i]] = 1;
        free(picked);
    }
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
    job_t jobs[256];
    pthread_t th[256];
    for (int t = 0; t < nthreads; ++t) {
        job_t *J = &jobs[t];
        J->seed = seed; J->rows = rows; J->cols = cols; J->body = body;
        J->p1 = p1; J->p2 = p2; J->p3 = p3;
        J->p_out = p_out; J->out_scale = out_scale; J->p_zero = p_zero;
        J->chan_mask = mask; J->chan_factor = chan_factor; J->out = out;
        J->row0 = rows * t / nthreads; J->row1 = rows * (t + 1) / nthreads;
    }
    int created[256] = {0};
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run, &jobs[t]) == 0) created[t] = 1;
        else run(&jobs[t]);               /* no thread: do the rows here */
    run(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (created[t]) pthread_join(th[t], NULL);
    free(mask);
    return 0;
}
