/*
 * Exhaustive check of an 8-bit code encoder (E4M3, E5M2 or INT8) over every
 * binary32 bit pattern.
 *
 * The expected code is derived independently of the encoder under test: the
 * caller passes the nvals non-negative finite values of the format in code
 * order (taken from a library decoder or written out), and each input is
 * placed between two neighbours by binary search; it must map to the nearer
 * one, to the even code index on an exact tie (the code whose mantissa, or
 * integer, is even), and to the largest code from the largest value upwards.
 * A negative input must give the positive input's code negated: the sign bit
 * set (sign-magnitude formats) or the two's complement of the code (INT8).
 * NaN must give a code >= nan_lo in its low seven bits (sign-magnitude), or
 * code 0 (two's complement).
 *
 * Build: gcc -O2 -fPIC -shared -pthread code_exhaustive.c -o libcode_exhaustive.so
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

typedef struct {
    uint64_t lo, hi;          /* non-negative patterns [lo, hi) */
    enc_fn enc;
    const double *vals;       /* nvals ascending values, codes 0..nvals-1 */
    int nvals, twos, nan_lo;
    int64_t bad;
    uint32_t first_bad;
} job_t;

static int expected(double v, const double *vals, int nvals)
{
    const int top = nvals - 1;
    if (v >= vals[top]) return top;
    int lo = 0, hi = top;                 /* vals[lo] <= v < vals[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (vals[mid] <= v) lo = mid; else hi = mid;
    }
    double m = 0.5 * (vals[lo] + vals[hi]);   /* exact in double */
    if (v < m) return lo;
    if (v > m) return hi;
    return (lo % 2 == 0) ? lo : hi;
}

static void *run(void *arg)
{
    job_t *J = (job_t *)arg;
    for (uint64_t p = J->lo; p < J->hi; ++p) {
        uint32_t u = (uint32_t)p;
        float f;
        memcpy(&f, &u, 4);
        uint8_t got = J->enc(f);
        uint32_t un = u | 0x80000000u;
        float fn;
        memcpy(&fn, &un, 4);
        uint8_t gotn = J->enc(fn);
        int ok;
        if (isnan(f)) {
            ok = J->twos ? (got == 0 && gotn == 0)
                         : ((got & 0x7F) >= J->nan_lo && (gotn & 0x7F) >= J->nan_lo);
        } else {
            int e = expected((double)f, J->vals, J->nvals);
            uint8_t en = J->twos ? (uint8_t)(-e) : (uint8_t)(e | 0x80);
            ok = (got == (uint8_t)e) && (gotn == en);
        }
        if (!ok) {
            if (J->bad == 0) J->first_bad = u;
            J->bad++;
        }
    }
    return NULL;
}

/* Returns the number of failing non-negative patterns in [lo, hi). */
int64_t code_check_range(uint64_t lo, uint64_t hi, void *enc, const double *vals, int nvals,
                         int twos, int nan_lo, int nthreads, uint32_t *first_bad)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    job_t jobs[64];
    pthread_t th[64];
    int created[64] = {0};
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].lo = lo + (hi - lo) * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].hi = lo + (hi - lo) * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].enc = (enc_fn)enc;
        jobs[t].vals = vals;
        jobs[t].nvals = nvals;
        jobs[t].twos = twos;
        jobs[t].nan_lo = nan_lo;
        jobs[t].bad = 0;
        jobs[t].first_bad = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run, &jobs[t]) == 0) created[t] = 1;
        else run(&jobs[t]);
    run(&jobs[0]);
    int64_t bad = 0;
    *first_bad = 0;
    for (int t = 1; t < nthreads; ++t)
        if (created[t]) pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t) {
        if (jobs[t].bad && bad == 0) *first_bad = jobs[t].first_bad;
        bad += jobs[t].bad;
    }
    return bad;
}
