/*
 * Exhaustive check of an E4M3 encoder over every binary32 bit pattern.
 *
 * The expected code is derived independently of the encoder under test: the
 * caller passes the 127 non-negative finite E4M3 values in code order (taken
 * from a library decoder), and each input is placed between two neighbours by
 * binary search; it must map to the nearer one, to the code with a zero
 * mantissa LSB on an exact tie, and to 0x7E (448) from 448 upwards.  Negative
 * inputs must give the positive input's code with the sign bit set; NaN must
 * give a NaN code.
 *
 * Build: gcc -O2 -fPIC -shared -pthread e4m3_exhaustive.c -o libe4m3_exhaustive.so
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

typedef struct {
    uint64_t lo, hi;          /* non-negative patterns [lo, hi) */
    enc_fn enc;
    const double *vals;       /* 127 ascending values, codes 0x00..0x7E */
    int64_t bad;
    uint32_t first_bad;
} job_t;

static uint8_t expected(double v, const double *vals)
{
    if (v >= vals[126]) return 0x7E;
    int lo = 0, hi = 126;                 /* vals[lo] <= v < vals[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (vals[mid] <= v) lo = mid; else hi = mid;
    }
    double m = 0.5 * (vals[lo] + vals[hi]);   /* exact in double */
    if (v < m) return (uint8_t)lo;
    if (v > m) return (uint8_t)hi;
    return (uint8_t)((lo % 2 == 0) ? lo : hi);
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
            ok = ((got & 0x7F) == 0x7F) && ((gotn & 0x7F) == 0x7F);
        } else {
            uint8_t e = expected((double)f, J->vals);
            ok = (got == e) && (gotn == (uint8_t)(e | 0x80));
        }
        if (!ok) {
            if (J->bad == 0) J->first_bad = u;
            J->bad++;
        }
    }
    return NULL;
}

/* Returns the number of failing non-negative patterns in [lo, hi). */
int64_t e4m3_check_range(uint64_t lo, uint64_t hi, void *enc, const double *vals,
                         int nthreads, uint32_t *first_bad)
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
        jobs[t].bad = 0;
        jobs[t].first_bad = 0;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run, &jobs[t]) == 0) created[t] = 1;
        else run(&jobs[t]);
    run(&jobs[0]);
    int64_t bad = 0;
    *first_bad = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (t > 0 && created[t]) pthread_join(th[t], NULL);
    }
    for (int t = 0; t < nthreads; ++t) {
        if (jobs[t].bad && bad == 0) *first_bad = jobs[t].first_bad;
        bad += jobs[t].bad;
    }
    return bad;
}
