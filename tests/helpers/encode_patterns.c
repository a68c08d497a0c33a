/*
 * Encode the binary32 values whose bit patterns are lo..hi-1 with a given
 * scalar encoder, on several threads (test helper for the GPU codec sweep).
 *
 * Build: gcc -O2 -fPIC -shared -pthread encode_patterns.c -o libencode_patterns.so
 */
#include <pthread.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float);

typedef struct {
    uint64_t lo, hi, base;
    enc_fn enc;
    uint8_t *out;
} job_t;

static void *run(void *arg)
{
    job_t *J = (job_t *)arg;
    for (uint64_t p = J->lo; p < J->hi; ++p) {
        uint32_t u = (uint32_t)p;
        float f;
        memcpy(&f, &u, 4);
        J->out[p - J->base] = J->enc(f);
    }
    return NULL;
}

void encode_pattern_range(uint64_t lo, uint64_t hi, void *enc, uint8_t *out, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    job_t jobs[64];
    pthread_t th[64];
    int created[64] = {0};
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].lo = lo + (hi - lo) * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].hi = lo + (hi - lo) * (uint64_t)(t + 1) / (uint64_t)nthreads;
        jobs[t].base = lo;
        jobs[t].enc = (enc_fn)enc;
        jobs[t].out = out;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run, &jobs[t]) == 0) created[t] = 1;
        else run(&jobs[t]);
    run(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (created[t]) pthread_join(th[t], NULL);
}
