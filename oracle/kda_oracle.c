/*
 * kda_oracle.c -- plain CPU oracle for Kimi Delta Attention.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Built with gcc
 * (plain C11 + POSIX threads), no SIMD intrinsics, no blocking or fusion.
 *
 * The recurrence is written once in kda_oracle_body.h and instantiated here
 * in double (the parity reference) and float (the timed CPU baseline).
 */
#include "kda_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdatomic.h>
#include <stdlib.h>

#define CAT_(a, b) a##b
#define CAT(a, b) CAT_(a, b)

/* Run fn(arg) on nthreads threads (the calling thread is one of them). */
static void run_pool(void* (*fn)(void*), void* arg, int32_t nthreads) {
    pthread_t* th;
    int32_t i, started = 0;
    if (nthreads <= 1) {
        fn(arg);
        return;
    }
    th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!th) {
        fn(arg);
        return;
    }
    /* Workers pull units from a shared counter, so a thread that fails to
     * start only means fewer workers, never a lost unit. */
    for (i = 0; i < nthreads - 1; ++i)
        if (pthread_create(&th[started], NULL, fn, arg) == 0) ++started;
    fn(arg);
    for (i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
}

#define REAL double
#define EXPF exp
#define SFX f64
#include "kda_oracle_body.h"
#undef REAL
#undef EXPF
#undef SFX

#define REAL float
#define EXPF expf
#define SFX f32
#include "kda_oracle_body.h"
#undef REAL
#undef EXPF
#undef SFX
