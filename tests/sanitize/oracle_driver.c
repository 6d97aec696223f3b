/*
 * oracle_driver.c -- runs the CPU oracle (oracle/kda_oracle.c, linked in)
 * built with AddressSanitizer and UndefinedBehaviorSanitizer, on small packed
 * problems that reach every branch of its loops: empty and one-token
 * sequences, non-square states, value-column blocks, several threads, h0
 * present and absent, h_T not stored, decode.  Each run is also checked
 * against something other than the oracle itself, so the sanitized build is
 * exercised on correct results:
 *   - an explicit-matrix evaluation of the KDA update, written here, with
 *     M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) as a Dk x Dk matrix
 *     ("Kimi K3 Architecture Explained", Step 3, the KDA equation);
 *   - beta = 0: every row decays by exp(sum of its log alphas) ("From
 *     GPT-2 to Kimi K3", ch. 4, a retention product over time);
 *   - resume: a sequence split in two gives the same result when the second
 *     part starts from the first part's h_T;
 *   - decode = a one-token prefill; threads and column blocks do not change
 *     a single bit; bad offsets are rejected.
 * Exit status 0 when every check passes; the sanitizers abort on the first
 * memory or undefined-behaviour error.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

static int failures = 0;

#define CHECK(cond, ...)                            \
    do {                                            \
        if (!(cond)) {                              \
            fprintf(stderr, "FAIL: " __VA_ARGS__);  \
            fprintf(stderr, "\n");                  \
            ++failures;                             \
        }                                           \
    } while (0)

/* xorshift64* uniform in [0, 1) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void) { /* sum of 12 uniforms: mean 6, variance 1 */
    double s = 0;
    for (int i = 0; i < 12; ++i) s += urand();
    return s - 6.0;
}

typedef struct {
    int64_t T;
    int32_t N, H, Dk, Dv;
    double *q, *k, *v, *g, *b, *h0;
    int64_t* cu;
} Problem;

static double* alloc_d(size_t n) {
    double* p = (double*)calloc(n ? n : 1, sizeof(double));
    if (!p) abort();
    return p;
}

static Problem make_problem(const int64_t* lens, int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                            int with_h0, double beta_const) {
    Problem p;
    p.N = N;
    p.H = H;
    p.Dk = Dk;
    p.Dv = Dv;
    p.cu = (int64_t*)calloc((size_t)N + 1, sizeof(int64_t));
    for (int32_t n = 0; n < N; ++n) p.cu[n + 1] = p.cu[n] + lens[n];
    p.T = p.cu[N];
    const size_t tk = (size_t)p.T * H * Dk, tv = (size_t)p.T * H * Dv;
    p.q = alloc_d(tk);
    p.k = alloc_d(tk);
    p.g = alloc_d(tk);
    p.v = alloc_d(tv);
    p.b = alloc_d((size_t)p.T * H);
    for (size_t r = 0; r < (size_t)p.T * H; ++r) {
        double nq = 0, nk = 0;
        for (int32_t i = 0; i < Dk; ++i) {
            p.q[r * Dk + i] = nrand();
            p.k[r * Dk + i] = nrand();
            nq += p.q[r * Dk + i] * p.q[r * Dk + i];
            nk += p.k[r * Dk + i] * p.k[r * Dk + i];
            p.g[r * Dk + i] = -5.0 / (1.0 + exp(-nrand()));
        }
        for (int32_t i = 0; i < Dk; ++i) {
            p.q[r * Dk + i] /= sqrt(nq);
            p.k[r * Dk + i] /= sqrt(nk);
        }
        for (int32_t j = 0; j < Dv; ++j) p.v[r * Dv + j] = nrand();
        p.b[r] = beta_const >= 0 ? beta_const : 1.0 / (1.0 + exp(-nrand()));
    }
    p.h0 = NULL;
    if (with_h0) {
        const size_t ns = (size_t)N * H * Dk * Dv;
        p.h0 = alloc_d(ns);
        for (size_t i = 0; i < ns; ++i) p.h0[i] = 0.3 * nrand();
    }
    return p;
}

static void free_problem(Problem* p) {
    free(p->q);
    free(p->k);
    free(p->v);
    free(p->g);
    free(p->b);
    free(p->h0);
    free(p->cu);
}

static double max_abs_diff(const double* a, const double* b, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) m = fmax(m, fabs(a[i] - b[i]));
    return m;
}

/* Explicit matrices: S <- M S + beta k v^T with M = (I - beta k k^T) Diag(alpha),
 * then o = S^T q.  Separate from the oracle's loop (which forms no matrix). */
static void explicit_eval(const Problem* p, double* o, double* hT) {
    const int32_t Dk = p->Dk, Dv = p->Dv, H = p->H;
    double* S = alloc_d((size_t)Dk * Dv);
    double* S2 = alloc_d((size_t)Dk * Dv);
    double* M = alloc_d((size_t)Dk * Dk);
    for (int32_t n = 0; n < p->N; ++n)
        for (int32_t h = 0; h < H; ++h) {
            for (int32_t i = 0; i < Dk * Dv; ++i)
                S[i] = p->h0 ? p->h0[((size_t)n * H + h) * Dk * Dv + i] : 0.0;
            for (int64_t t = p->cu[n]; t < p->cu[n + 1]; ++t) {
                const size_t r = (size_t)t * H + h;
                const double* k = p->k + r * Dk;
                const double* v = p->v + r * Dv;
                const double* g = p->g + r * Dk;
                const double bt = p->b[r];
                for (int32_t i = 0; i < Dk; ++i)
                    for (int32_t c = 0; c < Dk; ++c)
                        M[i * Dk + c] = ((i == c ? 1.0 : 0.0) - bt * k[i] * k[c]) * exp(g[c]);
                for (int32_t i = 0; i < Dk; ++i)
                    for (int32_t j = 0; j < Dv; ++j) {
                        double acc = bt * k[i] * v[j];
                        for (int32_t c = 0; c < Dk; ++c) acc += M[i * Dk + c] * S[c * Dv + j];
                        S2[i * Dv + j] = acc;
                    }
                memcpy(S, S2, sizeof(double) * (size_t)Dk * Dv);
                for (int32_t j = 0; j < Dv; ++j) {
                    double acc = 0;
                    for (int32_t i = 0; i < Dk; ++i) acc += S[i * Dv + j] * p->q[r * Dk + i];
                    o[r * Dv + j] = acc;
                }
            }
            memcpy(hT + ((size_t)n * H + h) * Dk * Dv, S, sizeof(double) * (size_t)Dk * Dv);
        }
    free(S);
    free(S2);
    free(M);
}

static void run_case(const int64_t* lens, int32_t N, int32_t H, int32_t Dk, int32_t Dv,
                     int with_h0) {
    Problem p = make_problem(lens, N, H, Dk, Dv, with_h0, -1.0);
    const size_t no = (size_t)p.T * H * Dv, ns = (size_t)N * H * Dk * Dv;
    double *o = alloc_d(no), *hT = alloc_d(ns), *o2 = alloc_d(no), *hT2 = alloc_d(ns);
    double *ox = alloc_d(no), *hx = alloc_d(ns);
    int rc = kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, p.cu, N, p.T, H, Dk, Dv, o, hT,
                                0, 1);
    CHECK(rc == 0, "fwd_f64 rc %d", rc);
    explicit_eval(&p, ox, hx);
    CHECK(max_abs_diff(o, ox, no) < 1e-12, "o vs explicit matrices (T=%lld)", (long long)p.T);
    CHECK(max_abs_diff(hT, hx, ns) < 1e-12, "h_T vs explicit matrices");
    /* threads and value-column blocks change no bit */
    rc = kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, p.cu, N, p.T, H, Dk, Dv, o2, hT2,
                            Dv > 1 ? Dv / 2 : 0, 5);
    CHECK(rc == 0 && memcmp(o, o2, no * sizeof(double)) == 0 &&
              memcmp(hT, hT2, ns * sizeof(double)) == 0,
          "threads / column blocks changed the result");
    /* h_T not stored */
    rc = kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, p.cu, N, p.T, H, Dk, Dv, o2, NULL,
                            3, 3);
    CHECK(rc == 0 && memcmp(o, o2, no * sizeof(double)) == 0, "h_T = NULL");
    /* the float instantiation, on the same values */
    {
        const size_t tk = (size_t)p.T * H * Dk, tv = (size_t)p.T * H * Dv;
        float *fq = malloc(sizeof(float) * (tk ? tk : 1)), *fk = malloc(sizeof(float) * (tk ? tk : 1));
        float *fg = malloc(sizeof(float) * (tk ? tk : 1)), *fv = malloc(sizeof(float) * (tv ? tv : 1));
        float *fb = malloc(sizeof(float) * ((size_t)p.T * H + 1)), *fo = malloc(sizeof(float) * (no ? no : 1));
        float *fh0 = with_h0 ? malloc(sizeof(float) * ns) : NULL, *fhT = malloc(sizeof(float) * ns);
        for (size_t i = 0; i < tk; ++i) {
            fq[i] = (float)p.q[i];
            fk[i] = (float)p.k[i];
            fg[i] = (float)p.g[i];
        }
        for (size_t i = 0; i < tv; ++i) fv[i] = (float)p.v[i];
        for (size_t i = 0; i < (size_t)p.T * H; ++i) fb[i] = (float)p.b[i];
        if (fh0)
            for (size_t i = 0; i < ns; ++i) fh0[i] = (float)p.h0[i];
        rc = kda_oracle_fwd_f32(fq, fk, fv, fg, fb, fh0, p.cu, N, p.T, H, Dk, Dv, fo, fhT, 0, 2);
        CHECK(rc == 0, "fwd_f32 rc %d", rc);
        double e = 0;
        for (size_t i = 0; i < no; ++i) e = fmax(e, fabs((double)fo[i] - o[i]));
        for (size_t i = 0; i < ns; ++i) e = fmax(e, fabs((double)fhT[i] - hT[i]));
        CHECK(e < 1e-4, "f32 vs f64 %.3e", e);
        free(fq);
        free(fk);
        free(fg);
        free(fv);
        free(fb);
        free(fo);
        free(fh0);
        free(fhT);
    }
    free(o);
    free(hT);
    free(o2);
    free(hT2);
    free(ox);
    free(hx);
    free_problem(&p);
}

static void beta_zero_case(void) {
    const int64_t lens[2] = {9, 4};
    const int32_t N = 2, H = 2, Dk = 6, Dv = 5;
    Problem p = make_problem(lens, N, H, Dk, Dv, 1, 0.0);
    const size_t ns = (size_t)N * H * Dk * Dv;
    double *o = alloc_d((size_t)p.T * H * Dv), *hT = alloc_d(ns);
    CHECK(kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, p.cu, N, p.T, H, Dk, Dv, o, hT, 0,
                             2) == 0,
          "beta = 0 rc");
    double e = 0;
    for (int32_t n = 0; n < N; ++n)
        for (int32_t h = 0; h < H; ++h)
            for (int32_t i = 0; i < Dk; ++i) {
                double gs = 0;
                for (int64_t t = p.cu[n]; t < p.cu[n + 1]; ++t) gs += p.g[((size_t)t * H + h) * Dk + i];
                for (int32_t j = 0; j < Dv; ++j) {
                    const size_t idx = (((size_t)n * H + h) * Dk + i) * Dv + j;
                    e = fmax(e, fabs(hT[idx] - exp(gs) * p.h0[idx]));
                }
            }
    CHECK(e < 1e-14, "beta = 0 closed form %.3e", e);
    free(o);
    free(hT);
    free_problem(&p);
}

static void resume_and_decode_case(void) {
    const int64_t whole[1] = {11};
    const int32_t H = 3, Dk = 8, Dv = 4;
    Problem p = make_problem(whole, 1, H, Dk, Dv, 1, -1.0);
    const size_t ns = (size_t)H * Dk * Dv;
    double *o = alloc_d((size_t)11 * H * Dv), *hT = alloc_d(ns);
    CHECK(kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, NULL, 1, 11, H, Dk, Dv, o, hT, 0,
                             1) == 0,
          "resume whole rc");
    /* first 7 tokens, then the last 4 from its state */
    double *o1 = alloc_d((size_t)11 * H * Dv), *h1 = alloc_d(ns), *h2 = alloc_d(ns);
    CHECK(kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, p.h0, NULL, 1, 7, H, Dk, Dv, o1, h1, 0,
                             1) == 0,
          "resume part 1 rc");
    const size_t rk = (size_t)7 * H * Dk, rv = (size_t)7 * H * Dv;
    CHECK(kda_oracle_fwd_f64(p.q + rk, p.k + rk, p.v + rv, p.g + rk, p.b + 7 * H, h1, NULL, 1, 4,
                             H, Dk, Dv, o1 + rv, h2, 0, 1) == 0,
          "resume part 2 rc");
    CHECK(max_abs_diff(o, o1, (size_t)11 * H * Dv) < 1e-13 && max_abs_diff(hT, h2, ns) < 1e-13,
          "resume");
    /* decode of token 7 from the state after 7 tokens = the prefill's token 7 */
    double* S = alloc_d(ns);
    double* od = alloc_d((size_t)H * Dv);
    memcpy(S, h1, ns * sizeof(double));
    CHECK(kda_oracle_decode_f64(p.q + rk, p.k + rk, p.v + rv, p.g + rk, p.b + 7 * H, S, 1, H, Dk,
                                Dv, od, 2) == 0,
          "decode rc");
    CHECK(max_abs_diff(od, o + rv, (size_t)H * Dv) < 1e-14, "decode = one prefill token");
    /* bad offsets are rejected without writing */
    int64_t bad[3] = {0, 9, 5};
    CHECK(kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, NULL, bad, 2, 11, H, Dk, Dv, o, NULL, 0,
                             1) != 0,
          "decreasing offsets accepted");
    int64_t past[2] = {0, 12};
    CHECK(kda_oracle_fwd_f64(p.q, p.k, p.v, p.g, p.b, NULL, past, 1, 11, H, Dk, Dv, o, NULL, 0,
                             1) != 0,
          "offsets past T accepted");
    free(o);
    free(hT);
    free(o1);
    free(h1);
    free(h2);
    free(S);
    free(od);
    free_problem(&p);
}

int main(void) {
    const int64_t l1[1] = {8};
    const int64_t l2[6] = {0, 1, 5, 0, 8, 3};
    const int64_t l3[3] = {2, 7, 1};
    run_case(l1, 1, 1, 4, 4, 0);
    run_case(l1, 1, 2, 7, 3, 1);    /* non-square state */
    run_case(l2, 6, 3, 5, 6, 1);    /* empty and one-token sequences */
    run_case(l3, 3, 2, 16, 16, 0);
    beta_zero_case();
    resume_and_decode_case();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
