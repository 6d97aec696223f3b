/*
 * kda_oracle_body.h -- the token-by-token KDA recurrence, written once and
 * instantiated for double and float by kda_oracle.c (REAL, EXPF, SFX).
 *
 * TEST INFRASTRUCTURE ONLY (see kda_oracle.h).
 *
 * One step for one head, on the state S (Dk x Dv, row i = key channel):
 *
 *   1. retain : S <- Diag(alpha_t) S, alpha_t[i] = exp(log_alpha_t[i])
 *   2. recall : p = S^T k_t                 (prediction for the new key)
 *   3. correct: S <- S + beta_t k_t (v_t - p)^T
 *   4. read   : o_t = S^T q_t               (after the token's own update)
 *
 * Steps 2-3 are the expansion of (I - beta k k^T) S' + beta k v^T with
 * S' = Diag(alpha) S: (I - beta k k^T) S' + beta k v^T
 *                   = S' + beta k (v - S'^T k)^T.
 * The order (decay first, then erase and write, then read) is the one of the
 * published KDA equation ("Kimi K3 Architecture Explained", Step 3, the
 * Diag(alpha_t) form; "From GPT-2 to Kimi K3", ch. 5, "Read the recurrence as
 * four verbs"); the recall/compare/correct reading of steps 2-3 is Step 2 of
 * the same blog ("The Delta Rule").
 */

/* Apply one token to the columns [j0, j1) of state S.  Columns are
 * independent: every value column j only ever reads column j of S. */
static void CAT(kda_step_, SFX)(REAL* S, int32_t Dk, int32_t Dv, int32_t j0,
                                int32_t j1, const REAL* q, const REAL* k,
                                const REAL* v, const REAL* log_alpha,
                                REAL beta, REAL* p, REAL* o) {
    int32_t i, j;
    /* 1. retain: scale row i by its own alpha */
    for (i = 0; i < Dk; ++i) {
        REAL a = EXPF(log_alpha[i]);
        REAL* row = S + (int64_t)i * Dv;
        for (j = j0; j < j1; ++j) row[j] *= a;
    }
    /* 2. recall: p = S^T k */
    for (j = j0; j < j1; ++j) p[j] = 0;
    for (i = 0; i < Dk; ++i) {
        const REAL* row = S + (int64_t)i * Dv;
        REAL ki = k[i];
        for (j = j0; j < j1; ++j) p[j] += row[j] * ki;
    }
    /* 3. correct: S += beta k (v - p)^T */
    for (i = 0; i < Dk; ++i) {
        REAL* row = S + (int64_t)i * Dv;
        REAL c = beta * k[i];
        for (j = j0; j < j1; ++j) row[j] += c * (v[j] - p[j]);
    }
    /* 4. read: o = S^T q */
    for (j = j0; j < j1; ++j) o[j] = 0;
    for (i = 0; i < Dk; ++i) {
        const REAL* row = S + (int64_t)i * Dv;
        REAL qi = q[i];
        for (j = j0; j < j1; ++j) o[j] += row[j] * qi;
    }
}

struct CAT(fwd_job_, SFX) {
    const REAL *q, *k, *v, *g, *beta, *h0;
    const int64_t* cu;
    int32_t N, H, Dk, Dv, dv_block, n_blocks;
    REAL *o, *hT;
    atomic_long next;
    long n_units;
};

static void CAT(fwd_unit_, SFX)(struct CAT(fwd_job_, SFX)* J, long unit) {
    const int32_t H = J->H, Dk = J->Dk, Dv = J->Dv;
    const int32_t blk = (int32_t)(unit % J->n_blocks);
    const long nh = unit / J->n_blocks;
    const int32_t h = (int32_t)(nh % H);
    const int32_t n = (int32_t)(nh / H);
    const int32_t j0 = blk * J->dv_block;
    const int32_t j1 = (j0 + J->dv_block < Dv) ? j0 + J->dv_block : Dv;
    REAL* S = (REAL*)calloc((size_t)Dk * Dv, sizeof(REAL));
    REAL* p = (REAL*)calloc((size_t)Dv, sizeof(REAL));
    int64_t t;
    int32_t i, j;
    if (!S || !p) { free(S); free(p); abort(); }
    if (J->h0) {
        const REAL* src = J->h0 + ((int64_t)n * H + h) * Dk * Dv;
        for (i = 0; i < Dk; ++i)
            for (j = j0; j < j1; ++j) S[(int64_t)i * Dv + j] = src[(int64_t)i * Dv + j];
    }
    for (t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const int64_t th = t * H + h;
        CAT(kda_step_, SFX)(S, Dk, Dv, j0, j1, J->q + th * Dk, J->k + th * Dk,
                            J->v + th * Dv, J->g + th * Dk, J->beta[th], p,
                            J->o + th * Dv);
    }
    if (J->hT) {
        REAL* dst = J->hT + ((int64_t)n * H + h) * Dk * Dv;
        for (i = 0; i < Dk; ++i)
            for (j = j0; j < j1; ++j) dst[(int64_t)i * Dv + j] = S[(int64_t)i * Dv + j];
    }
    free(S);
    free(p);
}

static void* CAT(fwd_worker_, SFX)(void* arg) {
    struct CAT(fwd_job_, SFX)* J = (struct CAT(fwd_job_, SFX)*)arg;
    for (;;) {
        long u = atomic_fetch_add(&J->next, 1);
        if (u >= J->n_units) break;
        CAT(fwd_unit_, SFX)(J, u);
    }
    return NULL;
}

int CAT(kda_oracle_fwd_, SFX)(const REAL* q, const REAL* k, const REAL* v,
                              const REAL* log_alpha, const REAL* beta,
                              const REAL* h0, const int64_t* cu_seqlens,
                              int32_t N, int64_t T_total, int32_t H, int32_t Dk,
                              int32_t Dv, REAL* o, REAL* h_T, int32_t dv_block,
                              int32_t nthreads) {
    struct CAT(fwd_job_, SFX) J;
    int64_t one[2];
    int32_t n;
    if (!q || !k || !v || !log_alpha || !beta || !o) return -1;
    if (N < 1 || T_total < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    if (!cu_seqlens) {
        if (N != 1) return -1;
        one[0] = 0;
        one[1] = T_total;
        cu_seqlens = one;
    }
    if (cu_seqlens[0] != 0 || cu_seqlens[N] != T_total) return -1;
    for (n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (dv_block <= 0 || dv_block > Dv) dv_block = Dv;
    J.q = q; J.k = k; J.v = v; J.g = log_alpha; J.beta = beta; J.h0 = h0;
    J.cu = cu_seqlens; J.N = N; J.H = H; J.Dk = Dk; J.Dv = Dv;
    J.dv_block = dv_block;
    J.n_blocks = (Dv + dv_block - 1) / dv_block;
    J.o = o; J.hT = h_T;
    atomic_init(&J.next, 0);
    J.n_units = (long)N * H * J.n_blocks;
    run_pool(CAT(fwd_worker_, SFX), &J, nthreads);
    return 0;
}

struct CAT(dec_job_, SFX) {
    const REAL *q, *k, *v, *g, *beta;
    REAL *S, *o, *p_all;
    int32_t H, Dk, Dv;
    atomic_long next;
    long n_units;
};

static void* CAT(dec_worker_, SFX)(void* arg) {
    struct CAT(dec_job_, SFX)* J = (struct CAT(dec_job_, SFX)*)arg;
    REAL* p = (REAL*)calloc((size_t)J->Dv, sizeof(REAL));
    if (!p) abort();
    for (;;) {
        long u = atomic_fetch_add(&J->next, 1);
        if (u >= J->n_units) break;
        CAT(kda_step_, SFX)(J->S + (int64_t)u * J->Dk * J->Dv, J->Dk, J->Dv, 0,
                            J->Dv, J->q + (int64_t)u * J->Dk,
                            J->k + (int64_t)u * J->Dk, J->v + (int64_t)u * J->Dv,
                            J->g + (int64_t)u * J->Dk, J->beta[u], p,
                            J->o + (int64_t)u * J->Dv);
    }
    free(p);
    return NULL;
}

int CAT(kda_oracle_decode_, SFX)(const REAL* q, const REAL* k, const REAL* v,
                                 const REAL* log_alpha, const REAL* beta,
                                 REAL* S, int32_t B, int32_t H, int32_t Dk,
                                 int32_t Dv, REAL* o, int32_t nthreads) {
    struct CAT(dec_job_, SFX) J;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return -1;
    if (B < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    J.q = q; J.k = k; J.v = v; J.g = log_alpha; J.beta = beta;
    J.S = S; J.o = o; J.p_all = NULL;
    J.H = H; J.Dk = Dk; J.Dv = Dv;
    atomic_init(&J.next, 0);
    J.n_units = (long)B * H;
    run_pool(CAT(dec_worker_, SFX), &J, nthreads);
    return 0;
}
