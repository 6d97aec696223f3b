/*
 * kda_oracle.h -- plain CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never does.  It shares no code, header or constant with the
 * HIP library.
 *
 * What it computes, per head, token by token (the recurrence itself, no
 * chunking, no reordering):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,        alpha_t = exp(log_alpha_t)  (one per key channel)
 *
 * Sources: "Kimi K3 Architecture Explained" (Analytics Vidhya), Step 3
 * "Forgetting, Channel by Channel", the KDA equation with Diag(alpha_t);
 * "An infra-oriented diagram of Kimi K3", the Kimi Delta Attention card
 * (same equation); "From GPT-2 to Kimi K3, from first principles", ch. 5
 * ("Read the recurrence as four verbs": retain, erase, write, read) and
 * ch. 6 (the read-out uses the state after the token's own update).
 *
 * Layouts (all row-major, contiguous):
 *   q, k, log_alpha : [T_total, H, Dk]
 *   v, o            : [T_total, H, Dv]
 *   beta            : [T_total, H]
 *   h0, h_T, S      : [N (or B), H, Dk, Dv]; row i = key channel, column j =
 *                     value channel (Diag(alpha) scales rows).
 *   cu_seqlens      : [N + 1] host int64 offsets of packed sequences
 *                     (NULL = one sequence of T_total tokens, N must be 1).
 * h0 == NULL means a zero initial state; h_T == NULL means "do not store".
 *
 * Threads: independent (sequence, head, value-column block) units are run on
 * nthreads POSIX threads (nthreads <= 0 means 1).  Value columns are
 * independent in the recurrence, so splitting them changes no arithmetic.
 *
 * Return value: 0 on success, -1 on a bad argument (nothing written).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int kda_oracle_fwd_f64(const double* q, const double* k, const double* v,
                       const double* log_alpha, const double* beta,
                       const double* h0, const int64_t* cu_seqlens,
                       int32_t N, int64_t T_total, int32_t H, int32_t Dk,
                       int32_t Dv, double* o, double* h_T, int32_t dv_block,
                       int32_t nthreads);

int kda_oracle_fwd_f32(const float* q, const float* k, const float* v,
                       const float* log_alpha, const float* beta,
                       const float* h0, const int64_t* cu_seqlens, int32_t N,
                       int64_t T_total, int32_t H, int32_t Dk, int32_t Dv,
                       float* o, float* h_T, int32_t dv_block,
                       int32_t nthreads);

/* One recurrent step for B independent sequences, S updated in place. */
int kda_oracle_decode_f64(const double* q, const double* k, const double* v,
                          const double* log_alpha, const double* beta,
                          double* S, int32_t B, int32_t H, int32_t Dk,
                          int32_t Dv, double* o, int32_t nthreads);

int kda_oracle_decode_f32(const float* q, const float* k, const float* v,
                          const float* log_alpha, const float* beta, float* S,
                          int32_t B, int32_t H, int32_t Dk, int32_t Dv,
                          float* o, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
