// kda_api.cpp -- the C ABI of libkda.so (declared in include/kda.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so all error paths are reachable (and tested) without a GPU.
// Kernel launches are asynchronous on the caller's stream.
#include "kda.h"

#include <stdint.h>

#include <initializer_list>
#include <limits>

#include "kda_launch.h"

namespace {

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty spans overlap nothing
};

Span span(const void* p, uint64_t bytes) {
    Span s;
    if (p && bytes) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + bytes;
    }
    return s;
}

bool overlaps(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool overlaps_any(const Span& a, std::initializer_list<Span> others) {
    for (const Span& b : others)
        if (overlaps(a, b)) return true;
    return false;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_dtype(kda_dtype dt) { return dt == KDA_F32 || dt == KDA_BF16; }

uint64_t esize(kda_dtype dt) { return dt == KDA_F32 ? 4u : 2u; }

// Largest element count a single tensor may have (keeps byte sizes in range).
constexpr uint64_t kMaxElems = (uint64_t)1 << 56;

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_str(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL_ARG: return "KDA_ERR_NULL_ARG: a required pointer is NULL";
        case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: unsupported size or option";
        case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: dtype is not KDA_F32 or KDA_BF16";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a pointer is not suitably aligned";
        case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input or another output";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace too small";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE: a HIP call or kernel launch failed";
    }
    return "KDA_ERR_UNKNOWN";
}

size_t kda_chunk_fwd_workspace_size(int64_t T_total, int32_t N, int32_t H, int32_t Dk,
                                    int32_t Dv, kda_dtype dt) {
    (void)T_total;
    (void)N;
    (void)H;
    (void)Dk;
    (void)Dv;
    (void)dt;
    return 0;  // the fused chunk kernel keeps every intermediate on chip
}

namespace {

// Prefix snapshots requested by kda_chunk_fwd_snap (interval 0 = none).
struct SnapReq {
    int32_t interval = 0;
    const int32_t* snap_cu = nullptr;
    int64_t n_snap = 0;
    float* snap = nullptr;
};

kda_status chunk_fwd_impl(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* beta, const float* h0, const int32_t* cu_seqlens,
                          int32_t N, int64_t T_total, int32_t H, int32_t Dk, int32_t Dv,
                          kda_dtype dt, void* o, float* h_T, void* workspace,
                          size_t workspace_bytes, int32_t chunk, int32_t dv_split,
                          const SnapReq& sr, int32_t flags, hipStream_t stream,
                          bool check_only = false, float* h_T2 = nullptr) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (N < 1 || T_total < 0 || H < 1 || H > KDA_MAX_HEADS || Dk != kda::kHeadDim ||
        Dv != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    if (!cu_seqlens && N != 1) return KDA_ERR_BAD_SHAPE;
    const uint64_t row = (uint64_t)H * kda::kHeadDim;
    if ((uint64_t)T_total > kMaxElems / row) return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)N * (uint64_t)H * 8u > (uint64_t)std::numeric_limits<int32_t>::max())
        return KDA_ERR_BAD_SHAPE;
    if (chunk != 0 && chunk != 16 && chunk != 32) return KDA_ERR_BAD_SHAPE;
    if (dv_split != 0 && dv_split != 1 && dv_split != 2 && dv_split != 4) return KDA_ERR_BAD_SHAPE;
    if (sr.interval != 0) {
        if (sr.interval < 0 || sr.interval % kda::kSnapUnit != 0 || sr.n_snap < 0)
            return KDA_ERR_BAD_SHAPE;
        const uint64_t per = (uint64_t)H * kda::kHeadDim * kda::kHeadDim;
        if ((uint64_t)sr.n_snap > kMaxElems / per) return KDA_ERR_BAD_SHAPE;
    }

    const bool need_v = !(flags & kda::kChunkVZero), need_o = !(flags & kda::kChunkNoOutput);
    if (T_total > 0 && (!k || !log_alpha || !beta || (need_v && !v) || (need_o && (!q || !o))))
        return KDA_ERR_NULL_ARG;
    if (sr.n_snap > 0 &&
        (!sr.snap || (N > 1 && !sr.snap_cu && !(flags & kda::kChunkSnapSlots))))
        return KDA_ERR_NULL_ARG;
    if (sr.snap && !aligned(sr.snap, 16)) return KDA_ERR_MISALIGNED;
    if (sr.snap_cu && !aligned(sr.snap_cu, 4)) return KDA_ERR_MISALIGNED;

    for (const void* p : {q, k, v, log_alpha, (const void*)h0, (const void*)o,
                          (const void*)h_T, (const void*)workspace})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    // beta rows are H elements, so a token offset keeps only element alignment
    if (beta && !aligned(beta, esize(dt))) return KDA_ERR_MISALIGNED;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_MISALIGNED;

    const uint64_t es = esize(dt);
    const uint64_t nTok = (uint64_t)T_total * row;
    const uint64_t nState = (uint64_t)N * H * kda::kHeadDim * kda::kHeadDim;
    const Span sq = span(q, nTok * es), sk = span(k, nTok * es), sv = span(v, nTok * es),
               sg = span(log_alpha, nTok * es), sb = span(beta, (uint64_t)T_total * H * es),
               sh0 = span(h0, h0 ? nState * 4 : 0),
               scu = span(cu_seqlens, cu_seqlens ? ((uint64_t)N + 1) * 4 : 0),
               so = span(o, nTok * es), shT = span(h_T, h_T ? nState * 4 : 0),
               sws = span(workspace, workspace_bytes);
    const uint64_t snap_es = (flags & kda::kChunkSnapBf16) ? 2 : 4;
    const Span ssn = span(sr.snap, sr.snap ? (uint64_t)sr.n_snap * (nState / N) * snap_es : 0),
               sscu = span(sr.snap_cu, sr.snap_cu ? ((uint64_t)N + 1) * 4 : 0);
    if (overlaps_any(so, {sq, sk, sv, sg, sb, sh0, scu, sws, sscu})) return KDA_ERR_ALIAS;
    if (overlaps_any(shT, {sq, sk, sv, sg, sb, sh0, scu, so, sws, sscu})) return KDA_ERR_ALIAS;
    if (overlaps_any(ssn, {sq, sk, sv, sg, sb, sh0, scu, so, shT, sws, sscu}))
        return KDA_ERR_ALIAS;

    const size_t need = kda_chunk_fwd_workspace_size(T_total, N, H, Dk, Dv, dt);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;

    int c = 0, s = 0;
    kda::chunk_default_config((int)dt, T_total, N, H, &c, &s);
    if (chunk) c = chunk;
    if (dv_split) s = dv_split;
    if (!kda::chunk_config_supported((int)dt, c, s)) return KDA_ERR_BAD_SHAPE;
    if (sr.interval != 0 && sr.interval % c != 0) return KDA_ERR_BAD_SHAPE;
    // bf16 snapshots exist in the pipelined bf16 kernel only (chunk 16, split 1 or 2)
    if ((flags & kda::kChunkSnapBf16) && !(dt == KDA_BF16 && c == 16 && s <= 2))
        return KDA_ERR_BAD_SHAPE;
    // both summary passes in one launch: the bf16 pipelined kernel at split 2
    if ((flags & kda::kChunkDualBM) && !(dt == KDA_BF16 && c == 16 && s == 2 && sr.n_snap == 0))
        return KDA_ERR_BAD_SHAPE;
    if (check_only) return KDA_OK;

    kda::ChunkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.h0 = h0;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.T_total = T_total;
    a.H = H;
    a.o = o;
    a.h_T = h_T;
    a.snap.snap = sr.n_snap > 0 ? sr.snap : nullptr;
    a.snap.snap_cu = sr.snap_cu;
    a.snap.n_snap = sr.n_snap;
    a.snap.every_chunks = sr.interval > 0 ? sr.interval / kda::kSnapUnit : 1;
    a.flags = flags;
    a.h_T2 = h_T2;
    if (kda::launch_chunk(a, (int)dt, c, s, stream) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

}  // namespace

kda_status kda_chunk_fwd_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                            const void* beta, const float* h0, const int32_t* cu_seqlens,
                            int32_t N, int64_t T_total, int32_t H, int32_t Dk, int32_t Dv,
                            kda_dtype dt, void* o, float* h_T, void* workspace,
                            size_t workspace_bytes, int32_t chunk, int32_t dv_split,
                            hipStream_t stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                          o, h_T, workspace, workspace_bytes, chunk, dv_split, SnapReq{}, 0,
                          stream);
}

kda_status kda_chunk_fwd_snap(const void* q, const void* k, const void* v,
                              const void* log_alpha, const void* beta, const float* h0,
                              const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                              int32_t Dk, int32_t Dv, kda_dtype dt, void* o, float* h_T,
                              int32_t interval, const int32_t* snap_cu, int64_t n_snap,
                              float* snap, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (interval <= 0) return KDA_ERR_BAD_SHAPE;
    SnapReq sr;
    sr.interval = interval;
    sr.snap_cu = snap_cu;
    sr.n_snap = n_snap;
    sr.snap = snap;
    return chunk_fwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                          o, h_T, workspace, workspace_bytes, 0, 0, sr, 0, stream);
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* h0, const int32_t* cu_seqlens, int32_t N,
                         int64_t T_total, int32_t H, int32_t Dk, int32_t Dv, kda_dtype dt,
                         void* o, float* h_T, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return kda_chunk_fwd_ex(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                            o, h_T, workspace, workspace_bytes, 0, 0, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* log_alpha,
                           const void* beta, float* S, int32_t B, int32_t H, int32_t Dk,
                           int32_t Dv, kda_dtype dt, void* o, hipStream_t stream) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (B < 0 || H < 1 || H > KDA_MAX_HEADS || Dk != kda::kHeadDim || Dv != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)B * (uint64_t)H > (uint64_t)std::numeric_limits<int32_t>::max())
        return KDA_ERR_BAD_SHAPE;
    if (B > 0 && (!q || !k || !v || !log_alpha || !beta || !S || !o)) return KDA_ERR_NULL_ARG;
    for (const void* p : {q, k, v, log_alpha, (const void*)S, (const void*)o})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    if (beta && !aligned(beta, esize(dt))) return KDA_ERR_MISALIGNED;

    const uint64_t es = esize(dt);
    const uint64_t nVec = (uint64_t)B * H * kda::kHeadDim;
    const Span sq = span(q, nVec * es), sk = span(k, nVec * es), sv = span(v, nVec * es),
               sg = span(log_alpha, nVec * es), sb = span(beta, (uint64_t)B * H * es),
               sS = span(S, nVec * kda::kHeadDim * 4), so = span(o, nVec * es);
    if (overlaps_any(so, {sq, sk, sv, sg, sb, sS})) return KDA_ERR_ALIAS;
    if (overlaps_any(sS, {sq, sk, sv, sg, sb})) return KDA_ERR_ALIAS;
    if (B == 0) return KDA_OK;

    kda::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S = S;
    a.B = B;
    a.H = H;
    a.o = o;
    if (kda::launch_decode(a, (int)dt, stream) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

kda_status kda_segment_summary(const void* q, const void* k, const void* v,
                               const void* log_alpha, const void* beta,
                               const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                               int32_t Dk, int32_t Dv, kda_dtype dt, float* M, float* B,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!M && !B) return KDA_ERR_NULL_ARG;
    if (N >= 1 && H >= 1) {
        const uint64_t n = (uint64_t)N * H * kda::kHeadDim * kda::kHeadDim * 4;
        if (M && B && overlaps(span(M, n), span(B, n))) return KDA_ERR_ALIAS;
    }
    // B: the state reached from a zero start.  M: the transition, i.e. the
    // state reached from the identity with V = 0 (v is passed along only so
    // that M is checked against it; that pass never reads it).  Both passes
    // are validated before either is launched.
    const int32_t fB = kda::kChunkNoOutput;
    const int32_t fM = kda::kChunkNoOutput | kda::kChunkVZero | kda::kChunkH0Identity;
    kda_status st = KDA_OK;
    if (B)
        st = chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, cu_seqlens, N, T_total, H, Dk, Dv,
                            dt, nullptr, B, workspace, workspace_bytes, 0, 0, SnapReq{}, fB,
                            stream, true);
    if (st == KDA_OK && M)
        st = chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, cu_seqlens, N, T_total, H, Dk, Dv,
                            dt, nullptr, M, workspace, workspace_bytes, 0, 0, SnapReq{}, fM,
                            stream, true);
    if (st != KDA_OK) return st;
    // bf16 with both: one launch whose state waves run both passes over the
    // operands its prep waves form once (the B pass's arguments, validated
    // above, carry the M states as a second output)
    if (M && B && dt == KDA_BF16)
        return chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, cu_seqlens, N, T_total, H, Dk,
                              Dv, dt, nullptr, B, workspace, workspace_bytes, 16, 2, SnapReq{},
                              fB | kda::kChunkDualBM, stream, false, M);
    if (B)
        st = chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, cu_seqlens, N, T_total, H, Dk, Dv,
                            dt, nullptr, B, workspace, workspace_bytes, 0, 0, SnapReq{}, fB,
                            stream);
    if (st == KDA_OK && M)
        st = chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, cu_seqlens, N, T_total, H, Dk, Dv,
                            dt, nullptr, M, workspace, workspace_bytes, 0, 0, SnapReq{}, fM,
                            stream);
    return st;
}

kda_status kda_segment_scan(const float* M, const float* B, const float* h0, int32_t R,
                            int32_t H, int32_t Dk, int32_t Dv, float* S_in, float* S_final,
                            hipStream_t stream) {
    if (R < 0 || H < 1 || H > KDA_MAX_HEADS || Dk != kda::kHeadDim || Dv != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    const uint64_t per = (uint64_t)H * kda::kHeadDim * kda::kHeadDim;
    if ((uint64_t)R > kMaxElems / per) return KDA_ERR_BAD_SHAPE;
    if (R > 0 && (!M || !B || !S_in)) return KDA_ERR_NULL_ARG;
    for (const void* p : {(const void*)M, (const void*)B, (const void*)h0, (const void*)S_in,
                          (const void*)S_final})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    const Span sM = span(M, M ? (uint64_t)R * per * 4 : 0), sB = span(B, B ? (uint64_t)R * per * 4 : 0),
               sh0 = span(h0, h0 ? per * 4 : 0), sS = span(S_in, S_in ? (uint64_t)R * per * 4 : 0),
               sF = span(S_final, S_final ? per * 4 : 0);
    if (overlaps_any(sS, {sM, sB, sh0, sF})) return KDA_ERR_ALIAS;
    if (overlaps_any(sF, {sM, sB, sh0})) return KDA_ERR_ALIAS;
    if (R == 0 && !S_final) return KDA_OK;
    if (kda::launch_segment_scan(M, B, h0, R, H, S_in, S_final, stream) != hipSuccess)
        return KDA_ERR_DEVICE;
    return KDA_OK;
}

kda_status kda_decode_multi(const void* q, const void* k, const void* v, const void* log_alpha,
                            const void* beta, float* S, const int32_t* n_tok, int32_t B,
                            int32_t K, int32_t H, int32_t Dk, int32_t Dv, kda_dtype dt,
                            int32_t update_state, void* o, hipStream_t stream) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (B < 0 || K < 1 || H < 1 || H > KDA_MAX_HEADS || Dk != kda::kHeadDim ||
        Dv != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)B * (uint64_t)H > (uint64_t)std::numeric_limits<int32_t>::max())
        return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)B * (uint64_t)K * (uint64_t)H > kMaxElems / kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    if (B > 0 && (!q || !k || !v || !log_alpha || !beta || !S || !o)) return KDA_ERR_NULL_ARG;
    for (const void* p : {q, k, v, log_alpha, (const void*)S, (const void*)o})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    if (beta && !aligned(beta, esize(dt))) return KDA_ERR_MISALIGNED;
    if (n_tok && !aligned(n_tok, 4)) return KDA_ERR_MISALIGNED;

    const uint64_t es = esize(dt);
    const uint64_t nVec = (uint64_t)B * K * H * kda::kHeadDim;
    const uint64_t nState = (uint64_t)B * H * kda::kHeadDim * kda::kHeadDim;
    const Span sq = span(q, nVec * es), sk = span(k, nVec * es), sv = span(v, nVec * es),
               sg = span(log_alpha, nVec * es), sb = span(beta, (uint64_t)B * K * H * es),
               sS = span(S, nState * 4), so = span(o, nVec * es),
               sn = span(n_tok, n_tok ? (uint64_t)B * 4 : 0);
    if (overlaps_any(so, {sq, sk, sv, sg, sb, sS, sn})) return KDA_ERR_ALIAS;
    if (overlaps_any(sS, {sq, sk, sv, sg, sb, sn})) return KDA_ERR_ALIAS;
    if (B == 0) return KDA_OK;

    kda::DecodeMultiArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S = S;
    a.n_tok = n_tok;
    a.B = B;
    a.K = K;
    a.H = H;
    a.update_state = update_state ? 1 : 0;
    a.o = o;
    if (kda::launch_decode_multi(a, (int)dt, stream) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

size_t kda_chunk_bwd_workspace_size(int64_t T_total, int32_t N, int32_t H, int32_t Dk,
                                    int32_t Dv, kda_dtype dt) {
    if (!valid_dtype(dt) || T_total < 0 || N < 1 || H < 1 || Dk != kda::kHeadDim ||
        Dv != kda::kHeadDim)
        return 0;
    // the state after every chunk and its gradient, one table entry per
    // chunk, in the input dtype (fp32 for fp32 inputs, bf16 for bf16 inputs)
    return 2u * (size_t)kda::chunk_slots(T_total, N) * (size_t)H * kda::kHeadDim *
           kda::kHeadDim * esize(dt);
}

}  // extern "C"

namespace {

// kda_chunk_bwd's validation and launches.  no_workspace: validate every
// argument except the workspace (which the caller supplies afterwards);
// check_only: return after validation, before any HIP call; side_stream:
// the reverse recursion may run on the library's side stream (created on
// first use), else everything runs in order on `stream`.
kda_status chunk_bwd_impl(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* beta, const float* h0, const int32_t* cu_seqlens,
                          int32_t N, int64_t T_total, int32_t H, int32_t Dk, int32_t Dv,
                          kda_dtype dt, const void* dout, const float* dhT, void* dq, void* dk,
                          void* dv, void* dlog_alpha, void* dbeta, float* dh0, void* workspace,
                          size_t workspace_bytes, hipStream_t stream, bool check_only,
                          bool no_workspace, bool side_stream = true) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (N < 1 || T_total < 0 || H < 1 || H > KDA_MAX_HEADS || Dk != kda::kHeadDim ||
        Dv != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    const uint64_t row = (uint64_t)H * kda::kHeadDim;
    if ((uint64_t)T_total > kMaxElems / row) return KDA_ERR_BAD_SHAPE;
    const int64_t n_slots = kda::chunk_slots(T_total, N);
    const uint64_t per = (uint64_t)H * kda::kHeadDim * kda::kHeadDim;
    if ((uint64_t)n_slots > kMaxElems / per / 2) return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)n_slots * (uint64_t)H > (uint64_t)std::numeric_limits<uint32_t>::max())
        return KDA_ERR_BAD_SHAPE;
    if (T_total > 0 && (!q || !k || !v || !log_alpha || !beta || !dout || !dq || !dk || !dv ||
                        !dlog_alpha || !dbeta))
        return KDA_ERR_NULL_ARG;
    for (const void* p : {dout, (const void*)dhT, (const void*)dq, (const void*)dk,
                          (const void*)dv, (const void*)dlog_alpha, (const void*)dh0})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    if (dbeta && !aligned(dbeta, esize(dt))) return KDA_ERR_MISALIGNED;
    const size_t need = kda_chunk_bwd_workspace_size(T_total, N, H, Dk, Dv, dt);
    if (!no_workspace && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    void* states = workspace;
    void* dstates =
        workspace ? static_cast<unsigned char*>(workspace) + (size_t)n_slots * per * esize(dt)
                  : nullptr;

    // the forward pass again, keeping the state after every chunk (validates
    // the forward arguments and the state table against them)
    SnapReq sr;
    sr.interval = kda::kChunk;
    sr.n_snap = n_slots;
    sr.snap = static_cast<float*>(states);
    const int32_t fflags = kda::kChunkNoOutput | kda::kChunkSnapSlots |
                           (dt == KDA_BF16 ? kda::kChunkSnapBf16 : 0);
    SnapReq sr_check = sr;
    if (no_workspace) {   // (the state table is checked once it is known)
        sr_check.n_snap = 0;
        sr_check.snap = nullptr;
    }
    kda_status st = chunk_fwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk,
                                   Dv, dt, nullptr, nullptr, nullptr, 0, kda::kChunk, 0, sr_check,
                                   fflags, stream, true);
    if (st != KDA_OK) return st;

    const uint64_t es = esize(dt);
    const uint64_t nTok = (uint64_t)T_total * row * es, nB = (uint64_t)T_total * H * es;
    const uint64_t nState = (uint64_t)N * per * 4;
    const Span sq = span(q, nTok), sk = span(k, nTok), sv = span(v, nTok),
               sg = span(log_alpha, nTok), sb = span(beta, nB),
               sh0 = span(h0, h0 ? nState : 0),
               scu = span(cu_seqlens, cu_seqlens ? ((uint64_t)N + 1) * 4 : 0),
               sdo = span(dout, nTok), sdhT = span(dhT, dhT ? nState : 0),
               sws = span(workspace, no_workspace ? 0 : need), sdq = span(dq, nTok),
               sdk = span(dk, nTok), sdv = span(dv, nTok), sdg = span(dlog_alpha, nTok),
               sdb = span(dbeta, nB), sdh0 = span(dh0, dh0 ? nState : 0);
    const Span outs[] = {sdq, sdk, sdv, sdg, sdb, sdh0};
    for (int i = 0; i < 6; ++i) {
        if (overlaps_any(outs[i], {sq, sk, sv, sg, sb, sh0, scu, sdo, sdhT, sws}))
            return KDA_ERR_ALIAS;
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], outs[j])) return KDA_ERR_ALIAS;
    }
    if (overlaps_any(sws, {sdo, sdhT})) return KDA_ERR_ALIAS;
    if (check_only) return KDA_OK;

    kda::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.h0 = h0;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.T_total = T_total;
    a.H = H;
    a.dout = dout;
    a.dhT = dhT;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dlog_alpha = dlog_alpha;
    a.dbeta = dbeta;
    a.dh0 = dh0;
    a.states = states;
    a.dstates = dstates;
    a.n_slots = n_slots;
    // R (reverse recursion) on a side stream next to F (forward recursion,
    // state table), G (gradients) after both.  For bf16 each recursion then
    // takes one workgroup per (sequence, head), so that both sets of chains
    // are resident together.  The allocation-free entry point runs F, R, G
    // in order on the caller's stream.
    hipStream_t side = side_stream ? kda::bwd_fork(stream) : nullptr;
    if (side) {
        const int split = dt == KDA_BF16 ? 1 : 0;
        const bool r_ok = kda::launch_bwd_rev(a, (int)dt, split, side) == hipSuccess;
        st = chunk_fwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                            nullptr, nullptr, nullptr, 0, kda::kChunk, split, sr, fflags, stream);
        const bool j_ok = kda::bwd_join(stream) == hipSuccess;
        if (st != KDA_OK) return st;
        if (!r_ok || !j_ok) return KDA_ERR_DEVICE;
        if (kda::launch_bwd_grad(a, (int)dt, stream) != hipSuccess) return KDA_ERR_DEVICE;
        return KDA_OK;
    }
    st = chunk_fwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                        nullptr, nullptr, nullptr, 0, kda::kChunk, 0, sr, fflags, stream);
    if (st != KDA_OK) return st;
    if (kda::launch_bwd_rev(a, (int)dt, 0, stream) != hipSuccess ||
        kda::launch_bwd_grad(a, (int)dt, stream) != hipSuccess)
        return KDA_ERR_DEVICE;
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* log_alpha,
                         const void* beta, const float* h0, const int32_t* cu_seqlens,
                         int32_t N, int64_t T_total, int32_t H, int32_t Dk, int32_t Dv,
                         kda_dtype dt, const void* dout, const float* dhT, void* dq, void* dk,
                         void* dv, void* dlog_alpha, void* dbeta, float* dh0, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
    return chunk_bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                          dout, dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, workspace,
                          workspace_bytes, stream, false, false);
}

kda_status kda_chunk_bwd_noalloc(const void* q, const void* k, const void* v,
                                 const void* log_alpha, const void* beta, const float* h0,
                                 const int32_t* cu_seqlens, int32_t N, int64_t T_total,
                                 int32_t H, int32_t Dk, int32_t Dv, kda_dtype dt,
                                 const void* dout, const float* dhT, void* dq, void* dk,
                                 void* dv, void* dlog_alpha, void* dbeta, float* dh0,
                                 hipStream_t stream) {
    // every argument first, on the host; then the size limit; only then the
    // one HIP call that finds this device's copy of the library's scratch
    kda_status st = chunk_bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk,
                                   Dv, dt, dout, dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, nullptr,
                                   0, stream, true, true);
    if (st != KDA_OK) return st;
    if (kda_chunk_bwd_workspace_size(T_total, N, H, Dk, Dv, dt) > KDA_BWD_NOALLOC_MAX_BYTES)
        return KDA_ERR_WORKSPACE;
    void* scratch = nullptr;
    if (kda::noalloc_scratch(&scratch) != hipSuccess || !scratch) return KDA_ERR_DEVICE;
    return chunk_bwd_impl(q, k, v, log_alpha, beta, h0, cu_seqlens, N, T_total, H, Dk, Dv, dt,
                          dout, dhT, dq, dk, dv, dlog_alpha, dbeta, dh0, scratch,
                          KDA_BWD_NOALLOC_MAX_BYTES, stream, false, false, false);
}

kda_status kda_prologue(const void* xq, const void* xk, const void* xv, const void* a_raw,
                        const void* b_raw, const float* conv_w, const float* a_bias,
                        const int32_t* cu_seqlens, int32_t N, int64_t T_total, int32_t H,
                        int32_t D, kda_dtype dt, const void* conv_state_in,
                        void* conv_state_out, float l2_eps, void* q, void* k, void* v,
                        void* log_alpha, void* beta, hipStream_t stream) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (N < 1 || T_total < 0 || H < 1 || H > KDA_MAX_HEADS || D != kda::kHeadDim)
        return KDA_ERR_BAD_SHAPE;
    if (!cu_seqlens && N != 1) return KDA_ERR_BAD_SHAPE;
    if (!(l2_eps >= 0.f) || l2_eps > std::numeric_limits<float>::max()) return KDA_ERR_BAD_SHAPE;
    const uint64_t row = (uint64_t)H * kda::kHeadDim;
    if ((uint64_t)T_total > kMaxElems / row) return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)N * 9u * row > kMaxElems) return KDA_ERR_BAD_SHAPE;
    if (T_total > 0 && (!xq || !xk || !xv || !a_raw || !b_raw || !conv_w || !a_bias || !q ||
                        !k || !v || !log_alpha || !beta))
        return KDA_ERR_NULL_ARG;
    for (const void* p : {xq, xk, xv, a_raw, (const void*)conv_w, (const void*)a_bias,
                          conv_state_in, (const void*)conv_state_out, (const void*)q,
                          (const void*)k, (const void*)v, (const void*)log_alpha})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    if ((b_raw && !aligned(b_raw, esize(dt))) || (beta && !aligned(beta, esize(dt))))
        return KDA_ERR_MISALIGNED;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_MISALIGNED;

    const uint64_t es = esize(dt);
    const uint64_t nTok = (uint64_t)T_total * row * es, nB = (uint64_t)T_total * H * es;
    const uint64_t nState = (uint64_t)N * 9u * row * es;
    const Span sxq = span(xq, nTok), sxk = span(xk, nTok), sxv = span(xv, nTok),
               sa = span(a_raw, nTok), sbr = span(b_raw, nB),
               sw = span(conv_w, T_total > 0 ? 3 * row * 4 * 4 : 0),
               sbias = span(a_bias, T_total > 0 ? row * 4 : 0),
               scu = span(cu_seqlens, cu_seqlens ? ((uint64_t)N + 1) * 4 : 0),
               ssi = span(conv_state_in, conv_state_in ? nState : 0),
               sso = span(conv_state_out, conv_state_out ? nState : 0), sq = span(q, nTok),
               sk = span(k, nTok), sv = span(v, nTok), sla = span(log_alpha, nTok),
               sbeta = span(beta, nB);
    for (const Span& o : {sq, sk, sv, sla, sbeta, sso})
        if (overlaps_any(o, {sxq, sxk, sxv, sa, sbr, sw, sbias, scu, ssi})) return KDA_ERR_ALIAS;
    const Span outs[] = {sq, sk, sv, sla, sbeta, sso};
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], outs[j])) return KDA_ERR_ALIAS;

    kda::PrologueArgs a;
    a.x[0] = xq;
    a.x[1] = xk;
    a.x[2] = xv;
    a.x[3] = a_raw;
    a.b_raw = b_raw;
    a.conv_w = conv_w;
    a.a_bias = a_bias;
    a.cu_seqlens = cu_seqlens;
    a.N = N;
    a.T_total = T_total;
    a.H = H;
    a.state_in = conv_state_in;
    a.state_out = conv_state_out;
    a.l2_eps = l2_eps;
    a.out[0] = q;
    a.out[1] = k;
    a.out[2] = v;
    a.out[3] = log_alpha;
    a.beta = beta;
    a.tb = kda::prologue_tokens_per_wave(T_total, H);
    a.n_tblocks = (int32_t)((T_total + a.tb - 1) / a.tb);
    // (the prologue's grid: four waves per workgroup)
    if ((uint64_t)(kda::prologue_conv_waves(a.n_tblocks, H, N) +
                   kda::prologue_gate_waves(a.n_tblocks, H)) >
        (uint64_t)std::numeric_limits<int32_t>::max() * 4u)
        return KDA_ERR_BAD_SHAPE;
    if (T_total == 0 && !conv_state_out) return KDA_OK;
    if (kda::launch_prologue(a, (int)dt, stream) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

kda_status kda_epilogue(const void* o, const void* g, const float* norm_w, int64_t T_total,
                        int32_t H, int32_t D, kda_dtype dt, float eps, void* y,
                        hipStream_t stream) {
    if (!valid_dtype(dt)) return KDA_ERR_BAD_DTYPE;
    if (T_total < 0 || H < 1 || H > KDA_MAX_HEADS || D != kda::kHeadDim) return KDA_ERR_BAD_SHAPE;
    if (!(eps >= 0.f) || eps > std::numeric_limits<float>::max()) return KDA_ERR_BAD_SHAPE;
    const uint64_t row = (uint64_t)H * kda::kHeadDim;
    if ((uint64_t)T_total > kMaxElems / row) return KDA_ERR_BAD_SHAPE;
    if ((uint64_t)T_total * H > (uint64_t)std::numeric_limits<int32_t>::max() * 64u)
        return KDA_ERR_BAD_SHAPE;
    if (T_total > 0 && (!o || !g || !norm_w || !y)) return KDA_ERR_NULL_ARG;
    for (const void* p : {o, g, (const void*)norm_w, (const void*)y})
        if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
    const uint64_t n = (uint64_t)T_total * row * esize(dt);
    const Span so = span(o, n), sg = span(g, n), sy = span(y, n),
               sw = span(norm_w, T_total > 0 ? row * 4 : 0);
    // in place over o or g is allowed (each element is read before it is written,
    // by the same lane); any other overlap is not
    if ((y != o && overlaps(sy, so)) || (y != g && overlaps(sy, sg)) || overlaps(sy, sw))
        return KDA_ERR_ALIAS;
    if (T_total == 0) return KDA_OK;
    kda::EpilogueArgs a;
    a.o = o;
    a.g = g;
    a.norm_w = norm_w;
    a.T_total = T_total;
    a.H = H;
    a.eps = eps;
    a.y = y;
    if (kda::launch_epilogue(a, (int)dt, stream) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

}  // extern "C"
