// kda_chunk_ws.hip -- wave-specialised, software-pipelined chunkwise KDA
// prefill for bf16 inputs on gfx950 (CDNA4).
//
// Same mathematics as kda_chunk.hip (chunkwise KDA with a UT transform and
// pseudo-values; see that file), with chunks of C = 16 tokens: one 16-token
// tile per chunk, so the decay reference point is the chunk start and every
// right-hand decay factor is at most e^80 ("From GPT-2 to Kimi K3", ch. 5
// "K3's lower-bounded decay"; "An infra-oriented diagram of Kimi K3", KDA
// card).  For a chunk with incoming state S0:
//   E_r = exp(G_r),  H_r = exp(G_C - G_r),  Gamma = exp(G_C)  (per channel)
//   Ktil = K o E, Qtil = Q o E, Khat = K / E, Kvec = K o H
//   A = strict_lower(diag(beta) Ktil Khat^T),  P = lower_incl(Qtil Khat^T)
//   T = (I + A)^{-1} diag(beta)
//   U = T (V - Ktil S0),  O = Qtil S0 + P U,  S_C = Diag(Gamma) S0 + Kvec^T U.
//
// Why a second kernel.  Per chunk, the state-independent work (decay
// factors, operand scaling, Gram tiles, the triangular solve) is a chain of
// short dependent steps with little parallelism inside one chunk, while the
// state update is a chain over chunks.  The pages' FlashKDA note describes
// overlapping the token-parallel work with the head-parallel state
// propagation ("From GPT-2 to Kimi K3", ch. 6 "Training, prefill, and decode
// use different paths").  Here the overlap is inside one workgroup of NSW + 8
// wavefronts (12 for a 64-column slice, 16 for all 128 columns):
//   waves 0..NSW-1 (state): each owns 16 * NCT value columns of the 128 x 128
//     state in MFMA accumulators for the whole sequence and runs the state
//     chain of chunk c with no global memory operation of its own (V comes
//     from an LDS ring, O goes to an LDS tile); state waves 0 and 1 then form
//     the Gram tiles of chunk c+2 (A and P);
//   the next 8 waves (prep), lane = (token r, 4 key channels): load q, k, log_alpha
//     of chunk c+3 straight into the lanes that use them (PD chunks ahead),
//     take the cumulative log-decay over the chunk's 16 tokens as a DPP scan
//     across the 16 lanes of a row and write the decay-scaled operands in
//     token rows; prep waves 0-3 also run the triangular solve of chunk c+1
//     (lane = one element of the 16 x 16 inverse), and two of them move V in
//     and O out as 16-byte row pieces.
// Every stage reads only what an earlier iteration wrote, so one barrier per
// chunk is the only synchronisation.  LDS holds ring buffers indexed by
// chunk, each at least as deep as its value lives.
// Two variants, chosen at launch: DEEP (sequences of 512 tokens and more on
// average) splits each Gram tile over two iterations and all four state
// waves, one pipeline stage deeper (the state then runs chunk c-1, the solve
// chunk c); DUAL (segment summaries) runs two groups of NSW state waves, one
// per summary pass, over the operands the prep waves form once.
//
// Workgroup order is XCD-aware: the `split` workgroups that share one
// (sequence, head) get ids with the same residue mod 8, i.e. the same XCD
// and L2, where their identical q / k / log_alpha reads hit.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kWsC = 16;      // tokens per chunk
constexpr int kXcds = 8;      // MI355X accelerator complex dies
constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the transcendental unit (v_exp_f32); |x| stays far inside its range here
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NCT, int NSW_, int PD, bool DEEP, bool DUAL>
struct WsCfg {
    static constexpr int NSW = NSW_;             // state waves per pass
    static constexpr int NSA = DUAL ? 2 * NSW : NSW;   // state waves in all
    static constexpr int NPW = 8;                // prep waves
    static constexpr int NT = 64 * (NSA + NPW);  // threads
    static constexpr int DV = 16 * NCT * NSW;    // value columns per workgroup
    // bf16 stride of [token][channel] rows: 280 bytes.  Consecutive rows then
    // start 6 banks apart, which keeps the 8-byte row reads of the MFMA
    // operands (16 rows at once), the transposed column reads and the prep
    // waves' 8-byte row writes free of bank conflicts; the 272-byte stride
    // (4 banks) made every operand row read a two-way conflict.
    static constexpr int KP = kHeadDim + 12;
    static constexpr int TP = kWsC + 8;          // bf16 stride of [.][token]
    static constexpr int AP = 20;                // fp32 stride of the A tile

    static constexpr size_t szTok = kWsC * KP * 2;        // [16][128] bf16
    static constexpr size_t szTile = kWsC * TP * 2;       // [16][16] bf16
    static constexpr size_t szA = kWsC * AP * 4;          // [16][16] fp32
    // ring buffers; chunk y's operands are written by the prep stage four
    // iterations before the state stage reads them
    static constexpr size_t KN0 = 0;                        // -Ktil, 5 slots
    static constexpr size_t QS0 = KN0 + 5 * szTok;          //  Qtil, 5 slots
    static constexpr size_t KV0 = QS0 + 5 * szTok;          //  Kvec rows, 5 slots
    static constexpr size_t GAM0 = KV0 + 5 * szTok;         //  Gamma, 5 slots
    static constexpr size_t KH0 = GAM0 + 5 * 512;           //  Khat, 3 slots
    static constexpr size_t BETA0 = KH0 + 3 * szTok;        //  beta, 4 slots
    static constexpr size_t A0 = BETA0 + 4 * 64;            //  A, 2 slots
    static constexpr size_t P0 = A0 + 2 * szA;              //  P, 3 slots
    static constexpr size_t T0 = P0 + 3 * szTile;           //  T, 2 slots
    static constexpr int VP = DV + 8;                       // bf16 stride of the V / O tiles
    static constexpr size_t szVO = kWsC * VP * 2;           // [16][DV] bf16
    static constexpr size_t VT0 = T0 + 2 * szTile;          //  V of the workgroup's columns, 5 slots
    static constexpr size_t OT0 = VT0 + 5 * szVO;           //  O of the workgroup's columns, 2 slots
    static constexpr size_t TILE0 = OT0 + 2 * szVO;         //  per state wave: bf16 snapshot staging
    static constexpr size_t szTiles = NSW * kWsC * kTileTP * 2;
    // bf16 snapshots: with room for two slots, the state waves only write
    // their tiles to LDS and the prep waves store them an iteration later
    static constexpr bool SNAP_PREP = TILE0 + 2 * szTiles <= 160 * 1024;
    static constexpr size_t bytes = TILE0 + (SNAP_PREP ? 2 : 1) * szTiles;

    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(kWsC == kSnapUnit, "snapshots fall on chunk ends");
};

template <int NCT, int NSW, int PD, bool DEEP, bool DUAL, bool SP>
__global__ __launch_bounds__((WsCfg<NCT, NSW, PD, DEEP, DUAL>::NT)) void chunk_ws_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ log_alpha, const bf16* __restrict__ beta,
    const float* __restrict__ h0, const int32_t* __restrict__ cu_seqlens, int64_t T_total,
    int32_t H, int32_t split, int32_t units, bf16* __restrict__ o, float* __restrict__ h_T,
    float* __restrict__ h_T2, SnapArgs snap, int32_t flags) {
    typedef WsCfg<NCT, NSW, PD, DEEP, DUAL> K;
    constexpr int GD = DEEP ? 1 : 0;   // extra pipeline depth of the split Gram tiles
    constexpr int KP = K::KP, TP = K::TP, AP = K::AP, DV = K::DV;

    // XCD-aware id: slices of one unit share the id's residue mod 8
    const int x = blockIdx.x;
    const int xcd = x % kXcds;
    const int qd = x / kXcds;
    const int slice = qd % split;
    const int unit = (qd / split) * kXcds + xcd;
    if (unit >= units) return;
    const int n = unit / H;
    const int h = unit % H;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    // (chunk indices into the rings are never negative)
    auto m5 = [](int y) { return (int)((unsigned)y % 5u); };
    auto m3 = [](int y) { return (int)((unsigned)y % 3u); };
    auto kn_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KN0 + m5(y) * K::szTok); };
    auto qs_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::QS0 + m5(y) * K::szTok); };
    auto kv_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KV0 + m5(y) * K::szTok); };
    auto gam_s = [&](int y) { return reinterpret_cast<float*>(smem + K::GAM0 + m5(y) * 512); };
    auto kh_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KH0 + m3(y) * K::szTok); };
    auto beta_s = [&](int y) { return reinterpret_cast<float*>(smem + K::BETA0 + (y & 3) * 64); };
    auto a_s = [&](int y) { return reinterpret_cast<float*>(smem + K::A0 + (y & 1) * K::szA); };
    auto p_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::P0 + m3(y) * K::szTile); };
    auto t_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::T0 + (y & 1) * K::szTile); };
    auto vt_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::VT0 + m5(y) * K::szVO); };
    auto ot_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::OT0 + (y & 1) * K::szVO); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index as a scalar: the role branches below are wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[n + 1] : T_total;
    const int64_t seqlen = eos - bos;
    const int nch = (int)((seqlen + kWsC - 1) / kWsC);
    const size_t rowstride = (size_t)H * kHeadDim;
    const size_t headoff = (size_t)h * kHeadDim;
    const int col0 = slice * DV;
    // pipeline iterations c = -3 .. last: the prep stage of iteration c
    // handles chunk c+3; the Gram stage chunk c+2 (with DEEP: the first
    // half, key channels 0-63, of chunk c+2 and the second half of chunk
    // c+1); the solve chunk c+1 (DEEP: c); the state chunk c (DEEP: c-1).
    // The loops step PD iterations per trip (register slots are compile-time
    // per position); iterations past `last` find no chunk to work on.
    const int last = nch - 1 + GD;
    const int nit = (last + 4 + PD - 1) / PD * PD;

    // An empty sequence has no chunks: only h_T = h0 is written, and no
    // input pointer is touched (they may be null when T_total is 0).  The
    // branch is uniform over the workgroup, so no barrier is skipped.
    if (nch == 0) {
        // (with DUAL, state waves NSW .. 2 NSW - 1 write the identity into h_T2)
        const bool mp = DUAL && wave >= NSW;
        float* hT = mp ? h_T2 : h_T;
        if (wave < K::NSA && hT) {
            const float* src = (h0 && !mp) ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim) : nullptr;
            const bool ident = mp || (flags & kChunkH0Identity);
            const int sw = mp ? wave - NSW : wave;
            float* dst = hT + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int j = col0 + 16 * (NCT * sw + ct) + l16;
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * it + 4 * g + e;
                        const int idx = row * kHeadDim + j;
                        dst[idx] = src ? src[idx] : (ident && row == j ? 1.f : 0.f);
                    }
            }
        }
        return;
    }

    // Gram tiles of chunk zc, on MFMA (transposed products: acc(s, r)):
    // A[r][s] = beta_r (Ktil_r . Khat_s), strictly lower and stored negated
    // (Kn = -Ktil; the solve then adds, one fused DPP multiply-add a step), or
    // P[r][s] = Qtil_r . Khat_s for s <= r.  Without DEEP, state waves 0 (A)
    // and 1 (P) form whole tiles (nk = 128 key channels from k0 = 0).  With
    // DEEP a tile is summed over two iterations by one state wave, half of
    // the key channels in each, the accumulator held in registers across the
    // barrier: chunks of even index by state waves 0 (A) and 1 (P), odd by 2
    // and 3, so that every state wave forms half a tile per iteration (one
    // more pipeline stage: worth it from a few dozen chunks per sequence).
    auto gram_part = [&](bool isP, int zc, int k0, int nk, bool finish, floatx4& acc) {
        const bf16* arow = kh_s(zc) + l16 * KP;
        const bf16* brow = (isP ? qs_s(zc) : kn_s(zc)) + l16 * KP;
        if (k0 == 0) acc = zero4();
#pragma unroll
        for (int kb = 0; kb < nk; kb += 32)
            acc = mma_bf16_k32(frag_k32(arow, k0 + kb, g), frag_k32(brow, k0 + kb, g), acc);
        if (!finish) return;
        if (!isP) {
            const float br = beta_s(zc)[l16];
            floatx4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (4 * g + e >= l16) ? 0.f : acc[e] * br;
            *reinterpret_cast<floatx4*>(a_s(zc) + l16 * AP + 4 * g) = out;
        } else {
            bf16x4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (bf16)((4 * g + e > l16) ? 0.f : acc[e]);
            *reinterpret_cast<bf16x4*>(p_s(zc) + l16 * TP + 4 * g) = out;
        }
    };

    if (wave < K::NSA) {
        // ======================= state waves =======================
        // With DUAL the workgroup runs two passes over the same operands
        // (segment summaries): waves 0 .. NSW-1 the B pass (zero start, V,
        // h_T), waves NSW .. 2 NSW - 1 the M pass (identity start, V = 0,
        // h_T2); sw is the wave's index within its pass.
        const bool mpass = DUAL && wave >= NSW;
        const int sw = mpass ? wave - NSW : wave;
        floatx4 S[NCT][8];
        {
            const float* src = (h0 && !mpass) ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim)
                                              : nullptr;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int j = col0 + 16 * (NCT * sw + ct) + l16;
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[ct][it][e] = src ? src[(16 * it + 4 * g + e) * kHeadDim + j] : 0.f;
            }
            // h0 = I (a separate uniform branch: folded into the loads above,
            // the selects cost registers across the whole chunk loop)
            if (!src && (mpass || (flags & kChunkH0Identity))) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int j = col0 + 16 * (NCT * sw + ct) + l16;
#pragma unroll
                    for (int it = 0; it < 8; ++it)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * it + 4 * g + e == j) S[ct][it][e] = 1.f;
                }
            }
        }
        // V arrives in, and O leaves through, LDS tiles of the workgroup's
        // DV columns (the prep waves move them between LDS and memory), so
        // the state waves issue no global memory operations per chunk.
        const int colw0 = col0 + 16 * NCT * sw + l16;  // this lane's first column
        const int64_t snap_base = (flags & kChunkSnapSlots) ? chunk_slot(bos, n)
                                  : snap.snap_cu ? (int64_t)snap.snap_cu[n] : 0;
        const uint32_t snap_lane = (uint32_t)((4 * g * kHeadDim + colw0) * 4);
        constexpr int VP = K::VP;
        const bool write_o = !(flags & kChunkNoOutput);

        floatx4 gacc = zero4();   // the Gram tile this wave is summing
        auto state_iter = [&](int cit) {
            const int c = cit - GD;   // the chunk of this iteration's state stage
            if (c >= 0 && c < nch) {
                const bf16* Kn = kn_s(c) + l16 * KP;
                const bf16* Qs = qs_s(c) + l16 * KP;
                const float* Gm = gam_s(c);
                floatx4 X[NCT], Ov[NCT], U[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    // rows 4g..4g+3 of this lane's column (transposed read);
                    // the M pass takes V as zero
                    if (mpass) {
                        X[ct] = zero4();
                    } else {
                        const bf16x4 v4 = lds_col4(vt_s(c) + 4 * g * VP + 16 * (NCT * sw + ct), VP, l16);
#pragma unroll
                        for (int e = 0; e < 4; ++e) X[ct][e] = (float)v4[e];
                    }
                    Ov[ct] = zero4();
                }
                // X = V - Ktil S, O = Qtil S
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const bf16x8 a = frag_k32(Kn, 32 * b, g);
                    const bf16x8 aq = frag_k32(Qs, 32 * b, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const bf16x8 sb = acc_frag_k32(S[ct][2 * b], S[ct][2 * b + 1]);
                        X[ct] = mma_bf16_k32(a, sb, X[ct]);
                        Ov[ct] = mma_bf16_k32(aq, sb, Ov[ct]);
                    }
                }
                // U = T X, O += P U
                const bf16x4 at = frag_k16(t_s(c) + l16 * TP, 0, g);
                const bf16x4 ap = frag_k16(p_s(c) + l16 * TP, 0, g);
                bf16x4 ub[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    U[ct] = mma_bf16_k16(at, acc_frag_k16(X[ct]), zero4());
                    ub[ct] = acc_frag_k16(U[ct]);
                    Ov[ct] = mma_bf16_k16_as_k32(ap, ub[ct], Ov[ct]);  // same opcode as Qtil S
                }
                if (write_o) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct)
                            ot_s(c)[(4 * g + e) * VP + 16 * (NCT * sw + ct) + l16] = (bf16)Ov[ct][e];
                }
                // S <- Diag(Gamma) S + Kvec^T U
                const bf16* Kv = kv_s(c);
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const floatx4 gm = *reinterpret_cast<const floatx4*>(Gm + 16 * it + 4 * g);
                    // Kvec^T rows 16 it .. +15 over tokens 4g .. 4g+3: a transposed read
                    const bf16x4 a = lds_col4(Kv + 4 * g * KP + 16 * it, KP, l16);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[ct][it] = mma_bf16_k16(a, ub[ct], S[ct][it] * gm);
                }
                // prefix snapshot after chunk c (uniform branch; rare)
                if (snap.snap && (c + 1) % snap.every_chunks == 0 &&
                    (int64_t)kWsC * (c + 1) <= seqlen) {
                    const int64_t idx = snap_base + (c + 1) / snap.every_chunks - 1;
                    if (idx < snap.n_snap) {
                        const size_t eo = ((size_t)idx * (size_t)H + h) * (kHeadDim * kHeadDim);
                        if (SP) {
                            // transposed tile into slot c & 1; the prep waves
                            // store the workgroup's tiles next iteration
                            bf16* tile = reinterpret_cast<bf16*>(smem + K::TILE0 + (c & 1) * K::szTiles) +
                                         (size_t)wave * NCT * kWsC * kTileTP;
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct)
                                tile_to_lds(S[ct], tile + ct * kWsC * kTileTP, lane);
                        } else if (flags & kChunkSnapBf16) {
                            // transposed entry: this wave's 16 columns are 16
                            // contiguous rows of 128
                            const rsrc_t rs = make_rsrc(reinterpret_cast<bf16*>(snap.snap) + eo,
                                                        kHeadDim * kHeadDim * 2);
                            bf16* tile = reinterpret_cast<bf16*>(smem + K::TILE0) +
                                         (size_t)wave * kWsC * kTileTP;
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct)
                                store_tile_t(S[ct], tile, rs,
                                             (uint32_t)((col0 + 16 * (NCT * sw + ct)) * kHeadDim * 2),
                                             lane);
                        } else {
                            const rsrc_t rs = make_rsrc(snap.snap + eo, kHeadDim * kHeadDim * 4);
#pragma unroll
                            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                                for (int it = 0; it < 8; ++it)
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        buf_store_f32(S[ct][it][e], rs, snap_lane,
                                                      ((16 * it + e) * kHeadDim + 16 * ct) * 4);
                        }
                    }
                }
            }
            // Gram tiles: the first half of chunk cit+2 (waves of its parity)
            // or the second half of chunk cit+1, whose tile is then written
            // (read by the solve in iteration cit+1 and by this stage in cit+2)
            if (DEEP && wave < 4) {
                const bool first = (wave >> 1) == (cit & 1);
                const int zc = first ? cit + 2 : cit + 1;
                if (zc >= 0 && zc < nch) gram_part(wave & 1, zc, first ? 0 : 64, 64, !first, gacc);
            } else if (!DEEP && wave < 2) {
                const int zc = cit + 2;
                if (zc >= 0 && zc < nch) gram_part(wave == 1, zc, 0, kHeadDim, true, gacc);
            }
            __syncthreads();
        };
        for (int c = -3; c < nit - 3; c += 4) {
            state_iter(c);
            state_iter(c + 1);
            state_iter(c + 2);
            state_iter(c + 3);
        }
        float* hT = mpass ? h_T2 : h_T;
        if (hT) {
            float* dst = hT + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int j = col0 + 16 * (NCT * sw + ct) + l16;
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(16 * it + 4 * g + e) * kHeadDim + j] = S[ct][it][e];
            }
        }
        return;
    }

    // ========================= prep waves =========================
    const int pw = wave - K::NSA;   // 0..7
    const int r = l16;              // token of the chunk
    const int ch0 = 16 * pw + 4 * g;  // first of this lane's 4 key channels
    // register slots of in-flight loads: chunk y lives in slot y % PD.  The
    // loads go through buffer resources over the chunk's rows inside the
    // sequence, so rows past its end read 0: they neither decay nor write.
    bf16x4 rq[PD], rk[PD], rg[PD];
    bf16 rb[PD];
    // V in / O out for the state waves: prep waves 4 - DV / 32 .. 3 move
    // one 16-byte piece of a row of the 16 x DV tile per lane: V of chunk
    // c+3 into its LDS tile (loaded PD iterations earlier) and O of chunk
    // c-1-GD out of its tile, in iteration c.  (Those waves also solve; the
    // prep waves that do not are the last to be issued and the busiest.)
    constexpr int VP = K::VP;
    static_assert(DV / 32 <= 4, "V / O waves are prep waves 0..3");
    const bool io_wave = pw >= 4 - DV / 32 && pw < 4;
    const int io_u = (pw - (4 - DV / 32)) * 64 + lane;
    const int io_row = io_u / (DV / 8), io_col = (io_u % (DV / 8)) * 8;
    const uint32_t io_off = (uint32_t)(((size_t)io_row * rowstride + headoff + col0 + io_col) * 2);
    const bool write_o = !(flags & kChunkNoOutput);
    // Per-chunk buffer resources, from scalar bases kept per sequence (the
    // scalar unit is shared by the waves of a SIMD, and 64-bit address and
    // size arithmetic per chunk and tensor was a large part of this
    // stage): chunk y starts y * cstride elements after the sequence's
    // first row and has chunk_rows(y) rows inside it (0 past the end).
    const size_t cstride = (size_t)kWsC * rowstride;
    const uint32_t last_rows = (uint32_t)(seqlen - (int64_t)kWsC * (nch - 1));
    auto chunk_rows = [&](int y) -> uint32_t {
        return y < nch - 1 ? (uint32_t)kWsC : y == nch - 1 ? last_rows : 0u;
    };
    const uint32_t row_bytes = (uint32_t)(rowstride * 2);
    const size_t seq0 = (size_t)bos * rowstride;
    const bf16 *q_seq = q + seq0, *k_seq = k + seq0, *g_seq = log_alpha + seq0, *v_seq = v + seq0;
    bf16* o_seq = o + seq0;
    const bf16* b_seq = beta + (size_t)bos * H;
    const bool q_none = flags & kChunkNoOutput, v_none = flags & kChunkVZero;
    bf16x8 rv[PD];
    auto store_o = [&](int y) {
        buf_store_b128(*reinterpret_cast<const bf16x8*>(ot_s(y) + io_row * VP + io_col),
                       make_rsrc_u32(o_seq + (size_t)y * cstride, chunk_rows(y) * row_bytes), io_off, 0);
    };
    // bf16 snapshot of chunk y from the state waves' LDS tiles (slot y & 1):
    // the workgroup's DV columns are DV contiguous rows of 128 in the
    // transposed entry; 512 prep lanes store 16-byte pieces
    const bool snap_prep = SP && snap.snap;
    const int64_t snap_base_p = (flags & kChunkSnapSlots) ? chunk_slot(bos, n)
                                : snap.snap_cu ? (int64_t)snap.snap_cu[n] : 0;
    auto store_snap = [&](int y) {
        if (!((y + 1) % snap.every_chunks == 0 && (int64_t)kWsC * (y + 1) <= seqlen)) return;
        const int64_t idx = snap_base_p + (y + 1) / snap.every_chunks - 1;
        if (idx >= snap.n_snap) return;
        const size_t eo = ((size_t)idx * (size_t)H + h) * (kHeadDim * kHeadDim);
        const rsrc_t rs = make_rsrc(reinterpret_cast<bf16*>(snap.snap) + eo, kHeadDim * kHeadDim * 2);
        const bf16* tiles = reinterpret_cast<const bf16*>(smem + K::TILE0 + (y & 1) * K::szTiles);
        const int pl = (wave - K::NSA) * 64 + lane;   // 0..511
#pragma unroll
        for (int m = 0; m < DV * 16 / 512; ++m) {
            const int p = m * 512 + pl, row = p >> 4, col8 = (p & 15) * 8;   // row: column of the state
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(tiles + (size_t)row * kTileTP + col8);
            buf_store_b128(x, rs, (uint32_t)(((size_t)(col0 + row) * kHeadDim + col8) * 2), 0);
        }
    };
    const uint32_t qo_lane = (uint32_t)(((size_t)r * rowstride + headoff + ch0) * 2);
    const uint32_t bo_lane = (uint32_t)(((size_t)r * H + h) * 2);
    auto load_chunk = [&](auto slot_c, int yc) {
        constexpr int s = decltype(slot_c)::value;
        const size_t off = (size_t)yc * cstride;
        const uint32_t rows = chunk_rows(yc), bytes = rows * row_bytes;
        // q feeds the outputs only: a pass without them reads none (zeros)
        rq[s] = buf_load_bf16x4(make_rsrc_u32(q_seq + off, q_none ? 0u : bytes), qo_lane);
        rk[s] = buf_load_bf16x4(make_rsrc_u32(k_seq + off, bytes), qo_lane);
        rg[s] = buf_load_bf16x4(make_rsrc_u32(g_seq + off, bytes), qo_lane);
        rb[s] = buf_load_bf16(make_rsrc_u32(b_seq + (size_t)yc * kWsC * H, rows * (uint32_t)H * 2), bo_lane);
        if (io_wave)
            rv[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   make_rsrc_u32(v_seq + off, v_none ? 0u : bytes),
                                                   (int)io_off, 0, 0));
    };
    load_chunk(std::integral_constant<int, 0>{}, 0);
    if constexpr (PD > 1) load_chunk(std::integral_constant<int, 1 % PD>{}, 1);
    if constexpr (PD > 2) load_chunk(std::integral_constant<int, 2 % PD>{}, 2);
    if constexpr (PD > 3) load_chunk(std::integral_constant<int, 3 % PD>{}, 3);

    auto prep_iter = [&](auto slot_c, int c) {
        constexpr int s = decltype(slot_c)::value;  // == (c + 3) % PD
        // (1) decay factors and scaled operands of chunk c+3
        const int yc = c + 3;
        if (yc < nch) {
            float kf[4], qf[4], lg[4];
            const float bt = (float)rb[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = (float)rk[s][e];
                qf[e] = (float)rq[s][e];
                lg[e] = (float)rg[s][e] * kLog2e;
            }
            bf16x4 kn, qs, kh, kv;
            floatx4 gam;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float P = row_prefix_sum(lg[e]);        // G_r / ln 2
                const float E = exp2f_fast(P);                // exp(G_r)       <= 1
                const float Einv = exp2f_fast(-P);            // exp(-G_r)      <= e^80
                gam[e] = row_bcast<15>(E);                    // exp(G_C): E of the last token
                const float Hs = gam[e] * Einv;               // exp(G_C - G_r) <= 1
                kn[e] = (bf16)(-kf[e] * E);
                qs[e] = (bf16)(qf[e] * E);
                kh[e] = (bf16)(kf[e] * Einv);
                kv[e] = (bf16)(kf[e] * Hs);
            }
            *reinterpret_cast<bf16x4*>(kv_s(yc) + r * KP + ch0) = kv;
            *reinterpret_cast<bf16x4*>(kn_s(yc) + r * KP + ch0) = kn;
            *reinterpret_cast<bf16x4*>(qs_s(yc) + r * KP + ch0) = qs;
            *reinterpret_cast<bf16x4*>(kh_s(yc) + r * KP + ch0) = kh;
            if (r == 0) *reinterpret_cast<floatx4*>(gam_s(yc) + ch0) = gam;
            if (pw == 0 && g == 0) beta_s(yc)[r] = bt;
            if (io_wave) *reinterpret_cast<bf16x8*>(vt_s(yc) + io_row * VP + io_col) = rv[s];
        }
        if (io_wave && write_o && c - 1 - GD >= 0 && c - 1 - GD < nch) store_o(c - 1 - GD);
        if (snap_prep && c - 1 - GD >= 0 && c - 1 - GD < nch) store_snap(c - 1 - GD);
        load_chunk(slot_c, yc + PD);
        // (3) UT transform of chunk c+1-GD on prep waves 0-3: lane = (row
        // l16, column 4 * pw + g) of X = (I + A)^{-1}; forward elimination
        // down the columns of A, the pivot X[sc][c] broadcast along the row
        // of 16 lanes by DPP.
        const int wc = c + 1 - GD;
        if (wc >= 0 && wc < nch && pw < 4) {
            const float* Arow = a_s(wc) + l16 * AP;
            float a[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(Arow + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * q4 + e] = v4[e];
            }
            const int col = 4 * pw + g;
            float xv = (l16 == col) ? 1.f : 0.f;
            // a = -A; A[r][sc] = 0 for sc >= r, so lanes above the pivot
            // are unchanged
            xv += row_bcast<0>(xv) * a[0];
            xv += row_bcast<1>(xv) * a[1];
            xv += row_bcast<2>(xv) * a[2];
            xv += row_bcast<3>(xv) * a[3];
            xv += row_bcast<4>(xv) * a[4];
            xv += row_bcast<5>(xv) * a[5];
            xv += row_bcast<6>(xv) * a[6];
            xv += row_bcast<7>(xv) * a[7];
            xv += row_bcast<8>(xv) * a[8];
            xv += row_bcast<9>(xv) * a[9];
            xv += row_bcast<10>(xv) * a[10];
            xv += row_bcast<11>(xv) * a[11];
            xv += row_bcast<12>(xv) * a[12];
            xv += row_bcast<13>(xv) * a[13];
            xv += row_bcast<14>(xv) * a[14];
            t_s(wc)[l16 * TP + col] = (bf16)(xv * beta_s(wc)[col]);
        }
        __syncthreads();
    };

    for (int c = -3; c < nit - 3; c += PD) {
        prep_iter(std::integral_constant<int, 0>{}, c);
        if constexpr (PD > 1) prep_iter(std::integral_constant<int, 1 % PD>{}, c + 1);
        if constexpr (PD > 2) prep_iter(std::integral_constant<int, 2 % PD>{}, c + 2);
        if constexpr (PD > 3) prep_iter(std::integral_constant<int, 3 % PD>{}, c + 3);
    }
    // O (and the snapshot) of the last chunk (written before the final barrier)
    if (io_wave && write_o) store_o(nch - 1);
    if (snap_prep) store_snap(nch - 1);
}

template <int NCT, int NSW, int PD, bool DEEP, bool DUAL, bool SP = false>
hipError_t launch_ws_t(const ChunkArgs& a, hipStream_t stream) {
    typedef WsCfg<NCT, NSW, PD, DEEP, DUAL> K;
    static_assert(PD % 2 == 0, "the state waves step two chunks per trip");
    static_assert(!SP || K::SNAP_PREP, "no room for two snapshot tile slots");
    const int split = kHeadDim / K::DV;
    auto kern = chunk_ws_kernel<NCT, NSW, PD, DEEP, DUAL, SP>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = raise_lds_limit_once((const void*)kern, (int)K::bytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0) return hipSuccess;
    const int64_t nwg = (units + kXcds - 1) / kXcds * kXcds * split;
    kern<<<dim3((unsigned)nwg), dim3(K::NT), K::bytes, stream>>>(
        (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.log_alpha,
        (const bf16*)a.beta, a.h0, a.cu_seqlens, a.T_total, a.H, split, (int32_t)units,
        (bf16*)a.o, a.h_T, a.h_T2, a.snap, a.flags);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_ws(const ChunkArgs& a, int split, hipStream_t stream) {
    if (chunk_ws2_supports(a, split)) return launch_chunk_ws2(a, split, stream);
    // the deeper pipeline costs one more iteration per sequence and saves a
    // few percent per iteration: used from 512 tokens per sequence on average
    const bool deep = a.N > 0 && a.T_total >= 512 * (int64_t)a.N;
    if (a.flags & kChunkDualBM) {   // 16 waves: 4 + 4 state waves of 64 columns
        if (split != 2) return hipErrorInvalidValue;
        return deep ? launch_ws_t<1, 4, 4, true, true>(a, stream)
                    : launch_ws_t<1, 4, 4, false, true>(a, stream);
    }
    switch (split) {
        case 1:   // 16 waves, 128 columns
            return deep ? launch_ws_t<1, 8, 4, true, false>(a, stream)
                        : launch_ws_t<1, 8, 4, false, false>(a, stream);
        case 2:   // 12 waves, 64 columns; bf16 snapshots staged for the prep waves
            if (a.snap.snap && (a.flags & kChunkSnapBf16))
                return deep ? launch_ws_t<1, 4, 4, true, false, true>(a, stream)
                            : launch_ws_t<1, 4, 4, false, false, true>(a, stream);
            return deep ? launch_ws_t<1, 4, 4, true, false>(a, stream)
                        : launch_ws_t<1, 4, 4, false, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
