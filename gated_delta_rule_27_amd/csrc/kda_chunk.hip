// kda_chunk.hip -- chunkwise KDA prefill for gfx950 (CDNA4).
//
// Method.  KDA is run in chunks of C tokens: inside a chunk the causal
// token interactions are dense matrix products, across chunks the 128 x 128
// state is carried recurrently ("From GPT-2 to Kimi K3, from first
// principles", ch. 6 "Chunkwise execution"; "An infra-oriented diagram of
// Kimi K3", KDA card: parallel tiles -> recurrent state).  The pages name
// the split (a UT transform and a pseudo-value term) without deriving it;
// the form used here, for one head, a chunk of positions r = 1..C and an
// incoming state S0 (row = key channel), with G_r = sum_{s<=r} log alpha_s
// per channel and Gamma_r = exp(G_r), is:
//
//   u_r := beta_r (v_r - (Diag(alpha_r) S_{r-1})^T k_r)      so that
//   S_r  = Diag(alpha_r) S_{r-1} + k_r u_r^T                 (exact rewrite
//          of (I - beta k k^T) Diag(alpha) S + beta k v^T),
//   (I + A) U = diag(beta) (V - Ktil S0),   A = strict_lower(diag(beta)
//          (K o Gamma)(K / Gamma)^T),  Ktil = K o Gamma,
//   T = (I + A)^{-1} diag(beta)                              (UT transform)
//   U = T (V - Ktil S0)                                      (pseudo-values)
//   O = Qtil S0 + lower_incl(Qtil (K / Gamma)^T) U,          Qtil = Q o Gamma
//   S_C = Diag(Gamma_C) S0 + Kvec^T U,        Kvec_s = k_s o Gamma_C / Gamma_s.
//
// Decay-factor range.  Exponents are never formed from the chunk start when
// they could overflow: the Gram products use, for row tile R (16 tokens),
// the reference point just before R, so left factors are <= 1 and right
// factors are <= 1 except on the diagonal tile.  There, log alpha >= -5
// bounds the log-decay summed over 16 tokens by -80, so a right factor is
// at most e^80 = 5.5e34, which bf16 (max 3.4e38) still represents ("From
// GPT-2 to Kimi K3", ch. 5 "K3's lower-bounded decay").  Every tile, on the
// diagonal or off it, is therefore an ordinary MFMA product.
//
// Kernel structure (one launch does the whole prefill).  One workgroup owns
// one (sequence, head, value-column slice) chain and walks that sequence's
// chunks in order.  Per chunk:
//   (a) intra-chunk, independent of the state: per-channel running products
//       of alpha, the decay-scaled operands in LDS, the Gram tiles
//       A = K K^T and P = Q K^T on MFMA, the unit-lower-triangular solve
//       T = (I + A)^{-1} diag(beta) in LDS (16 x 16 diagonal blocks by
//       forward substitution, off-diagonal blocks on fp32 MFMA);
//   (b) state propagation: each wavefront owns 16 * NCT value columns of
//       the state in accumulator registers for the whole sequence and
//       computes X = V - Ktil S, U = T X, O = Qtil S + P U and
//       S <- Diag(Gamma_C) S + Kvec^T U.  An accumulator tile is used
//       directly as the B operand of the next product, so the state and
//       the pseudo-values never leave registers; only the shared A operands
//       come from LDS.
// Value columns are independent, so a head's 128 columns may be split over
// `split` workgroups; each recomputes (a).  The next chunk's inputs are
// loaded into registers while (b) runs.
//
// Precision: bf16 inputs use bf16 MFMA operands (16x16x32) with fp32
// accumulation and an fp32 state; fp32 inputs use fp32 MFMA (16x16x4)
// throughout.  The running decay products, Gram outputs and the triangular
// solve are fp32 in both cases.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

template <typename TIn, int C, int NW, int NCT>
struct ChunkCfg {
    typedef TIn TOp;  // MFMA operand type
    static constexpr int NT = 64 * NW;
    static constexpr int NB = C / 16;                 // 16-token tiles per chunk
    static constexpr int NPAIR = NB * (NB + 1) / 2;   // causal tile pairs
    static constexpr int DV = 16 * NCT * NW;          // value columns per workgroup
    static constexpr int PADK = 16 / (int)sizeof(TOp);
    static constexpr int KP = kHeadDim + PADK;        // row stride of [token][channel]
    static constexpr int CP = C + PADK;               // row stride of [.][token]
    static constexpr int AP = C + 4;                  // row stride of the fp32 A tile
    static constexpr int LP = 20;                     // row stride of 16x16 fp32 blocks
    static constexpr int VP = DV + 4;                 // row stride of V (fp32)
    static constexpr int VEC = 16 / (int)sizeof(TIn); // elements per 16-byte load
    static constexpr int VROW = DV / VEC;             // 16-byte loads per V row
    static constexpr int NVL = (C * VROW + NT - 1) / NT;

    // LDS layout (bytes)
    static constexpr size_t szTok = (size_t)C * KP * sizeof(TOp);
    static constexpr size_t oXk = 0;
    static constexpr size_t oXq = oXk + szTok;
    static constexpr size_t oKn = oXq + szTok;
    static constexpr size_t oQs = oKn + szTok;
    static constexpr size_t oKh = oQs + szTok;
    static constexpr size_t oKvT = oKh + (size_t)NPAIR * 16 * KP * sizeof(TOp);
    static constexpr size_t oT = oKvT + (size_t)kHeadDim * CP * sizeof(TOp);
    static constexpr size_t oP = oT + (size_t)C * CP * sizeof(TOp);
    static constexpr size_t oA = oP + (size_t)C * CP * sizeof(TOp);
    static constexpr size_t oLi = oA + (size_t)C * AP * sizeof(float);
    static constexpr size_t oLiT = oLi + (size_t)NB * 16 * LP * sizeof(float);
    static constexpr size_t oV = oLiT + (size_t)NB * 16 * LP * sizeof(float);
    static constexpr size_t oBeta = oV + (size_t)C * VP * sizeof(float);
    static constexpr size_t oGam = oBeta + (size_t)C * sizeof(float);
    static constexpr size_t bytes = oGam + (size_t)kHeadDim * sizeof(float);

    static_assert(C == 16 || C == 32, "chunk length");
    static_assert(NW == 2 || NW == 4, "waves per workgroup");
    static_assert(NT >= kHeadDim, "one thread per key channel");
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

__host__ __device__ constexpr int pair_index(int R, int S) { return R * (R + 1) / 2 + S; }

template <typename TIn, int C, int NW, int NCT>
__global__ __launch_bounds__(64 * NW) void chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ log_alpha, const TIn* __restrict__ beta,
    const float* __restrict__ h0, const int32_t* __restrict__ cu_seqlens,
    int64_t T_total, int32_t H, int32_t split, TIn* __restrict__ o,
    float* __restrict__ h_T, SnapArgs snap, int32_t flags) {
    typedef ChunkCfg<TIn, C, NW, NCT> K;
    typedef typename K::TOp TOp;
    constexpr bool kBF16 = sizeof(TOp) == 2;
    constexpr int NB = K::NB, KP = K::KP, CP = K::CP, AP = K::AP, LP = K::LP,
                  VP = K::VP, DV = K::DV;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    TOp* sXk = reinterpret_cast<TOp*>(smem + K::oXk);
    TOp* sXq = reinterpret_cast<TOp*>(smem + K::oXq);
    TOp* sKn = reinterpret_cast<TOp*>(smem + K::oKn);
    TOp* sQs = reinterpret_cast<TOp*>(smem + K::oQs);
    TOp* sKh = reinterpret_cast<TOp*>(smem + K::oKh);
    TOp* sKvT = reinterpret_cast<TOp*>(smem + K::oKvT);
    TOp* sT = reinterpret_cast<TOp*>(smem + K::oT);
    TOp* sP = reinterpret_cast<TOp*>(smem + K::oP);
    float* sA = reinterpret_cast<float*>(smem + K::oA);
    float* sLi = reinterpret_cast<float*>(smem + K::oLi);
    float* sLiT = reinterpret_cast<float*>(smem + K::oLiT);
    float* sV = reinterpret_cast<float*>(smem + K::oV);
    float* sBeta = reinterpret_cast<float*>(smem + K::oBeta);
    float* sGam = reinterpret_cast<float*>(smem + K::oGam);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int wg = blockIdx.x;
    const int slice = wg % split;
    const int h = (wg / split) % H;
    const int n = wg / (split * H);
    const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[n + 1] : T_total;
    const size_t rowstride = (size_t)H * kHeadDim;  // elements between tokens
    const size_t headoff = (size_t)h * kHeadDim;
    const int col0 = slice * DV;                     // first value column of the slice

    // upper-triangular blocks of T and P are never written: clear them once
    for (int idx = tid; idx < C * CP; idx += K::NT) {
        sT[idx] = from_f32<TOp>(0.f);
        sP[idx] = from_f32<TOp>(0.f);
    }

    // ---- state: wave w owns value columns col0 + 16*(NCT*w + ct) + l16 ----
    floatx4 S[NCT][8];
    {
        const float* src = h0 ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim) : nullptr;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int j = col0 + 16 * (NCT * wave + ct) + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[ct][it][e] = src ? src[(16 * it + 4 * g + e) * kHeadDim + j] : 0.f;
        }
        // h0 = I (a separate uniform branch: folded into the loads above, the
        // selects cost registers across the whole chunk loop)
        if (!src && (flags & kChunkH0Identity)) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int j = col0 + 16 * (NCT * wave + ct) + l16;
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (16 * it + 4 * g + e == j) S[ct][it][e] = 1.f;
            }
        }
    }
    const bool v_zero = flags & kChunkVZero;
    const bool write_o = !(flags & kChunkNoOutput);

    // ---- register prefetch of one chunk's inputs ----
    // channel thread (tid < 128): q, k, log alpha of channel tid for C tokens
    TIn pq[C], pk[C], pg[C];
    typename Vec16<TIn>::type pv[K::NVL];
    TIn pb = from_f32<TIn>(0.f);
    auto prefetch = [&](int64_t t0, int len) {
        if (tid < kHeadDim) {
#pragma unroll
            for (int r = 0; r < C; ++r) {
                const bool ok = r < len;
                const size_t off = (size_t)(t0 + r) * rowstride + headoff + tid;
                pq[r] = ok && write_o ? q[off] : from_f32<TIn>(0.f);  // q feeds o only
                pk[r] = ok ? k[off] : from_f32<TIn>(0.f);
                pg[r] = ok ? log_alpha[off] : from_f32<TIn>(0.f);
            }
        }
#pragma unroll
        for (int u = 0; u < K::NVL; ++u) {
            const int idx = tid + u * K::NT;
            const int r = idx / K::VROW, cv = idx % K::VROW;
            typename Vec16<TIn>::type x = {};
            if (idx < C * K::VROW && r < len && !v_zero)
                x = *reinterpret_cast<const typename Vec16<TIn>::type*>(
                    v + (size_t)(t0 + r) * rowstride + headoff + col0 + cv * K::VEC);
            pv[u] = x;
        }
        if (tid < C) pb = tid < len ? beta[(size_t)(t0 + tid) * H + h] : from_f32<TIn>(0.f);
    };

    if (bos < eos) prefetch(bos, (int)((eos - bos) < C ? (eos - bos) : C));
    __syncthreads();

    for (int64_t t0 = bos; t0 < eos; t0 += C) {
        const int len = (int)((eos - t0) < C ? (eos - t0) : C);

        // ================= (a) intra-chunk =================
        // (a1) V, beta into LDS
#pragma unroll
        for (int u = 0; u < K::NVL; ++u) {
            const int idx = tid + u * K::NT;
            if (idx < C * K::VROW) {
                const int r = idx / K::VROW, cv = idx % K::VROW;
#pragma unroll
                for (int e = 0; e < K::VEC; ++e) sV[r * VP + cv * K::VEC + e] = to_f32(pv[u][e]);
            }
        }
        if (tid < C) sBeta[tid] = to_f32(pb);

        // (a2) per key channel: running decay products and scaled operands
        if (tid < kHeadDim) {
            const int i = tid;
            float al[C];
#pragma unroll
            for (int r = 0; r < C; ++r) al[r] = __expf(to_f32(pg[r]));
            float Et[NB];  // per-tile total decay exp(G_end(R) - G_end(R-1))
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                float p = 1.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) p *= al[16 * R + e];
                Et[R] = p;
            }
            float gam = 1.f;
#pragma unroll
            for (int R = 0; R < NB; ++R) gam *= Et[R];
            sGam[i] = gam;
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                float rho = 1.f, sig = 1.f;  // exp(G_ref(R)), exp(G_C - G_end(R))
#pragma unroll
                for (int R2 = 0; R2 < NB; ++R2) {
                    if (R2 < R) rho *= Et[R2];
                    if (R2 > R) sig *= Et[R2];
                }
                float E[16], Hs[16];
                float cum = 1.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    cum *= al[16 * R + e];
                    E[e] = cum;  // exp(G_r - G_ref(R))
                }
                float suf = 1.f;
#pragma unroll
                for (int e = 15; e >= 0; --e) {
                    Hs[e] = suf;  // exp(G_end(R) - G_r)
                    suf *= al[16 * R + e];
                }
                const float invEt = 1.f / fmaxf(Et[R], 1.17549435e-38f);
                TOp kv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = 16 * R + e;
                    const float kr = to_f32(pk[r]);
                    const float qr = to_f32(pq[r]);
                    const float kE = kr * E[e], qE = qr * E[e];
                    sXk[r * KP + i] = from_f32<TOp>(kE);
                    sXq[r * KP + i] = from_f32<TOp>(qE);
                    sKn[r * KP + i] = from_f32<TOp>(-kE * rho);
                    sQs[r * KP + i] = from_f32<TOp>(qE * rho);
                    const float kh = kr * Hs[e];
                    kv[e] = from_f32<TOp>(kh * sig);
                    // column operands of the Gram tiles (R2, R), R2 >= R
                    float c = invEt;
#pragma unroll
                    for (int R2 = R; R2 < NB; ++R2) {
                        sKh[(pair_index(R2, R) * 16 + e) * KP + i] = from_f32<TOp>(kh * c);
                        c = (R2 == R) ? 1.f : c * Et[R2];
                    }
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) sKvT[i * CP + 16 * R + e] = kv[e];
            }
        }
        __syncthreads();

        // (a3) Gram tiles on MFMA.  Transposed products give row-major tiles:
        // acc(row s, col r) = sum_i Khat[s][i] X[r][i].
        for (int job = wave; job < 2 * K::NPAIR; job += NW) {
            const int p = job >> 1;
            const bool isP = job & 1;
            int R = 0;
            while (pair_index(R + 1, 0) <= p) ++R;
            const int Sp = p - pair_index(R, 0);
            const TOp* arow = sKh + (p * 16 + l16) * KP;
            const TOp* brow = (isP ? sXq : sXk) + (16 * R + l16) * KP;
            floatx4 acc = zero4();
            if constexpr (kBF16) {
#pragma unroll
                for (int kb = 0; kb < kHeadDim; kb += 32)
                    acc = mma_bf16_k32(frag_k32(arow, kb, g), frag_k32(brow, kb, g), acc);
            } else {
#pragma unroll
                for (int kb = 0; kb < kHeadDim; kb += 16)
                    acc = mma_f32_k16(frag_k16(arow, kb, g), frag_k16(brow, kb, g), acc);
            }
            const int r = 16 * R + l16;
            const int sb = 16 * Sp + 4 * g;
            if (!isP) {
                const float br = sBeta[r];
                floatx4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    out[e] = (R == Sp && 4 * g + e >= l16) ? 0.f : acc[e] * br;
                *reinterpret_cast<floatx4*>(sA + r * AP + sb) = out;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sP[r * CP + sb + e] = from_f32<TOp>((R == Sp && 4 * g + e > l16) ? 0.f : acc[e]);
            }
        }
        __syncthreads();

        // (a4) UT transform, diagonal 16x16 blocks: lane = (block, column c)
        // forward substitution of (I + A_RR) x = e_c.
        if (wave == 0 && lane < 16 * NB) {
            const int R = lane >> 4, c = lane & 15;
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float a = (rr == c) ? 1.f : 0.f;
                const float* arow = sA + (16 * R + rr) * AP + 16 * R;
#pragma unroll
                for (int s = 0; s < rr; ++s) a -= arow[s] * x[s];
                x[rr] = a;
            }
            const float bc = sBeta[16 * R + c];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                sLi[(R * 16 + rr) * LP + c] = x[rr];
                sLiT[(R * 16 + c) * LP + rr] = x[rr];
                sT[(16 * R + rr) * CP + 16 * R + c] = from_f32<TOp>(x[rr] * bc);
            }
        }
        if constexpr (NB > 1) {
            __syncthreads();
            // (a5) off-diagonal block (1, 0): Linv_10 = -Linv_11 A_10 Linv_00
            if (wave == NW - 1) {
                const floatx4 y = mma_f32_k16(frag_k16(sA + (16 + l16) * AP, 0, g),
                                              frag_k16(sLiT + l16 * LP, 0, g), zero4());
                const floatx4 z = mma_f32_k16(frag_k16(sLi + (16 + l16) * LP, 0, g), y, zero4());
                const float bc = sBeta[l16];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sT[(16 + 4 * g + e) * CP + l16] = from_f32<TOp>(-z[e] * bc);
            }
        }
        __syncthreads();

        // start loading the next chunk while the state update runs
        {
            const int64_t tn = t0 + C;
            if (tn < eos) prefetch(tn, (int)((eos - tn) < C ? (eos - tn) : C));
        }

        // ================= (b) state propagation =================
        floatx4 X[NCT][NB], O[NCT][NB], U[NCT][NB];
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int jl = 16 * (NCT * wave + ct) + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) X[ct][mt][e] = sV[(16 * mt + 4 * g + e) * VP + jl];
                O[ct][mt] = zero4();
            }
            const TOp* rk = sKn + (16 * mt + l16) * KP;
            const TOp* rq = sQs + (16 * mt + l16) * KP;
            if constexpr (kBF16) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const bf16x8 a = frag_k32(rk, 32 * b, g);
                    const bf16x8 aq = frag_k32(rq, 32 * b, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const bf16x8 sb = acc_frag_k32(S[ct][2 * b], S[ct][2 * b + 1]);
                        X[ct][mt] = mma_bf16_k32(a, sb, X[ct][mt]);
                        O[ct][mt] = mma_bf16_k32(aq, sb, O[ct][mt]);
                    }
                }
            } else {
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const floatx4 a = frag_k16(rk, 16 * it, g);
                    const floatx4 aq = frag_k16(rq, 16 * it, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        X[ct][mt] = mma_f32_k16(a, S[ct][it], X[ct][mt]);
                        O[ct][mt] = mma_f32_k16(aq, S[ct][it], O[ct][mt]);
                    }
                }
            }
        }
        // U = T X and O += P U (T, P lower triangular; k over chunk tokens)
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const TOp* rt = sT + (16 * mt + l16) * CP;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) U[ct][mt] = zero4();
            if constexpr (kBF16 && C >= 32) {
#pragma unroll
                for (int pb2 = 0; pb2 < NB / 2; ++pb2) {
                    if (32 * pb2 > 16 * mt + 15) continue;
                    const bf16x8 a = frag_k32(rt, 32 * pb2, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        U[ct][mt] = mma_bf16_k32(
                            a, acc_frag_k32(X[ct][2 * pb2], X[ct][2 * pb2 + 1]), U[ct][mt]);
                }
            } else if constexpr (kBF16) {
                const bf16x4 a = frag_k16(rt, 0, g);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    U[ct][mt] = mma_bf16_k16(a, acc_frag_k16(X[ct][0]), U[ct][mt]);
            } else {
#pragma unroll
                for (int kt = 0; kt <= mt; ++kt) {
                    const floatx4 a = frag_k16(rt, 16 * kt, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) U[ct][mt] = mma_f32_k16(a, X[ct][kt], U[ct][mt]);
                }
            }
        }
        // (bf16: P U accumulates in its own tile and is added on the VALU, so
        // no accumulator passes from the fp32 MFMA chain above to a bf16 MFMA)
#pragma unroll
        for (int mt = 0; mt < NB; ++mt) {
            const TOp* rp = sP + (16 * mt + l16) * CP;
            if constexpr (kBF16 && C >= 32) {
                floatx4 PU[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) PU[ct] = zero4();
#pragma unroll
                for (int pb2 = 0; pb2 < NB / 2; ++pb2) {
                    if (32 * pb2 > 16 * mt + 15) continue;
                    const bf16x8 a = frag_k32(rp, 32 * pb2, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        PU[ct] = mma_bf16_k32(
                            a, acc_frag_k32(U[ct][2 * pb2], U[ct][2 * pb2 + 1]), PU[ct]);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) O[ct][mt] += PU[ct];
            } else if constexpr (kBF16) {
                const bf16x4 a = frag_k16(rp, 0, g);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    O[ct][mt] += mma_bf16_k16(a, acc_frag_k16(U[ct][0]), zero4());
            } else {
#pragma unroll
                for (int kt = 0; kt <= mt; ++kt) {
                    const floatx4 a = frag_k16(rp, 16 * kt, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) O[ct][mt] = mma_f32_k16(a, U[ct][kt], O[ct][mt]);
                }
            }
        }
        // outputs of this chunk
#pragma unroll
        for (int mt = 0; mt < NB; ++mt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int j = col0 + 16 * (NCT * wave + ct) + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mt + 4 * g + e;
                    if (r < len && write_o)
                        o[(size_t)(t0 + r) * rowstride + headoff + j] = from_f32<TIn>(O[ct][mt][e]);
                }
            }
        // S <- Diag(Gamma_C) S + Kvec^T U
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            floatx4 gm;
#pragma unroll
            for (int e = 0; e < 4; ++e) gm[e] = sGam[16 * it + 4 * g + e];
            const TOp* rv = sKvT + (16 * it + l16) * CP;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[ct][it] *= gm;
            if constexpr (kBF16 && C >= 32) {
#pragma unroll
                for (int pb2 = 0; pb2 < NB / 2; ++pb2) {
                    const bf16x8 a = frag_k32(rv, 32 * pb2, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        S[ct][it] = mma_bf16_k32(
                            a, acc_frag_k32(U[ct][2 * pb2], U[ct][2 * pb2 + 1]), S[ct][it]);
                }
            } else if constexpr (kBF16) {
                const bf16x4 a = frag_k16(rv, 0, g);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[ct][it] = mma_bf16_k16(a, acc_frag_k16(U[ct][0]), S[ct][it]);
            } else {
#pragma unroll
                for (int kt = 0; kt < NB; ++kt) {
                    const floatx4 a = frag_k16(rv, 16 * kt, g);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[ct][it] = mma_f32_k16(a, U[ct][kt], S[ct][it]);
                }
            }
        }
        // prefix snapshot after this chunk (uniform branch; rare).  C divides
        // kSnapUnit * every_chunks (checked by the caller).
        if (snap.snap && len == C) {
            const int64_t done = t0 + C - bos;  // tokens of the sequence consumed
            const int64_t every = (int64_t)kSnapUnit * snap.every_chunks;
            if (done % every == 0) {
                const int64_t base = (flags & kChunkSnapSlots) ? chunk_slot(bos, n)
                                     : snap.snap_cu ? (int64_t)snap.snap_cu[n] : 0;
                const int64_t idx = base + done / every - 1;
                if (idx < snap.n_snap) {
                    // buffer stores: one lane offset, the rest in the scalar
                    // offset, so no per-element addresses stay live
                    const rsrc_t rs = make_rsrc(
                        snap.snap + ((size_t)idx * (size_t)H + h) * (kHeadDim * kHeadDim),
                        kHeadDim * kHeadDim * 4);
                    const uint32_t lane =
                        (uint32_t)((4 * g * kHeadDim + col0 + 16 * NCT * wave + l16) * 4);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                        for (int it = 0; it < 8; ++it)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                buf_store_f32(S[ct][it][e], rs, lane,
                                              ((16 * it + e) * kHeadDim + 16 * ct) * 4);
                }
            }
        }
        __syncthreads();
    }

    if (h_T) {
        float* dst = h_T + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const int j = col0 + 16 * (NCT * wave + ct) + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * it + 4 * g + e) * kHeadDim + j] = S[ct][it][e];
        }
    }
}

template <typename TIn, int C, int NW, int NCT>
hipError_t launch(const ChunkArgs& a, hipStream_t stream) {
    typedef ChunkCfg<TIn, C, NW, NCT> K;
    const int split = kHeadDim / K::DV;
    auto kern = chunk_kernel<TIn, C, NW, NCT>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = raise_lds_limit_once((const void*)kern, (int)K::bytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t nwg = (int64_t)a.N * a.H * split;
    if (nwg == 0) return hipSuccess;
    kern<<<dim3((unsigned)nwg), dim3(K::NT), K::bytes, stream>>>(
        (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, (const TIn*)a.log_alpha,
        (const TIn*)a.beta, a.h0, a.cu_seqlens, a.T_total, a.H, split, (TIn*)a.o, a.h_T,
        a.snap, a.flags);
    return hipGetLastError();
}

// split -> (waves, column tiles per wave): split 1 = 4x2, 2 = 4x1, 4 = 2x1
template <typename TIn, int C>
hipError_t launch_split(const ChunkArgs& a, int split, hipStream_t stream) {
    switch (split) {
        case 1: return launch<TIn, C, 4, 2>(a, stream);
        case 2: return launch<TIn, C, 4, 1>(a, stream);
        case 4: return launch<TIn, C, 2, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs& a, int dtype, int chunk, int split,
                        hipStream_t stream) {
    if (dtype == 0) {
        return chunk == 16 ? launch_split<float, 16>(a, split, stream)
                           : launch_split<float, 32>(a, split, stream);
    }
    if (chunk == 16 && chunk_ws2_supports(a, split)) return launch_chunk_ws2(a, split, stream);
    if (chunk == 32 && chunk_ws3_supports(a, split)) return launch_chunk_ws3(a, split, stream);
    return chunk == 16 ? launch_split<bf16, 16>(a, split, stream)
                       : launch_split<bf16, 32>(a, split, stream);
}

}  // namespace kda
