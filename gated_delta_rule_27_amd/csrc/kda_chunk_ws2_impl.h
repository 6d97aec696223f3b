// kda_chunk_ws2_impl.h -- wave-specialised, software-pipelined chunkwise KDA
// prefill for bf16 inputs on gfx950 (CDNA4): the kernel template and its
// launch, instantiated by kda_chunk_ws2.hip (whole-head workgroups) and
// kda_chunk_ws2_s2.hip (half-head workgroups).
//
// Same mathematics as kda_chunk.hip (chunkwise KDA with a UT transform and
// pseudo-values; see that file), with chunks of C = 16 tokens: one 16-token
// tile per chunk, so the decay reference point is the chunk start and every
// right-hand decay factor is at most e^80 ("From GPT-2 to Kimi K3", ch. 5
// "K3's lower-bounded decay"; "An infra-oriented diagram of Kimi K3", KDA
// card).  For a chunk with incoming state S0:
//   E_r = exp(G_r),  Gamma = exp(G_C)  (per key channel)
//   Ktil = K o E, Qtil = Q o E, Khat = K / E, Kvec = K o Gamma / E
//   A = strict_lower(diag(beta) Ktil Khat^T),  P = lower_incl(Qtil Khat^T)
//   T = (I + A)^{-1} diag(beta)
//   U = T (V - Ktil S0),  O = Qtil S0 + P U,  S_C = Diag(Gamma) S0 + Kvec^T U.
//
// Per chunk, the state-independent work (decay factors, operand scaling,
// Gram tiles, the triangular solve) is a chain of short dependent steps with
// little parallelism inside one chunk, while the state update is a chain
// over chunks.  The pages' FlashKDA note describes overlapping the
// token-parallel work with the head-parallel state propagation ("From GPT-2
// to Kimi K3", ch. 6 "Training, prefill, and decode use different paths").
// Here the overlap is inside one workgroup of NSW state waves and 8 prep
// waves (12 waves for a 64-column slice, 16 for all 128 columns):
//   state waves: each owns 16 value columns of the 128 x 128 state in MFMA
//     accumulators for the whole sequence and runs the state chain of chunk
//     c with no global memory operation of its own (V comes from an LDS
//     ring, O goes to an LDS tile); state wave 0 (and 1, when o is written)
//     then forms a Gram tile of chunk c+2 (A, P);
//   prep waves, lane = (token r, 4 key channels): load q, k, log_alpha of a
//     chunk four chunks ahead straight into the lanes that use them, take
//     the cumulative log-decay over the chunk's 16 tokens as a DPP scan
//     across the 16 lanes of a row and write the decay-scaled operands of
//     chunk c+3 in token rows; prep waves 0 and 1 also run the UT solve of
//     chunk c+1 (two columns of the 16 x 16 inverse per lane), and prep
//     waves 2-3 (0-3 for all 128 columns) move V in and O out as 16-byte
//     row pieces.
// Every stage reads only what an earlier iteration wrote, so one barrier
// per chunk is the only synchronisation; the state waves carry the chain
// from chunk to chunk and issue at a raised priority.
//
// No unit bounds the per-chunk iteration: on MI355X (SQ counters, 4096
// tokens x 96 heads) the VALU is about half busy, the LDS under half and the
// MFMA unit a seventh, while a wave spends about a third of its time
// issuing, a third waiting for issue behind the other waves of its SIMD and
// the rest waiting on dependencies and the barrier.  The iteration is set
// by the longest dependency chains and the instruction streams of the
// busiest waves, hence:
//   * every ring buffer holds 2 or 4 chunks and the loop is unrolled four
//     times, so each ring slot is a compile-time constant (no modular
//     arithmetic on the scalar unit);
//   * no stage tests whether its chunk exists.  The rings start out holding
//     the identity chunk (Gamma = 1, everything else 0: the state passes
//     through unchanged), and chunks past the end of a sequence read zeros
//     through their buffer resources (log alpha = 0, beta = 0, V = 0), which
//     is again the identity; their outputs fall outside the resources and
//     are dropped.
//   * every wave runs a loop of its own role (state waves with or without a
//     Gram tile; prep waves with the UT solve, with V / O, or with the
//     scaled operands alone), so that each loop body is one basic block per
//     chunk and the compiler interleaves the long dependency chains (the
//     solve, the state chain) with the independent work of the same wave.
//     On MI355X this took the 4096-token, 96-head prefill from 245 us to
//     229 us; spreading the same work over 16 waves was slower (260 us).
// Variants, chosen at launch: NSW = 4 (split 2) or 8 (split 1); NOOUT for
// passes without outputs (the backward's forward recursion, segment
// summaries); DUAL (segment summaries, split 2) runs two groups of 4 state
// waves, one per summary pass, over the operands the prep waves form once.
// The state waves also write snapshots: fp32 states straight from their
// accumulators, bf16 per-chunk tables through an LDS staging tile.
//
// Workgroup order is XCD-aware: the `split` workgroups that share one
// (sequence, head) get ids with the same residue mod 8, i.e. the same XCD
// and L2, where their identical q / k / log_alpha reads hit.
#pragma once

#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC2 = 16;       // tokens per chunk
constexpr int kXcd2 = 8;      // MI355X accelerator complex dies
constexpr float kLog2e2 = 1.4426950408889634f;

template <int NSW_, bool DUAL = false>
struct Ws2Cfg {
    static constexpr int NSW = NSW_;             // state waves per pass (16 value columns each)
    static constexpr int NSA = DUAL ? 2 * NSW : NSW;   // state waves in all
    static constexpr int NPW = 8;                // prep waves
    static constexpr int NT = 64 * (NSA + NPW);  // threads
    static constexpr int DV = 16 * NSW;          // value columns per workgroup
    // bf16 stride of [token][channel] rows: 280 bytes, 6 banks apart, which
    // keeps 8-byte row reads, transposed column reads and 8-byte row writes
    // of 16 rows free of bank conflicts
    static constexpr int KP = kHeadDim + 12;
    static constexpr int TP = kC2 + 8;           // bf16 stride of [.][token]
    static constexpr int AP = 20;                // fp32 stride of the A tile
    static constexpr int VP = DV + 8;            // bf16 stride of the V / O tiles

    static constexpr size_t szTok = kC2 * KP * 2;
    static constexpr size_t szTile = kC2 * TP * 2;
    static constexpr size_t szA = kC2 * AP * 4;
    static constexpr size_t szVO = kC2 * VP * 2;
    static constexpr size_t KN0 = 0;                        // -Ktil, 4 slots
    static constexpr size_t QS0 = KN0 + 4 * szTok;          //  Qtil, 4 slots
    static constexpr size_t KV0 = QS0 + 4 * szTok;          //  Kvec rows, 4 slots
    static constexpr size_t KH0 = KV0 + 4 * szTok;          //  Khat, 2 slots
    static constexpr size_t GAM0 = KH0 + 2 * szTok;         //  Gamma, 4 slots
    static constexpr size_t BETA0 = GAM0 + 4 * 512;         //  beta, 4 slots
    static constexpr size_t A0 = BETA0 + 4 * 64;            //  A, 2 slots
    static constexpr size_t P0 = A0 + 2 * szA;              //  P, 4 slots
    static constexpr size_t T0 = P0 + 4 * szTile;           //  T, 2 slots
    static constexpr size_t VT0 = T0 + 2 * szTile;          //  V, 4 slots
    static constexpr size_t OT0 = VT0 + 4 * szVO;           //  O, 2 slots
    static constexpr size_t TILE0 = OT0 + 2 * szVO;         //  per state wave: bf16 table staging
    static constexpr size_t bytes = TILE0 + NSW * kC2 * kTileTP * 2;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(bytes % 16 == 0, "16-byte initialisation");
};

// Ring slot of chunk c0 + 4j + K + OFF for a loop that starts at c0 = -3.
template <int K, int OFF>
constexpr int slot4() { return (K + OFF + 1) & 3; }
template <int K, int OFF>
constexpr int slot2() { return (K + OFF + 1) & 1; }

// NOOUT: a pass without outputs (the backward's forward recursion, segment
// summaries): the state waves skip the Qtil S and P U products and the P
// Gram tile, which only feed o.  DUAL (segment summaries, implies NOOUT):
// two groups of NSW state waves share the prep waves' operands: waves
// 0 .. NSW-1 run the B pass (h0 or zero start, V, h_T), waves
// NSW .. 2 NSW-1 the M pass (identity start, V = 0, h_T2).
template <int NSW, bool NOOUT, bool DUAL>
__global__ __launch_bounds__((Ws2Cfg<NSW, DUAL>::NT)) void chunk_ws2_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ log_alpha, const bf16* __restrict__ beta,
    const float* __restrict__ h0, const int32_t* __restrict__ cu_seqlens, int64_t T_total,
    int32_t H, int32_t split, int32_t units, bf16* __restrict__ o, float* __restrict__ h_T,
    float* __restrict__ h_T2, SnapArgs snap, int32_t flags) {
    typedef Ws2Cfg<NSW, DUAL> K;
    static_assert(!DUAL || NOOUT, "the paired passes write no outputs");
    constexpr int KP = K::KP, TP = K::TP, AP = K::AP, DV = K::DV, VP = K::VP;

    // XCD-aware id: the column slices of one (sequence, head) share the
    // id's residue mod 8, i.e. one XCD and its L2
    const int x = blockIdx.x;
    const int xcd = x % kXcd2;
    const int qd = x / kXcd2;
    const int slice = qd % split;
    const int unit = (qd / split) * kXcd2 + xcd;
    if (unit >= units) return;
    const int n = unit / H;
    const int h = unit % H;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto kn_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::KN0 + s * K::szTok); };
    auto qs_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::QS0 + s * K::szTok); };
    auto kv_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::KV0 + s * K::szTok); };
    auto kh_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::KH0 + s * K::szTok); };
    auto gam_s = [&](int s) { return reinterpret_cast<float*>(smem + K::GAM0 + s * 512); };
    auto beta_s = [&](int s) { return reinterpret_cast<float*>(smem + K::BETA0 + s * 64); };
    auto a_s = [&](int s) { return reinterpret_cast<float*>(smem + K::A0 + s * K::szA); };
    auto p_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::P0 + s * K::szTile); };
    auto t_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::T0 + s * K::szTile); };
    auto vt_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::VT0 + s * K::szVO); };
    auto ot_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::OT0 + s * K::szVO); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[n + 1] : T_total;
    const int64_t seqlen = eos - bos;
    const int nch = (int)((seqlen + kC2 - 1) / kC2);
    const size_t rowstride = (size_t)H * kHeadDim;
    const size_t headoff = (size_t)h * kHeadDim;
    const int col0 = slice * DV;
    // iterations c = -3 .. nch (the last one stores the outputs of chunk
    // nch - 1), rounded up to whole trips of four
    const int trips = (nch + 4 + 3) / 4;

    if (nch == 0) {   // empty sequence: h_T = h0 (or zero / identity); the M pass: I
        const bool mp = DUAL && wave >= NSW;
        float* hT = mp ? h_T2 : h_T;
        if (wave < K::NSA && hT) {
            const float* src = (h0 && !mp) ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim) : nullptr;
            const bool ident = mp || (flags & kChunkH0Identity);
            float* dst = hT + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
            const int j = col0 + 16 * (mp ? wave - NSW : wave) + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * it + 4 * g + e;
                    const int idx = row * kHeadDim + j;
                    dst[idx] = src ? src[idx] : (ident && row == j ? 1.f : 0.f);
                }
        }
        return;
    }

    // The rings start out holding the identity chunk: zeros, Gamma = 1.
    {
        typedef unsigned int uintx4_t __attribute__((ext_vector_type(4)));
        for (size_t b = (size_t)tid * 16; b < K::bytes; b += (size_t)K::NT * 16)
            *reinterpret_cast<uintx4_t*>(smem + b) = uintx4_t{0u, 0u, 0u, 0u};
        __syncthreads();
        for (int i = tid; i < 4 * kHeadDim; i += K::NT) gam_s(0)[i] = 1.f;
        __syncthreads();
    }

    if (wave < K::NSA) {
        // ======================= state waves =======================
        // the state chain is the pipeline's longest dependency path: its
        // waves win issue arbitration against the prep waves of their SIMD
        __builtin_amdgcn_s_setprio(3);
        // sw: the wave's index within its pass (the M pass of DUAL takes
        // the identity start and V = 0)
        const bool mpass = DUAL && wave >= NSW;
        const int sw = mpass ? wave - NSW : wave;
        floatx4 S[8];
        {
            const float* src = (h0 && !mpass) ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim)
                                              : nullptr;
            const int j = col0 + 16 * sw + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[it][e] = src ? src[(16 * it + 4 * g + e) * kHeadDim + j] : 0.f;
            if (!src && (mpass || (flags & kChunkH0Identity))) {
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (16 * it + 4 * g + e == j) S[it][e] = 1.f;
            }
        }
        const bool write_o = !(flags & kChunkNoOutput);
        const bool v_zero = mpass || (flags & kChunkVZero);
        const bf16 z = (bf16)0.f;
        // Snapshots: the state after every `every_chunks` full chunks of the
        // sequence, the j-th into entry base + j - 1 (base = snap_cu[n], or
        // the sequence's first table slot for the backward's per-chunk
        // tables); fp32 row-major, or bf16 transposed through a wave-private
        // LDS tile (kChunkSnapBf16).  The chunk after which the next one is
        // due is counted down, so the test per chunk is one comparison.
        int64_t snap_idx = (flags & kChunkSnapSlots) ? chunk_slot(bos, n)
                           : snap.snap_cu ? (int64_t)snap.snap_cu[n] : 0;
        const uint32_t snap_lane = (uint32_t)((4 * g * kHeadDim + col0 + 16 * sw + l16) * 4);
        int next_snap = snap.snap ? snap.every_chunks - 1 : 0x7fffffff;

        auto state_iter = [&](auto kc, auto gram, int c) {
            constexpr int KK = decltype(kc)::value;
            constexpr int sc = slot4<KK, 0>();      // chunk c
            constexpr int sc2 = slot2<KK, 0>();
            const bf16* Kn = kn_s(sc) + l16 * KP;
            const bf16* Qs = qs_s(sc) + l16 * KP;
            floatx4 X;
            [[maybe_unused]] floatx4 Ov = zero4();
            if (v_zero) {
                X = zero4();
            } else {
                const bf16x4 v4 = lds_col4(vt_s(sc) + 4 * g * VP + 16 * sw, VP, l16);
#pragma unroll
                for (int e = 0; e < 4; ++e) X[e] = (float)v4[e];
            }
            // X = V - Ktil S, O = Qtil S
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16x8 sb = acc_frag_k32(S[2 * b], S[2 * b + 1]);
                X = mma_bf16_k32(frag_k32(Kn, 32 * b, g), sb, X);
                if constexpr (!NOOUT) Ov = mma_bf16_k32(frag_k32(Qs, 32 * b, g), sb, Ov);
            }
            // U = T X, O += P U (as the k = 32 product with a zero upper half,
            // the same opcode as the Qtil S chain on this accumulator)
            const bf16x4 at = frag_k16(t_s(sc2) + l16 * TP, 0, g);
            const floatx4 U = mma_bf16_k16(at, acc_frag_k16(X), zero4());
            const bf16x4 ub = acc_frag_k16(U);
            if constexpr (!NOOUT) {
                const bf16x4 ap = frag_k16(p_s(sc) + l16 * TP, 0, g);
                Ov = mma_bf16_k32(bf16x8{ap[0], ap[1], ap[2], ap[3], z, z, z, z},
                                  bf16x8{ub[0], ub[1], ub[2], ub[3], z, z, z, z}, Ov);
            }
            if (!NOOUT && write_o) {
                bf16* ot = ot_s(sc2) + 16 * sw + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) ot[(4 * g + e) * VP] = (bf16)Ov[e];
            }
            // S <- Diag(Gamma) S + Kvec^T U
            // Gamma of rows 16 it + 4 g + e: lane (l16, g) of the row of lanes g
            // holds Gamma[16 (l16 / 2) + 4 g + 2 (l16 % 2) + {0, 1}], broadcast
            // to the row inside the multiply
            const float2 gv = *reinterpret_cast<const float2*>(
                gam_s(sc) + 16 * (l16 >> 1) + 4 * g + 2 * (l16 & 1));
            const bf16* Kv = kv_s(sc);
            auto scale_row = [&](auto itc) {
                constexpr int it = decltype(itc)::value;
                floatx4 sc4;
                sc4[0] = S[it][0] * row_bcast<2 * it>(gv.x);
                sc4[1] = S[it][1] * row_bcast<2 * it>(gv.y);
                sc4[2] = S[it][2] * row_bcast<2 * it + 1>(gv.x);
                sc4[3] = S[it][3] * row_bcast<2 * it + 1>(gv.y);
                const bf16x4 a = lds_col4(Kv + 4 * g * KP + 16 * it, KP, l16);
                S[it] = mma_bf16_k16(a, ub, sc4);
            };
            scale_row(std::integral_constant<int, 0>{});
            scale_row(std::integral_constant<int, 1>{});
            scale_row(std::integral_constant<int, 2>{});
            scale_row(std::integral_constant<int, 3>{});
            scale_row(std::integral_constant<int, 4>{});
            scale_row(std::integral_constant<int, 5>{});
            scale_row(std::integral_constant<int, 6>{});
            scale_row(std::integral_constant<int, 7>{});
            if (c == next_snap) {   // uniform branch
                if ((int64_t)kC2 * (c + 1) <= seqlen && snap_idx < snap.n_snap) {
                    const size_t eo = ((size_t)snap_idx * (size_t)H + h) * (kHeadDim * kHeadDim);
                    if (flags & kChunkSnapBf16) {
                        // transposed entry: this wave's 16 columns are 16
                        // contiguous rows of 128
                        const rsrc_t rs = make_rsrc(reinterpret_cast<bf16*>(snap.snap) + eo,
                                                    kHeadDim * kHeadDim * 2);
                        bf16* tile = reinterpret_cast<bf16*>(smem + K::TILE0) +
                                     (size_t)wave * kC2 * kTileTP;
                        store_tile_t(S, tile, rs, (uint32_t)((col0 + 16 * sw) * kHeadDim * 2), lane);
                    } else {
                        const rsrc_t rs = make_rsrc(snap.snap + eo, kHeadDim * kHeadDim * 4);
#pragma unroll
                        for (int it = 0; it < 8; ++it)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                buf_store_f32(S[it][e], rs, snap_lane, ((16 * it + e) * kHeadDim) * 4);
                    }
                }
                ++snap_idx;
                next_snap += snap.every_chunks;
            }
            // Gram tiles of chunk c+2: wave 0 A (stored negated), wave 1 P
            if constexpr (decltype(gram)::value) {
                constexpr int sg = slot4<KK, 2>();
                constexpr int sgh = slot2<KK, 2>();
                const bool isP = wave == 1;
                const bf16* arow = kh_s(sgh) + l16 * KP;
                const bf16* brow = (isP ? qs_s(sg) : kn_s(sg)) + l16 * KP;
                floatx4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < kHeadDim; kb += 32)
                    acc = mma_bf16_k32(frag_k32(arow, kb, g), frag_k32(brow, kb, g), acc);
                if (!isP) {
                    const float br = beta_s(sg)[l16];
                    floatx4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = (4 * g + e >= l16) ? 0.f : acc[e] * br;
                    *reinterpret_cast<floatx4*>(a_s(sgh) + l16 * AP + 4 * g) = out;
                } else {
                    bf16x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = (bf16)((4 * g + e > l16) ? 0.f : acc[e]);
                    *reinterpret_cast<bf16x4*>(p_s(sg) + l16 * TP + 4 * g) = out;
                }
            }
            __syncthreads();
        };
        auto state_loop = [&](auto gram) {
            for (int t = 0, c = -3; t < trips; ++t, c += 4) {
                state_iter(std::integral_constant<int, 0>{}, gram, c);
                state_iter(std::integral_constant<int, 1>{}, gram, c + 1);
                state_iter(std::integral_constant<int, 2>{}, gram, c + 2);
                state_iter(std::integral_constant<int, 3>{}, gram, c + 3);
            }
        };
        // (without outputs P is not needed: wave 1 forms no tile)
        if (wave == 0 || (!NOOUT && wave == 1)) state_loop(std::true_type{});
        else state_loop(std::false_type{});
        float* hT = mpass ? h_T2 : h_T;
        if (hT) {
            float* dst = hT + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
            const int j = col0 + 16 * sw + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * it + 4 * g + e) * kHeadDim + j] = S[it][e];
        }
        return;
    }

    // ========================= prep waves =========================
    const int pw = wave - K::NSA;       // 0..7
    const int r = l16;                  // token of the chunk
    const int ch0 = 16 * pw + 4 * g;    // first of this lane's 4 key channels
    bf16x4 rq[4], rk[4], rg[4];
    bf16 rb[4];
    bf16x8 rv[4];
    static_assert(DV / 32 <= 4, "V / O waves are prep waves 0..3");
    const bool io_wave = pw >= 4 - DV / 32 && pw < 4;
    const int io_u = (pw - (4 - DV / 32)) * 64 + lane;
    const int io_row = io_u / (DV / 8), io_col = (io_u % (DV / 8)) * 8;
    const uint32_t io_off = (uint32_t)(((size_t)io_row * rowstride + headoff + col0 + io_col) * 2);
    const bool write_o = !(flags & kChunkNoOutput);
    // chunk y starts y * cstride elements after the sequence's first row and
    // has chunk_rows(y) rows inside it (0 before the start or past the end)
    const size_t cstride = (size_t)kC2 * rowstride;
    const uint32_t last_rows = (uint32_t)(seqlen - (int64_t)kC2 * (nch - 1));
    auto chunk_rows = [&](int y) -> uint32_t {
        return (y < 0 || y >= nch) ? 0u : (y < nch - 1 ? (uint32_t)kC2 : last_rows);
    };
    const uint32_t row_bytes = (uint32_t)(rowstride * 2);
    const size_t seq0 = (size_t)bos * rowstride;
    const bf16 *q_seq = q + seq0, *k_seq = k + seq0, *g_seq = log_alpha + seq0, *v_seq = v + seq0;
    bf16* o_seq = o + seq0;
    const bf16* b_seq = beta + (size_t)bos * H;
    const bool q_none = flags & kChunkNoOutput, v_none = flags & kChunkVZero;
    const uint32_t qo_lane = (uint32_t)(((size_t)r * rowstride + headoff + ch0) * 2);
    const uint32_t bo_lane = (uint32_t)(((size_t)r * H + h) * 2);
    auto load_chunk = [&](auto slot_c, int yc, auto io) {
        constexpr int s = decltype(slot_c)::value;
        // (a chunk index below zero gives an empty resource: no address is formed)
        const size_t off = yc > 0 ? (size_t)yc * cstride : 0;
        const uint32_t rows = chunk_rows(yc), bytes = rows * row_bytes;
        rq[s] = buf_load_bf16x4(make_rsrc_u32(q_seq + off, q_none ? 0u : bytes), qo_lane);
        rk[s] = buf_load_bf16x4(make_rsrc_u32(k_seq + off, bytes), qo_lane);
        rg[s] = buf_load_bf16x4(make_rsrc_u32(g_seq + off, bytes), qo_lane);
        rb[s] = buf_load_bf16(make_rsrc_u32(b_seq + (yc > 0 ? (size_t)yc * kC2 * H : 0),
                                            rows * (uint32_t)H * 2),
                              bo_lane);
        if (io)
            rv[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                   make_rsrc_u32(v_seq + off, v_none ? 0u : bytes),
                                                   (int)io_off, 0, 0));
    };
    load_chunk(std::integral_constant<int, 0>{}, 0, io_wave);
    load_chunk(std::integral_constant<int, 1>{}, 1, io_wave);
    load_chunk(std::integral_constant<int, 2>{}, 2, io_wave);
    load_chunk(std::integral_constant<int, 3>{}, 3, io_wave);

    auto prep_iter = [&](auto kc, int c, auto solve, auto io) {
        constexpr int KK = decltype(kc)::value;   // register slot of chunk c+3 = KK
        constexpr int s3 = slot4<KK, 3>();
        constexpr int s3h = slot2<KK, 3>();
        // (1) decay factors and scaled operands of chunk c+3
        {
            float kf[4], qf[4], lg[4];
            const float bt = (float)rb[KK];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = (float)rk[KK][e];
                qf[e] = (float)rq[KK][e];
                lg[e] = (float)rg[KK][e] * kLog2e2;
            }
            bf16x4 kn, qs, kh, kv;
            floatx4 gam;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float Pr = row_prefix_sum(lg[e]);           // G_r / ln 2
                const float E = __builtin_amdgcn_exp2f(Pr);       // exp(G_r)       <= 1
                const float Einv = __builtin_amdgcn_exp2f(-Pr);   // exp(-G_r)      <= e^80
                gam[e] = row_bcast<15>(E);                        // exp(G_C)
                const float Hs = gam[e] * Einv;                   // exp(G_C - G_r) <= 1
                kn[e] = (bf16)(-kf[e] * E);
                qs[e] = (bf16)(qf[e] * E);
                kh[e] = (bf16)(kf[e] * Einv);
                kv[e] = (bf16)(kf[e] * Hs);
            }
            *reinterpret_cast<bf16x4*>(kv_s(s3) + r * KP + ch0) = kv;
            *reinterpret_cast<bf16x4*>(kn_s(s3) + r * KP + ch0) = kn;
            *reinterpret_cast<bf16x4*>(qs_s(s3) + r * KP + ch0) = qs;
            *reinterpret_cast<bf16x4*>(kh_s(s3h) + r * KP + ch0) = kh;
            if (r == 0) *reinterpret_cast<floatx4*>(gam_s(s3) + ch0) = gam;
            if (pw == 0 && g == 0) beta_s(s3)[r] = bt;
            if (io) *reinterpret_cast<bf16x8*>(vt_s(s3) + io_row * VP + io_col) = rv[KK];
        }
        // (2) O of chunk c-1 out of its tile (dropped outside the sequence)
        if (io && write_o) {
            constexpr int so = slot2<KK, -1>();
            const int y = c - 1;
            buf_store_b128(*reinterpret_cast<const bf16x8*>(ot_s(so) + io_row * VP + io_col),
                           make_rsrc_u32(o_seq + (y > 0 ? (size_t)y * cstride : 0),
                                         chunk_rows(y) * row_bytes),
                           io_off, 0);
        }
        // loads of chunk c+7 into this register slot
        load_chunk(kc, c + 7, io);
        // (3) UT transform of chunk c+1 on prep waves 0 and 1: lane = elements
        // (row l16, columns 8 pw + g and 8 pw + g + 4) of (I + A)^{-1},
        // forward elimination of both columns with the pivot broadcast along
        // the row of 16 lanes inside the FMA
        if constexpr (decltype(solve)::value) {
            constexpr int s1 = slot4<KK, 1>();
            constexpr int s1h = slot2<KK, 1>();
            const float* Arow = a_s(s1h) + l16 * AP;
            float a[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(Arow + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[4 * q4 + e] = v4[e];
            }
            const int ca = 8 * pw + g, cb = ca + 4;
            float xa = (l16 == ca) ? 1.f : 0.f, xb = (l16 == cb) ? 1.f : 0.f;
            row_bcast_fmac_x2<0>(xa, xb, a[0]);
            row_bcast_fmac_x2<1>(xa, xb, a[1]);
            row_bcast_fmac_x2<2>(xa, xb, a[2]);
            row_bcast_fmac_x2<3>(xa, xb, a[3]);
            row_bcast_fmac_x2<4>(xa, xb, a[4]);
            row_bcast_fmac_x2<5>(xa, xb, a[5]);
            row_bcast_fmac_x2<6>(xa, xb, a[6]);
            row_bcast_fmac_x2<7>(xa, xb, a[7]);
            row_bcast_fmac_x2<8>(xa, xb, a[8]);
            row_bcast_fmac_x2<9>(xa, xb, a[9]);
            row_bcast_fmac_x2<10>(xa, xb, a[10]);
            row_bcast_fmac_x2<11>(xa, xb, a[11]);
            row_bcast_fmac_x2<12>(xa, xb, a[12]);
            row_bcast_fmac_x2<13>(xa, xb, a[13]);
            row_bcast_fmac_x2<14>(xa, xb, a[14]);
            t_s(s1h)[l16 * TP + ca] = (bf16)(xa * beta_s(s1)[ca]);
            t_s(s1h)[l16 * TP + cb] = (bf16)(xb * beta_s(s1)[cb]);
        }
        __syncthreads();
    };
    auto prep_loop = [&](auto solve, auto io) {
        int c = -3;
        for (int t = 0; t < trips; ++t, c += 4) {
            prep_iter(std::integral_constant<int, 0>{}, c, solve, io);
            prep_iter(std::integral_constant<int, 1>{}, c + 1, solve, io);
            prep_iter(std::integral_constant<int, 2>{}, c + 2, solve, io);
            prep_iter(std::integral_constant<int, 3>{}, c + 3, solve, io);
        }
    };
    if (pw < 2) {
        if (io_wave) prep_loop(std::true_type{}, std::true_type{});
        else prep_loop(std::true_type{}, std::false_type{});
    } else if (io_wave) {
        prep_loop(std::false_type{}, std::true_type{});
    } else {
        prep_loop(std::false_type{}, std::false_type{});
    }
}

template <int NSW, bool NOOUT, bool DUAL = false>
hipError_t launch_ws2_t(const ChunkArgs& a, hipStream_t stream) {
    typedef Ws2Cfg<NSW, DUAL> K;
    const int split = kHeadDim / K::DV;
    auto kern = chunk_ws2_kernel<NSW, NOOUT, DUAL>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = raise_lds_limit_once((const void*)kern, (int)K::bytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0) return hipSuccess;
    const int64_t nwg = (units + kXcd2 - 1) / kXcd2 * kXcd2 * split;
    kern<<<dim3((unsigned)nwg), dim3(K::NT), K::bytes, stream>>>(
        (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.log_alpha,
        (const bf16*)a.beta, a.h0, a.cu_seqlens, a.T_total, a.H, split, (int32_t)units,
        (bf16*)a.o, a.h_T, a.h_T2, a.snap, a.flags);
    return hipGetLastError();
}

}  // namespace

}  // namespace kda
