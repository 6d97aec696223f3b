// kda_chunk_ws3.hip -- bf16 prefill with 32-token chunks (two 16-token
// sub-tiles), split 2 (64 value columns per workgroup), gfx950.
//
// Per chunk of 32 tokens with incoming state S0 (sub-tile a = tokens 0..15,
// b = 16..31; decay references as in "From GPT-2 to Kimi K3", ch. 5 "K3's
// lower-bounded decay" and ch. 6 "Chunkwise execution"):
//   every sub-tile is scanned from its own start: E = exp(G) <= 1, 1/E <=
//   e^80 (16 tokens of log-decay above -5), Gam_a, Gam_b its total decay;
//   chunk-relative operands for the state:
//     Ktil = [-k_a E_a ; -k_b E_b Gam_a],  Qtil = [q_a E_a ; q_b E_b Gam_a],
//     Kvec = [k_a Gam_a / E_a * Gam_b ; k_b Gam_b / E_b],  Gamma = Gam_a Gam_b;
//   the 32 x 32 Gram matrices from sub-tile-relative factors only:
//     A_aa = beta_a (k_a E_a)(k_a / E_a)^T,  A_bb likewise,
//     A_ba = beta_b (k_b E_b)(k_a Gam_a / E_a)^T   (both factors <= 1),
//     P the same with q in place of beta k (diagonal blocks inclusive);
//   T = (I + A)^{-1} diag(beta), U = T (V - Ktil S0),
//   O = Qtil S0 + P U,  S_C = Diag(Gamma) S0 + Kvec^T U.
// Chunk-relative factors below e^-80 may underflow to zero; they multiply
// contributions that are at most that small.  No factor exceeds e^80.
//
// Waves: 0-3 state (16 value columns each, the state in MFMA accumulators;
// every product is a 16x16x32 bf16 MFMA: K = 128 channels or 32 tokens);
// 4-11 prep (lane = token r of both sub-tiles x 4 key channels).  Prep waves
// 0-3 also run the UT solve, 4-6 the Gram tiles, 6-7 move V in and O out.
// Pipeline: iteration c preps chunk c+3, forms the Gram tiles of c+2,
// solves c+1 and advances the state through c; one barrier per iteration.
// Ring slots are compile-time constants (loop unrolled four times); the
// rings start as the identity chunk (Gamma = 1, all else 0) and chunks
// outside a sequence read zeros through their buffer resources (again the
// identity), their outputs falling outside the resources.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC3 = 32;       // tokens per chunk
constexpr int kSub = 16;      // tokens per sub-tile
constexpr int kXcd3 = 8;      // MI355X accelerator complex dies
constexpr float kLog2e3 = 1.4426950408889634f;

struct Ws3Cfg {
    static constexpr int NSW = 4;                // state waves
    static constexpr int NPW = 8;                // prep waves
    static constexpr int NT = 64 * (NSW + NPW);  // threads
    static constexpr int DV = 16 * NSW;          // value columns per workgroup
    // bf16 stride of [token][channel] rows: 280 bytes (6 banks apart: row
    // reads, transposed column reads and row writes of 16 rows conflict-free)
    static constexpr int KP = kHeadDim + 12;
    static constexpr int TP = kC3 + 4;           // bf16 stride of T and P rows (72 bytes)
    static constexpr int AP = 20;                // fp32 stride of A rows
    static constexpr int VP = DV + 8;            // bf16 stride of the V / O tiles

    static constexpr size_t szRow16 = kSub * KP * 2;     // 16 token rows
    static constexpr size_t szTP = kC3 * TP * 2;
    static constexpr size_t szA = 3 * kSub * AP * 4;     // A_aa, A_ba, A_bb
    static constexpr size_t szVO = kC3 * VP * 2;
    // 4 slots: Ktil rows a, Qtil rows a (Gram operands, then state operands)
    static constexpr size_t KNA0 = 0;
    static constexpr size_t QSA0 = KNA0 + 4 * szRow16;
    // 2 slots: Ktil rows b, Qtil rows b, Kvec rows a and b (state operands)
    static constexpr size_t KNB0 = QSA0 + 4 * szRow16;
    static constexpr size_t QSB0 = KNB0 + 2 * szRow16;
    static constexpr size_t KV0 = QSB0 + 2 * szRow16;    // 32 rows
    // 2 slots: Gram-only operands: Khat a and b (32 rows), sub-tile-relative
    // Ktil_b and Qtil_b, Kvec_a relative to the end of sub-tile a
    static constexpr size_t KH0 = KV0 + 2 * 2 * szRow16;
    static constexpr size_t KNS0 = KH0 + 2 * 2 * szRow16;
    static constexpr size_t QSS0 = KNS0 + 2 * szRow16;
    static constexpr size_t KVS0 = QSS0 + 2 * szRow16;
    static constexpr size_t GAM0 = KVS0 + 2 * szRow16;   // Gamma, 4 slots
    static constexpr size_t BETA0 = GAM0 + 4 * 512;      // beta, 4 slots
    static constexpr size_t A0 = BETA0 + 4 * 128;        // A blocks, 2 slots
    static constexpr size_t P0 = A0 + 2 * szA;           // P, 4 slots
    static constexpr size_t T0 = P0 + 4 * szTP;          // T, 2 slots
    static constexpr size_t VT0 = T0 + 2 * szTP;         // V, 2 slots
    static constexpr size_t OT0 = VT0 + 2 * szVO;        // O, 2 slots
    static constexpr size_t bytes = OT0 + 2 * szVO;
    static_assert(bytes <= 160 * 1024, "LDS budget");
    static_assert(bytes % 16 == 0, "16-byte initialisation");
};

// Ring slot of chunk c0 + 4j + K + OFF for a loop that starts at c0 = -3.
template <int K, int OFF>
constexpr int slot4() { return (K + OFF + 1) & 3; }
template <int K, int OFF>
constexpr int slot2() { return (K + OFF + 1) & 1; }

// fp32 rounded to bf16 (RNE) in pairs (v_cvt_pk_bf16_f32): converted one
// element at a time, the compiler repacks every pair with a permute.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 t) {
    const bf16x2 lo = __builtin_convertvector(floatx2{t[0], t[1]}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(floatx2{t[2], t[3]}, bf16x2);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}
// B operand over k = 32 from accumulator tiles lo (k 4g..) and hi (k 16+4g..)
__device__ __forceinline__ bf16x8 to_bf16x8(floatx4 lo, floatx4 hi) {
    return __builtin_shufflevector(to_bf16x4(lo), to_bf16x4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// Values a prep lane carries from the prep of a chunk to the iteration that
// writes the chunk's state operands (two iterations later).
struct Held {
    bf16x4 knb, qsb, kva, kvb;
};

__global__ __launch_bounds__(Ws3Cfg::NT) void chunk_ws3_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ log_alpha, const bf16* __restrict__ beta,
    const float* __restrict__ h0, const int32_t* __restrict__ cu_seqlens, int64_t T_total,
    int32_t H, int32_t units, bf16* __restrict__ o, float* __restrict__ h_T, int32_t flags) {
    typedef Ws3Cfg K;
    constexpr int KP = K::KP, TP = K::TP, AP = K::AP, DV = K::DV, VP = K::VP, NSW = K::NSW;
    constexpr int split = kHeadDim / DV;

    // XCD-aware id: the two column slices of one (sequence, head) share the
    // id's residue mod 8, i.e. one XCD and its L2
    const int x = blockIdx.x;
    const int xcd = x % kXcd3;
    const int qd = x / kXcd3;
    const int slice = qd % split;
    const int unit = (qd / split) * kXcd3 + xcd;
    if (unit >= units) return;
    const int n = unit / H;
    const int h = unit % H;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto row16 = [&](size_t base, int s) {
        return reinterpret_cast<bf16*>(smem + base + s * K::szRow16);
    };
    auto kna_s = [&](int s) { return row16(K::KNA0, s); };
    auto qsa_s = [&](int s) { return row16(K::QSA0, s); };
    auto knb_s = [&](int s) { return row16(K::KNB0, s); };
    auto qsb_s = [&](int s) { return row16(K::QSB0, s); };
    auto kv_s = [&](int s) { return row16(K::KV0, 2 * s); };     // 32 rows
    auto kh_s = [&](int s) { return row16(K::KH0, 2 * s); };     // 32 rows
    auto kns_s = [&](int s) { return row16(K::KNS0, s); };
    auto qss_s = [&](int s) { return row16(K::QSS0, s); };
    auto kvs_s = [&](int s) { return row16(K::KVS0, s); };
    auto gam_s = [&](int s) { return reinterpret_cast<float*>(smem + K::GAM0 + s * 512); };
    auto beta_s = [&](int s) { return reinterpret_cast<float*>(smem + K::BETA0 + s * 128); };
    auto a_s = [&](int s) { return reinterpret_cast<float*>(smem + K::A0 + s * K::szA); };
    auto p_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::P0 + s * K::szTP); };
    auto t_s = [&](int s) { return reinterpret_cast<bf16*>(smem + K::T0 + s * K::szTP); };
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
    const int nch = (int)((seqlen + kC3 - 1) / kC3);
    const size_t rowstride = (size_t)H * kHeadDim;
    const size_t headoff = (size_t)h * kHeadDim;
    const int col0 = slice * DV;
    // iterations c = -3 .. nch (the last one stores the outputs of chunk
    // nch - 1), in whole trips of four
    const int trips = (nch + 4 + 3) / 4;

    if (nch == 0) {   // empty sequence: h_T = h0 (or zero / identity)
        if (wave < NSW && h_T) {
            const float* src = h0 ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim) : nullptr;
            const bool ident = flags & kChunkH0Identity;
            float* dst = h_T + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
            const int j = col0 + 16 * wave + l16;
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

    if (wave < NSW) {
        // ======================= state waves =======================
        floatx4 S[8];
        {
            const float* src = h0 ? h0 + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim) : nullptr;
            const int j = col0 + 16 * wave + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[it][e] = src ? src[(16 * it + 4 * g + e) * kHeadDim + j] : 0.f;
            if (!src && (flags & kChunkH0Identity)) {
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (16 * it + 4 * g + e == j) S[it][e] = 1.f;
            }
        }
        const bool write_o = !(flags & kChunkNoOutput);
        const bool v_zero = flags & kChunkVZero;

        auto state_core = [&](auto kc) {
            constexpr int KK = decltype(kc)::value;
            constexpr int s4 = slot4<KK, 0>();      // chunk c
            constexpr int s2 = slot2<KK, 0>();
            floatx4 Xa, Xb, Oa = zero4(), Ob = zero4();
            if (v_zero) {
                Xa = zero4();
                Xb = zero4();
            } else {
                const bf16* vt = vt_s(s2) + 16 * wave;
                const bf16x4 va = lds_col4(vt + 4 * g * VP, VP, l16);
                const bf16x4 vb = lds_col4(vt + (kSub + 4 * g) * VP, VP, l16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Xa[e] = (float)va[e];
                    Xb[e] = (float)vb[e];
                }
            }
            // X = V + (-Ktil) S, O = Qtil S over the 128 channels
            const bf16* kna = kna_s(s4) + l16 * KP;
            const bf16* knb = knb_s(s2) + l16 * KP;
            const bf16* qsa = qsa_s(s4) + l16 * KP;
            const bf16* qsb = qsb_s(s2) + l16 * KP;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const bf16x8 sb = to_bf16x8(S[2 * b], S[2 * b + 1]);
                Xa = mma_bf16_k32(frag_k32(kna, 32 * b, g), sb, Xa);
                Xb = mma_bf16_k32(frag_k32(knb, 32 * b, g), sb, Xb);
                Oa = mma_bf16_k32(frag_k32(qsa, 32 * b, g), sb, Oa);
                Ob = mma_bf16_k32(frag_k32(qsb, 32 * b, g), sb, Ob);
            }
            // U = T X and O += P U over the 32 tokens of the chunk
            const bf16x8 xb = to_bf16x8(Xa, Xb);
            const bf16* tt = t_s(s2) + l16 * TP;
            const floatx4 Ua = mma_bf16_k32(frag_k32(tt, 0, g), xb, zero4());
            const floatx4 Ub = mma_bf16_k32(frag_k32(tt + kSub * TP, 0, g), xb, zero4());
            const bf16x8 ub = to_bf16x8(Ua, Ub);
            const bf16* pp = p_s(s4) + l16 * TP;
            Oa = mma_bf16_k32(frag_k32(pp, 0, g), ub, Oa);
            Ob = mma_bf16_k32(frag_k32(pp + kSub * TP, 0, g), ub, Ob);
            if (write_o) {
                bf16* ot = ot_s(s2) + 16 * wave + l16;
                const bf16x4 oa = to_bf16x4(Oa), ob = to_bf16x4(Ob);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ot[(4 * g + e) * VP] = oa[e];
                    ot[(kSub + 4 * g + e) * VP] = ob[e];
                }
            }
            // S <- Diag(Gamma) S + Kvec^T U
            const float* Gm = gam_s(s4);
            const bf16* Kv = kv_s(s2);
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const floatx4 gm = *reinterpret_cast<const floatx4*>(Gm + 16 * it + 4 * g);
                const bf16x4 alo = lds_col4(Kv + 4 * g * KP + 16 * it, KP, l16);
                const bf16x4 ahi = lds_col4(Kv + (kSub + 4 * g) * KP + 16 * it, KP, l16);
                const bf16x8 a = bf16x8{alo[0], alo[1], alo[2], alo[3],
                                        ahi[0], ahi[1], ahi[2], ahi[3]};
                S[it] = mma_bf16_k32(a, ub, S[it] * gm);
            }
        };
        // one loop per role (the work after the state update)
        auto run_state = [&](auto extra) {
            int c = -3;
            for (int t = 0; t < trips; ++t) {
                auto body = [&](auto kc) {
                    state_core(kc);
                    extra(kc, c);
                    __syncthreads();
                    ++c;
                };
                body(std::integral_constant<int, 0>{});
                body(std::integral_constant<int, 1>{});
                body(std::integral_constant<int, 2>{});
                body(std::integral_constant<int, 3>{});
            }
        };
        if (wave < 3) {
            // Gram tiles of chunk c+2.  Lane (l16, g) of an accumulator holds
            // entry (row l16, columns 4g..4g+3) of the block: the A operand
            // names the columns (earlier tokens s), the B operand the rows
            // (tokens r).  State wave 0: A_aa, P_aa; 1: A_bb, P_bb; 2: A_ba,
            // P_ba (P and -A share the column operand).
            const int blk = wave;
            const bool diag = blk < 2;
            const int rr = blk == 0 ? l16 : kSub + l16;      // chunk row of token r
            const int ablk = blk == 0 ? 0 : (blk == 1 ? 2 : 1);
            run_state([&](auto kc, int) {
                constexpr int KK = decltype(kc)::value;
                constexpr int s2 = slot4<KK, 2>();
                constexpr int s2h = slot2<KK, 2>();
                const bf16* colop =
                    (blk == 0 ? kh_s(s2h) : (blk == 1 ? kh_s(s2h) + kSub * KP : kvs_s(s2h))) +
                    l16 * KP;
                const bf16* rowk = (blk == 0 ? kna_s(s2) : kns_s(s2h)) + l16 * KP;
                const bf16* rowq = (blk == 0 ? qsa_s(s2) : qss_s(s2h)) + l16 * KP;
                floatx4 accA = zero4(), accP = zero4();
#pragma unroll
                for (int kb = 0; kb < kHeadDim; kb += 32) {
                    const bf16x8 cf = frag_k32(colop, kb, g);
                    accA = mma_bf16_k32(cf, frag_k32(rowk, kb, g), accA);
                    accP = mma_bf16_k32(cf, frag_k32(rowq, kb, g), accP);
                }
                const float br = beta_s(s2)[rr];
                floatx4 outA, outP;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int sc = 4 * g + e;
                    outA[e] = (diag && sc >= l16) ? 0.f : accA[e] * br;
                    outP[e] = (diag && sc > l16) ? 0.f : accP[e];
                }
                // A blocks: [A_aa ; A_ba ; A_bb] rows of 16, stored negated
                *reinterpret_cast<floatx4*>(a_s(s2h) + (ablk * kSub + l16) * AP + 4 * g) = outA;
                // P rows: token rr, columns of sub-tile a (blocks aa, ba) or b
                bf16* prow = p_s(s2) + rr * TP + (blk == 1 ? kSub : 0) + 4 * g;
                *reinterpret_cast<bf16x4*>(prow) = to_bf16x4(outP);
                if (blk == 0)   // P_ab = 0
                    *reinterpret_cast<bf16x4*>(prow + kSub) = bf16x4{};
            });
        } else {
            // V in and O out: lane moves four 16-byte pieces of the 32 x DV
            // tile: rows lane / 8 + 8 m, columns 8 (lane % 8) .. +7
            static_assert(DV == 64, "V / O piece mapping");
            const int io_row = lane >> 3, io_col = (lane & 7) * 8;
            const uint32_t io_off =
                (uint32_t)(((size_t)io_row * rowstride + headoff + col0 + io_col) * 2);
            const uint32_t row_bytes = (uint32_t)(rowstride * 2);
            const uint32_t io_step = 8 * row_bytes;
            const size_t cstride = (size_t)kC3 * rowstride;
            const uint32_t last_rows = (uint32_t)(seqlen - (int64_t)kC3 * (nch - 1));
            auto chunk_rows = [&](int y) -> uint32_t {
                return (y < 0 || y >= nch) ? 0u : (y < nch - 1 ? (uint32_t)kC3 : last_rows);
            };
            const size_t seq0 = (size_t)bos * rowstride;
            const bf16* v_seq = v + seq0;
            bf16* o_seq = o + seq0;
            // V of chunk c+1, loaded one iteration ahead (chunk -2 is zero)
            bf16x8 rv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) rv[m] = bf16x8{};
            run_state([&](auto kc, int c) {
                constexpr int KK = decltype(kc)::value;
                constexpr int s1h = slot2<KK, 1>();
                bf16* vt = vt_s(s1h) + io_row * VP + io_col;
#pragma unroll
                for (int m = 0; m < 4; ++m) *reinterpret_cast<bf16x8*>(vt + 8 * m * VP) = rv[m];
                if (write_o) {
                    constexpr int so = slot2<KK, -1>();
                    const int y = c - 1;
                    const rsrc_t ro = make_rsrc_u32(o_seq + (y > 0 ? (size_t)y * cstride : 0),
                                                    chunk_rows(y) * row_bytes);
                    const bf16* ot = ot_s(so) + io_row * VP + io_col;
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        buf_store_b128(*reinterpret_cast<const bf16x8*>(ot + 8 * m * VP), ro,
                                       io_off + m * io_step, 0);
                }
                const int yv = c + 2;
                const rsrc_t rsv = make_rsrc_u32(v_seq + (yv > 0 ? (size_t)yv * cstride : 0),
                                                 v_zero ? 0u : chunk_rows(yv) * row_bytes);
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    rv[m] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                                           rsv, (int)(io_off + m * io_step), 0, 0));
            });
        }
        if (h_T) {
            float* dst = h_T + ((size_t)n * (size_t)H + h) * (kHeadDim * kHeadDim);
            const int j = col0 + 16 * wave + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * it + 4 * g + e) * kHeadDim + j] = S[it][e];
        }
        return;
    }

    // ========================= prep waves =========================
    const int pw = wave - NSW;          // 0..7
    const int r = l16;                  // token r of sub-tile a, 16 + r of b
    const int ch0 = 16 * pw + 4 * g;    // first of this lane's 4 key channels
    // chunk y starts y * cstride elements after the sequence's first row and
    // has chunk_rows(y) rows inside it (0 before the start or past the end)
    const size_t cstride = (size_t)kC3 * rowstride;
    const uint32_t last_rows = (uint32_t)(seqlen - (int64_t)kC3 * (nch - 1));
    auto chunk_rows = [&](int y) -> uint32_t {
        return (y < 0 || y >= nch) ? 0u : (y < nch - 1 ? (uint32_t)kC3 : last_rows);
    };
    const uint32_t row_bytes = (uint32_t)(rowstride * 2);
    const uint32_t sub_bytes = kSub * row_bytes;           // sub-tile b offset
    const size_t seq0 = (size_t)bos * rowstride;
    const bool q_none = flags & kChunkNoOutput;

    // q, k, log alpha, beta of chunk c+3, loaded one iteration ahead
    bf16x4 rqa, rqb, rka, rkb, rga, rgb;
    bf16 rba, rbb;
    {
        const uint32_t qo_lane = (uint32_t)(((size_t)r * rowstride + headoff + ch0) * 2);
        const uint32_t bo_lane = (uint32_t)(((size_t)r * H + h) * 2);
        const uint32_t bo_sub = (uint32_t)(kSub * H * 2);
        const bf16 *q_seq = q + seq0, *k_seq = k + seq0, *g_seq = log_alpha + seq0;
        const bf16* b_seq = beta + (size_t)bos * H;
        auto load_chunk = [&](int yc) {
            // (a chunk index below zero gives an empty resource: no address is formed)
            const size_t off = yc > 0 ? (size_t)yc * cstride : 0;
            const uint32_t rows = chunk_rows(yc), bytes = rows * row_bytes;
            const rsrc_t rq = make_rsrc_u32(q_seq + off, q_none ? 0u : bytes);
            const rsrc_t rk = make_rsrc_u32(k_seq + off, bytes);
            const rsrc_t rg = make_rsrc_u32(g_seq + off, bytes);
            const rsrc_t rb = make_rsrc_u32(b_seq + (yc > 0 ? (size_t)yc * kC3 * H : 0),
                                            rows * (uint32_t)H * 2);
            rqa = buf_load_bf16x4(rq, qo_lane);
            rqb = buf_load_bf16x4(rq, qo_lane + sub_bytes);
            rka = buf_load_bf16x4(rk, qo_lane);
            rkb = buf_load_bf16x4(rk, qo_lane + sub_bytes);
            rga = buf_load_bf16x4(rg, qo_lane);
            rgb = buf_load_bf16x4(rg, qo_lane + sub_bytes);
            rba = buf_load_bf16(rb, bo_lane);
            rbb = buf_load_bf16(rb, bo_lane + bo_sub);
        };

        // state operands of chunk y, held from its prep (iteration y - 3) to
        // the iteration that writes them (y - 1): register slot y & 3
        Held held[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x4 z4 = bf16x4{};
            held[s].knb = held[s].qsb = held[s].kva = held[s].kvb = z4;
        }

        auto prep_core = [&](auto kc) {
            constexpr int KK = decltype(kc)::value;   // c + 3 = 4j + KK
            constexpr int s3 = slot4<KK, 3>();
            constexpr int s3h = slot2<KK, 3>();
            // (1) state operands of chunk c+1, prepped two iterations ago
            {
                constexpr int HS = (KK + 2) & 3;
                constexpr int s1h = slot2<KK, 1>();
                *reinterpret_cast<bf16x4*>(knb_s(s1h) + r * KP + ch0) = held[HS].knb;
                *reinterpret_cast<bf16x4*>(qsb_s(s1h) + r * KP + ch0) = held[HS].qsb;
                *reinterpret_cast<bf16x4*>(kv_s(s1h) + r * KP + ch0) = held[HS].kva;
                *reinterpret_cast<bf16x4*>(kv_s(s1h) + (kSub + r) * KP + ch0) = held[HS].kvb;
            }
            // (2) decay factors and scaled operands of chunk c+3, one operand
            // at a time (each rounded and written as soon as it is formed)
            floatx4 Ea, Eia, Ga, Eb, Eib, Gb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // G_r / ln 2 within each sub-tile
                const float pa = row_prefix_sum((float)rga[e] * kLog2e3);
                const float pb = row_prefix_sum((float)rgb[e] * kLog2e3);
                Ea[e] = __builtin_amdgcn_exp2f(pa);          // <= 1
                Eia[e] = __builtin_amdgcn_exp2f(-pa);        // <= e^80
                Eb[e] = __builtin_amdgcn_exp2f(pb);
                Eib[e] = __builtin_amdgcn_exp2f(-pb);
                Ga[e] = row_bcast<15>(Ea[e]);                // decay over sub-tile a
                Gb[e] = row_bcast<15>(Eb[e]);
            }
            auto put = [&](bf16* dst, floatx4 val) {
                *reinterpret_cast<bf16x4*>(dst + ch0) = to_bf16x4(val);
            };
            floatx4 t, u;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -(float)rka[e] * Ea[e];
            put(kna_s(s3) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = (float)rqa[e] * Ea[e];
            put(qsa_s(s3) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = (float)rka[e] * Eia[e];
            put(kh_s(s3h) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = (float)rka[e] * (Ga[e] * Eia[e]);   // to the end of sub-tile a, <= 1
                u[e] = t[e] * Gb[e];                       // to the chunk end
            }
            held[KK].kva = to_bf16x4(u);
            put(kvs_s(s3h) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = -(float)rkb[e] * Eb[e];
                u[e] = t[e] * Ga[e];                       // to the chunk start
            }
            held[KK].knb = to_bf16x4(u);
            put(kns_s(s3h) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = (float)rqb[e] * Eb[e];
                u[e] = t[e] * Ga[e];
            }
            held[KK].qsb = to_bf16x4(u);
            put(qss_s(s3h) + r * KP, t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = (float)rkb[e] * Eib[e];
                u[e] = (float)rkb[e] * (Gb[e] * Eib[e]);   // to the chunk end
            }
            held[KK].kvb = to_bf16x4(u);
            put(kh_s(s3h) + (kSub + r) * KP, t);
            if (r == 0) *reinterpret_cast<floatx4*>(gam_s(s3) + ch0) = Ga * Gb;
            if (pw == 0 && g == 0) {
                beta_s(s3)[r] = (float)rba;
                beta_s(s3)[kSub + r] = (float)rbb;
            }
        };

        // one loop per role (the role's work after the common prep), so no
        // wave carries another role's registers
        auto run = [&](auto extra) {
            load_chunk(0);
            int c = -3;
            for (int t = 0; t < trips; ++t) {
                auto body = [&](auto kc) {
                    prep_core(kc);
                    load_chunk(c + 4);
                    extra(kc, c);
                    __syncthreads();
                    ++c;
                };
                body(std::integral_constant<int, 0>{});
                body(std::integral_constant<int, 1>{});
                body(std::integral_constant<int, 2>{});
                body(std::integral_constant<int, 3>{});
            }
        };

        if (pw < 4) {
            // UT transform of chunk c+1: lane = column j = 4 pw + g of
            // sub-tile a (rows r and 16 + r) and column 16 + j (row 16 + r)
            // of (I + A)^{-1}: forward elimination down the 32 columns of A,
            // each pivot broadcast along the row of 16 lanes (A is stored
            // negated and strictly lower triangular)
            const int j = 4 * pw + g;
            run([&](auto kc, int) {
                constexpr int KK = decltype(kc)::value;
                constexpr int s1 = slot4<KK, 1>();
                constexpr int s1h = slot2<KK, 1>();
                const float* Ab = a_s(s1h);
                float aaa[16], aba[16], abb[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const floatx4 v0 = *reinterpret_cast<const floatx4*>(Ab + l16 * AP + 4 * q4);
                    const floatx4 v1 =
                        *reinterpret_cast<const floatx4*>(Ab + (kSub + l16) * AP + 4 * q4);
                    const floatx4 v2 =
                        *reinterpret_cast<const floatx4*>(Ab + (2 * kSub + l16) * AP + 4 * q4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        aaa[4 * q4 + e] = v0[e];
                        aba[4 * q4 + e] = v1[e];
                        abb[4 * q4 + e] = v2[e];
                    }
                }
                float xt = (l16 == j) ? 1.f : 0.f;   // column j, row r
                float xb = 0.f;                      // column j, row 16 + r
                float yb = xt;                       // column 16 + j, row 16 + r
                // pivots 0..15 (rows of sub-tile a): both rows of column j
#define KDA_SOLVE_A(I) row_bcast_fmac2<I>(xb, xt, aba[I]); row_bcast_fmac<I>(xt, aaa[I]);
                KDA_SOLVE_A(0) KDA_SOLVE_A(1) KDA_SOLVE_A(2) KDA_SOLVE_A(3)
                KDA_SOLVE_A(4) KDA_SOLVE_A(5) KDA_SOLVE_A(6) KDA_SOLVE_A(7)
                KDA_SOLVE_A(8) KDA_SOLVE_A(9) KDA_SOLVE_A(10) KDA_SOLVE_A(11)
                KDA_SOLVE_A(12) KDA_SOLVE_A(13) KDA_SOLVE_A(14)
#undef KDA_SOLVE_A
                row_bcast_fmac2<15>(xb, xt, aba[15]);
                // pivots 16..30 (rows of sub-tile b): columns j and 16 + j
#define KDA_SOLVE_B(I) row_bcast_fmac<I>(xb, abb[I]); row_bcast_fmac<I>(yb, abb[I]);
                KDA_SOLVE_B(0) KDA_SOLVE_B(1) KDA_SOLVE_B(2) KDA_SOLVE_B(3)
                KDA_SOLVE_B(4) KDA_SOLVE_B(5) KDA_SOLVE_B(6) KDA_SOLVE_B(7)
                KDA_SOLVE_B(8) KDA_SOLVE_B(9) KDA_SOLVE_B(10) KDA_SOLVE_B(11)
                KDA_SOLVE_B(12) KDA_SOLVE_B(13) KDA_SOLVE_B(14)
#undef KDA_SOLVE_B
                const float bj = beta_s(s1)[j], bj2 = beta_s(s1)[kSub + j];
                bf16* tt = t_s(s1h);
                tt[l16 * TP + j] = (bf16)(xt * bj);
                tt[l16 * TP + kSub + j] = (bf16)0.f;
                tt[(kSub + l16) * TP + j] = (bf16)(xb * bj);
                tt[(kSub + l16) * TP + kSub + j] = (bf16)(yb * bj2);
            });
        } else {
            run([&](auto, int) {});
        }
    }
}

}  // namespace

bool chunk_ws3_supports(const ChunkArgs& a, int split) {
    return split == 2 && !a.snap.snap &&
           !(a.flags & (kChunkDualBM | kChunkSnapBf16 | kChunkSnapSlots));
}

hipError_t launch_chunk_ws3(const ChunkArgs& a, int split, hipStream_t stream) {
    if (!chunk_ws3_supports(a, split)) return hipErrorInvalidValue;
    typedef Ws3Cfg K;
    auto kern = chunk_ws3_kernel;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = raise_lds_limit_once((const void*)kern, (int)K::bytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0) return hipSuccess;
    const int64_t nwg = (units + kXcd3 - 1) / kXcd3 * kXcd3 * (kHeadDim / K::DV);
    kern<<<dim3((unsigned)nwg), dim3(K::NT), K::bytes, stream>>>(
        (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.log_alpha,
        (const bf16*)a.beta, a.h0, a.cu_seqlens, a.T_total, a.H, (int32_t)units, (bf16*)a.o,
        a.h_T, a.flags);
    return hipGetLastError();
}

}  // namespace kda
