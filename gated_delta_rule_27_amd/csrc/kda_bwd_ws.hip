// kda_bwd_ws.hip -- the reverse recursion of the KDA backward pass for bf16
// inputs, wave-specialised and software-pipelined like the bf16 prefill
// kernel (kda_chunk_ws2.hip), walking the chunks of a sequence backwards.
//
// For a chunk with the decay-scaled operands of the forward (kda_bwd.hip,
// header) and the state gradient D arriving from later chunks:
//   dU = Kv D + P^T dO,   dX = T^T dU,
//   D  <- Diag(Gamma) D + Qt^T dO - Kt^T dX          (the chunk before)
// and D is stored, before the update, as the table entry of the chunk.
// This is the transpose of the forward's state chain, so the same pipeline
// carries it: in iteration y the state waves run step y (the chunk y from
// the end), state waves 0 and 1 form the Gram tiles of step y+2, prep waves
// 0 and 1 solve the UT transform of step y+1 (two columns per lane), and the
// 8 prep waves load q, k, log alpha of step y+3 into the lanes that use
// them, take the decay scan across the 16 lanes of a row and write the
// scaled operands; one barrier per step.  Each prep wave runs a loop of its
// own role (solve or not, dO or not), so that its loop body is one basic
// block per step (3.6% faster than role branches inside one loop, and the
// two-column solve a further 1%).  The operands the recursion needs differ
// from the forward's: Kv by rows, Qt^T and -Kt^T by columns, P^T and T^T.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 16;        // tokens per chunk
constexpr int kXcd = 8;       // accelerator complex dies
constexpr float kLn2Inv = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int NSW_>
struct RwsCfg {
    static constexpr int NSW = NSW_;              // state waves, 16 columns each
    static constexpr int NPW = 8;                 // prep waves
    static constexpr int NT = 64 * (NSW + NPW);
    static constexpr int DV = 16 * NSW;           // value columns per workgroup
    static constexpr int KP = kHeadDim + 8;       // bf16 stride of [token][channel]
    static constexpr int TP = kC + 8;             // bf16 stride of [.][token]
    static constexpr int AP = 20;                 // fp32 stride of the A tile
    static constexpr int VP = DV + 8;              // bf16 stride of the dO tile
    static constexpr size_t szTok = kC * KP * 2;
    static constexpr size_t szTile = kC * TP * 2;
    static constexpr size_t szA = kC * AP * 4;
    static constexpr size_t szDO = kC * VP * 2;
    // ring buffers indexed by step; written by prep three iterations before
    // the state stage reads them (Gram operands: one iteration before).
    // Token rows throughout: the state stage reads the operands it needs by
    // columns (Qt^T, -Kt^T) with transposed LDS reads.
    static constexpr size_t KV0 = 0;                         // Kv rows, 4 slots
    static constexpr size_t KN0 = KV0 + 4 * szTok;           // -Kt rows, 4 slots
    static constexpr size_t QS0 = KN0 + 4 * szTok;           // Qt rows, 4 slots
    static constexpr size_t GAM0 = QS0 + 4 * szTok;          // Gamma, 4 slots
    static constexpr size_t KH0 = GAM0 + 4 * 512;            // Khat rows (Gram), 2 slots
    static constexpr size_t DO0 = KH0 + 2 * szTok;           // dO of the workgroup's columns, 4 slots
    static constexpr size_t BETA0 = DO0 + 4 * szDO;          // beta, 3 slots
    static constexpr size_t A0 = BETA0 + 3 * 64;             // A, 2 slots
    static constexpr size_t PT0 = A0 + 2 * szA;              // P^T, 3 slots
    static constexpr size_t TT0 = PT0 + 3 * szTile;          // T^T, 2 slots
    static constexpr size_t TILE0 = TT0 + 2 * szTile;        // per state wave: D table staging
    static constexpr size_t bytes = TILE0 + NSW * kC * kTileTP * 2;
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

template <int NSW>
__global__ __launch_bounds__((RwsCfg<NSW>::NT)) void bwd_dh_ws_kernel(BwdArgs a, int32_t split,
                                                                      int32_t units) {
    typedef RwsCfg<NSW> K;
    constexpr int KP = K::KP, TP = K::TP, AP = K::AP, DV = K::DV;
    constexpr size_t kState = (size_t)kHeadDim * kHeadDim;

    const int x = blockIdx.x;
    const int xcd = x % kXcd;
    const int qd = x / kXcd;
    const int slice = qd % split;
    const int unit = (qd / split) * kXcd + xcd;
    if (unit >= units) return;
    const int n = unit / a.H;
    const int h = unit % a.H;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    auto kv_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KV0 + (y & 3) * K::szTok); };
    auto gam_s = [&](int y) { return reinterpret_cast<float*>(smem + K::GAM0 + (y & 3) * 512); };
    auto kn_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KN0 + (y & 3) * K::szTok); };
    auto qs_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::QS0 + (y & 3) * K::szTok); };
    auto do_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::DO0 + (y & 3) * K::szDO); };
    auto kh_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::KH0 + (y & 1) * K::szTok); };
    auto beta_s = [&](int y) { return reinterpret_cast<float*>(smem + K::BETA0 + (y % 3) * 64); };
    auto a_s = [&](int y) { return reinterpret_cast<float*>(smem + K::A0 + (y & 1) * K::szA); };
    auto pt_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::PT0 + (y % 3) * K::szTile); };
    auto tt_s = [&](int y) { return reinterpret_cast<bf16*>(smem + K::TT0 + (y & 1) * K::szTile); };

    const bf16* q = static_cast<const bf16*>(a.q);
    const bf16* k = static_cast<const bf16*>(a.k);
    const bf16* lg = static_cast<const bf16*>(a.log_alpha);
    const bf16* bt = static_cast<const bf16*>(a.beta);
    const bf16* dout = static_cast<const bf16*>(a.dout);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int g = lane >> 4;

    const int64_t bos = a.cu_seqlens ? (int64_t)a.cu_seqlens[n] : 0;
    const int64_t eos = a.cu_seqlens ? (int64_t)a.cu_seqlens[n + 1] : a.T_total;
    const int64_t seqlen = eos - bos;
    const int nch = (int)((seqlen + kC - 1) / kC);
    const size_t rowstride = (size_t)a.H * kHeadDim;
    const size_t headoff = (size_t)h * kHeadDim;
    const int col0 = slice * DV;
    const int64_t slot0 = chunk_slot(bos, n);
    const int nit = (nch + 3 + 3) / 4 * 4;
    // chunk of step y (steps run from the last chunk to the first); a
    // negative result or one past the end means "no chunk"
    auto chunk_of = [&](int y) { return nch - 1 - y; };

    if (nch == 0) {   // dh0 = dhT; uniform over the workgroup
        if (wave < NSW && a.dh0) {
            const float* src = a.dhT ? a.dhT + ((size_t)n * a.H + h) * kState : nullptr;
            float* dst = a.dh0 + ((size_t)n * a.H + h) * kState;
            const int j = col0 + 16 * wave + l16;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int idx = (16 * it + 4 * g + e) * kHeadDim + j;
                    dst[idx] = src ? src[idx] : 0.f;
                }
        }
        return;
    }

    // Gram tiles of step zy: acc(s, r) = sum_i Khat_s[i] X_r[i] with X = -Kt
    // (A[r][s] = beta_r Kt_r . Khat_s, strictly lower, stored negated for the
    // solve to add) or Qt (P[r][s], s <= r,
    // stored transposed as P^T[s][r])
    auto gram_tile = [&](bool isP, int zy) {
        const bf16* arow = kh_s(zy) + l16 * KP;
        const bf16* brow = (isP ? qs_s(zy) : kn_s(zy)) + l16 * KP;
        floatx4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < kHeadDim; kb += 32)
            acc = mma_bf16_k32(frag_k32(arow, kb, g), frag_k32(brow, kb, g), acc);
        if (!isP) {
            const float br = beta_s(zy)[l16];
            floatx4 out;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e] = (4 * g + e >= l16) ? 0.f : acc[e] * br;
            *reinterpret_cast<floatx4*>(a_s(zy) + l16 * AP + 4 * g) = out;
        } else {
            bf16* pt = pt_s(zy);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pt[(4 * g + e) * TP + l16] = (bf16)((4 * g + e > l16) ? 0.f : acc[e]);
        }
    };

    // chunk cc's rows inside the sequence as buffer resources (empty when
    // cc is not a chunk: rows past the end read 0), from per-sequence
    // scalar bases: one multiply per chunk, no 64-bit size arithmetic
    const size_t cstride = (size_t)kC * rowstride;
    const uint32_t last_rows = (uint32_t)(seqlen - (int64_t)kC * (nch - 1));
    auto chunk_rows = [&](int cc) -> uint32_t {
        return cc < 0 ? 0u : cc < nch - 1 ? (uint32_t)kC : cc == nch - 1 ? last_rows : 0u;
    };
    const uint32_t row_bytes = (uint32_t)(rowstride * 2);
    const size_t seq0 = (size_t)bos * rowstride;
    auto tok_rsrc = [&](const bf16* base, int cc) {
        return make_rsrc_u32(base + seq0 + (size_t)(cc < 0 ? 0 : cc) * cstride, chunk_rows(cc) * row_bytes);
    };
    auto beta_rsrc = [&](int cc) {
        return make_rsrc_u32(bt + (size_t)bos * a.H + (size_t)(cc < 0 ? 0 : cc) * kC * a.H,
                             chunk_rows(cc) * (uint32_t)a.H * 2);
    };

    if (wave < NSW) {
        // ======================= state waves =======================
        const int colw0 = col0 + 16 * wave + l16;
        floatx4 D[8];
        {
            const float* src = a.dhT ? a.dhT + ((size_t)n * a.H + h) * kState : nullptr;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    D[it][e] = src ? src[(16 * it + 4 * g + e) * kHeadDim + colw0] : 0.f;
        }
        // dO of a step arrives in an LDS tile (the prep waves load it):
        // rows 4g .. 4g+3 of this lane's column by a transposed read
        constexpr int VP = K::VP;
        auto state_iter = [&](int y) {
            if (y >= 0 && y < nch) {
                const int cc = chunk_of(y);
                floatx4 dob;
                {
                    const bf16x4 d4 = lds_col4(do_s(y) + 4 * g * VP + 16 * wave, VP, l16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dob[e] = (float)d4[e];
                }
                // the table entry of this chunk: D before the update
                {
                    const rsrc_t rs = make_rsrc(
                        static_cast<bf16*>(a.dstates) + ((size_t)(slot0 + cc) * a.H + h) * kState,
                        (int64_t)kState * 2);
                    // transposed like the state table: this wave's 16
                    // columns are 16 contiguous rows of 128
                    store_tile_t(D, reinterpret_cast<bf16*>(smem + K::TILE0) +
                                        (size_t)wave * kC * kTileTP,
                                 rs, (uint32_t)((col0 + 16 * wave) * kHeadDim * 2), lane);
                }
                // dU = Kv D + P^T dO
                const bf16* Kv = kv_s(y) + l16 * KP;
                floatx4 dU = zero4();
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    dU = mma_bf16_k32(frag_k32(Kv, 32 * b, g), acc_frag_k32(D[2 * b], D[2 * b + 1]),
                                      dU);
                dU += mma_bf16_k16(frag_k16(pt_s(y) + l16 * TP, 0, g), acc_frag_k16(dob), zero4());
                // dX = T^T dU
                const floatx4 dX =
                    mma_bf16_k16(frag_k16(tt_s(y) + l16 * TP, 0, g), acc_frag_k16(dU), zero4());
                // D <- Diag(Gamma) D + Qt^T dO - Kt^T dX
                const float* Gm = gam_s(y);
                const bf16* Qs = qs_s(y);
                const bf16* Kn = kn_s(y);
                // both terms as one k = 32 product: this lane's eight k slots are
                // (dO, token 4g + e) and (dX, token 4g + e), e = 0..3, matched by
                // the Qt^T and -Kt^T rows 16 it .. +15 over the same tokens
                const bf16x4 dob16 = acc_frag_k16(dob), dX16 = acc_frag_k16(dX);
                const bf16x8 bx{dob16[0], dob16[1], dob16[2], dob16[3], dX16[0], dX16[1], dX16[2], dX16[3]};
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const floatx4 gm = *reinterpret_cast<const floatx4*>(Gm + 16 * it + 4 * g);
                    const bf16x4 qa = lds_col4(Qs + 4 * g * KP + 16 * it, KP, l16);
                    const bf16x4 ka = lds_col4(Kn + 4 * g * KP + 16 * it, KP, l16);
                    D[it] = mma_bf16_k32(bf16x8{qa[0], qa[1], qa[2], qa[3], ka[0], ka[1], ka[2], ka[3]},
                                         bx, D[it] * gm);
                }
            }
            if (wave < 2) {
                const int zy = y + 2;
                if (zy >= 0 && zy < nch) gram_tile(wave == 1, zy);
            }
            __syncthreads();
        };
        for (int y = -3; y < nit - 3; y += 4) {
            state_iter(y);
            state_iter(y + 1);
            state_iter(y + 2);
            state_iter(y + 3);
        }
        if (a.dh0) {
            float* dst = a.dh0 + ((size_t)n * a.H + h) * kState;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[(16 * it + 4 * g + e) * kHeadDim + colw0] = D[it][e];
        }
        return;
    }

    // ========================= prep waves =========================
    const int pw = wave - NSW;        // 0..7
    const int r = l16;                // token of the chunk
    const int ch0 = 16 * pw + 4 * g;  // first of this lane's 4 key channels
    bf16x4 rq[4], rk[4], rg[4];
    bf16 rb[4];
    // dO for the state waves: prep waves 4 - DV / 32 .. 3 load one 16-byte
    // piece of a row of the step's 16 x DV tile per lane, four steps ahead,
    // and write it to the tile in the iteration that prepares the step
    constexpr int VP = K::VP;
    static_assert(DV / 32 <= 4, "dO waves are prep waves 0..3");
    const bool io_wave = pw >= 4 - DV / 32 && pw < 4;
    const int io_u = (pw - (4 - DV / 32)) * 64 + lane;
    const int io_row = io_u / (DV / 8), io_col = (io_u % (DV / 8)) * 8;
    const uint32_t io_off = (uint32_t)(((size_t)io_row * rowstride + headoff + col0 + io_col) * 2);
    bf16x8 rdo[4];
    const uint32_t qo_lane = (uint32_t)(((size_t)r * rowstride + headoff + ch0) * 2);
    const uint32_t bo_lane = (uint32_t)(((size_t)r * a.H + h) * 2);
    auto load_step = [&](auto slot_c, int y, auto io) {
        constexpr int s = decltype(slot_c)::value;
        const int cc = chunk_of(y);
        rq[s] = buf_load_bf16x4(tok_rsrc(q, cc), qo_lane);
        rk[s] = buf_load_bf16x4(tok_rsrc(k, cc), qo_lane);
        rg[s] = buf_load_bf16x4(tok_rsrc(lg, cc), qo_lane);
        rb[s] = buf_load_bf16(beta_rsrc(cc), bo_lane);
        if (io)
            rdo[s] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(tok_rsrc(dout, cc), (int)io_off, 0, 0));
    };
    load_step(std::integral_constant<int, 0>{}, 0, io_wave);
    load_step(std::integral_constant<int, 1>{}, 1, io_wave);
    load_step(std::integral_constant<int, 2>{}, 2, io_wave);
    load_step(std::integral_constant<int, 3>{}, 3, io_wave);

    auto prep_iter = [&](auto slot_c, int y, auto solve, auto io) {
        constexpr int s = decltype(slot_c)::value;  // == (y + 3) & 3
        // (1) decay factors and scaled operands of step y+3
        const int yp = y + 3;
        if (yp < nch) {
            float kf[4], qf[4], lgv[4];
            const float b = (float)rb[s];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = (float)rk[s][e];
                qf[e] = (float)rq[s][e];
                lgv[e] = (float)rg[s][e] * kLn2Inv;
            }
            bf16x4 kv, kn, qs, kh;
            floatx4 gam;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float P = row_prefix_sum(lgv[e]);       // G_r / ln 2
                const float E = exp2_fast(P);                 // exp(G_r)       <= 1
                const float Einv = exp2_fast(-P);             // exp(-G_r)      <= e^80
                gam[e] = row_bcast<15>(E);                    // exp(G_C)
                const float Hs = gam[e] * Einv;               // exp(G_C - G_r) <= 1
                const float kt = kf[e] * E, qt = qf[e] * E;
                kv[e] = (bf16)(kf[e] * Hs);
                kn[e] = (bf16)(-kt);
                qs[e] = (bf16)qt;
                kh[e] = (bf16)(kf[e] * Einv);
            }
            *reinterpret_cast<bf16x4*>(kv_s(yp) + r * KP + ch0) = kv;
            *reinterpret_cast<bf16x4*>(kn_s(yp) + r * KP + ch0) = kn;
            *reinterpret_cast<bf16x4*>(qs_s(yp) + r * KP + ch0) = qs;
            *reinterpret_cast<bf16x4*>(kh_s(yp) + r * KP + ch0) = kh;
            if (r == 0) *reinterpret_cast<floatx4*>(gam_s(yp) + ch0) = gam;
            if (pw == 0 && g == 0) beta_s(yp)[r] = b;
            if (io) *reinterpret_cast<bf16x8*>(do_s(yp) + io_row * VP + io_col) = rdo[s];
        }
        load_step(slot_c, yp + 4, io);
        // (2) UT transform of step y+1 on prep waves 0 and 1: lane = (row l16,
        // columns 8 pw + g and 8 pw + g + 4) of (I + A)^{-1};
        // T^T[col][row] = inverse * beta_col
        const int wy = y + 1;
        if (decltype(solve)::value && wy >= 0 && wy < nch) {
            const float* Arow = a_s(wy) + l16 * AP;
            float av[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4 v4 = *reinterpret_cast<const floatx4*>(Arow + 4 * q4);
#pragma unroll
                for (int e = 0; e < 4; ++e) av[4 * q4 + e] = v4[e];
            }
            const int ca = 8 * pw + g, cb = ca + 4;
            float xa = (l16 == ca) ? 1.f : 0.f, xb = (l16 == cb) ? 1.f : 0.f;   // av = -A
            row_bcast_fmac_x2<0>(xa, xb, av[0]);
            row_bcast_fmac_x2<1>(xa, xb, av[1]);
            row_bcast_fmac_x2<2>(xa, xb, av[2]);
            row_bcast_fmac_x2<3>(xa, xb, av[3]);
            row_bcast_fmac_x2<4>(xa, xb, av[4]);
            row_bcast_fmac_x2<5>(xa, xb, av[5]);
            row_bcast_fmac_x2<6>(xa, xb, av[6]);
            row_bcast_fmac_x2<7>(xa, xb, av[7]);
            row_bcast_fmac_x2<8>(xa, xb, av[8]);
            row_bcast_fmac_x2<9>(xa, xb, av[9]);
            row_bcast_fmac_x2<10>(xa, xb, av[10]);
            row_bcast_fmac_x2<11>(xa, xb, av[11]);
            row_bcast_fmac_x2<12>(xa, xb, av[12]);
            row_bcast_fmac_x2<13>(xa, xb, av[13]);
            row_bcast_fmac_x2<14>(xa, xb, av[14]);
            tt_s(wy)[ca * TP + l16] = (bf16)(xa * beta_s(wy)[ca]);
            tt_s(wy)[cb * TP + l16] = (bf16)(xb * beta_s(wy)[cb]);
        }
        __syncthreads();
    };
    auto prep_loop = [&](auto solve, auto io) {
        for (int y = -3; y < nit - 3; y += 4) {
            prep_iter(std::integral_constant<int, 0>{}, y, solve, io);
            prep_iter(std::integral_constant<int, 1>{}, y + 1, solve, io);
            prep_iter(std::integral_constant<int, 2>{}, y + 2, solve, io);
            prep_iter(std::integral_constant<int, 3>{}, y + 3, solve, io);
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

template <int NSW>
hipError_t launch_rws(const BwdArgs& a, hipStream_t stream) {
    typedef RwsCfg<NSW> K;
    const int split = kHeadDim / K::DV;
    auto kern = bwd_dh_ws_kernel<NSW>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = raise_lds_limit_once((const void*)kern, (int)K::bytes, lds_set);
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.N * a.H;
    if (units == 0) return hipSuccess;
    const int64_t nwg = (units + kXcd - 1) / kXcd * kXcd * split;
    kern<<<dim3((unsigned)nwg), dim3(K::NT), K::bytes, stream>>>(a, split, (int32_t)units);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dh_ws(const BwdArgs& a, int split, hipStream_t stream) {
    // as the forward: all 128 columns per workgroup from 256 chains, else two
    // workgroups of 64 columns per (sequence, head)
    if (split == 0) split = (int64_t)a.N * a.H >= 256 ? 1 : 2;
    return split == 1 ? launch_rws<8>(a, stream) : launch_rws<4>(a, stream);
}

}  // namespace kda
