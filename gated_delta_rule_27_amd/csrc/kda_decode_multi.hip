// kda_decode_multi.hip -- up to K recurrent KDA steps per cached state in
// one pass over it (speculative verify and replay); the single-step kernel
// and the recurrence it applies are in kda_decode.hip.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

// Up to K recurrent steps per sequence in one pass over its state: the state
// is read once, stays in registers across the tokens, and is written back
// only when update_state is set (a speculative draft is verified without
// touching the cached state, and the accepted prefix replayed on chip:
// "From GPT-2 to Kimi K3", "Speculative decoding cannot naively roll KDA
// back").  Token t of sequence b is applied only for t < n_b (n_tok[b]
// clamped to [0, K]); later tokens are skipped and write no output.
//
// Mapping: a workgroup of 256 * NS threads owns NS states, four wavefronts
// per state; wavefront w of a state owns value columns 32 w .. 32 w + 31 over
// all 128 rows, lane = (row slice lane / 8: rows 16 (lane / 8) .. +15,
// column group lane % 8: 4 columns).  The column sums p = S'^T k and
// r = S'^T q then stay inside the wavefront (16 rows in registers, then 8
// row slices by lane exchanges), so a token needs no barrier: the per-token
// vectors of up to KB tokens are staged in LDS per block (three barriers
// per block), and each wavefront runs its tokens on its own.
//
// Inside a block the registers hold the state divided by the running decay:
// with A_t = alpha_0 ... alpha_t per key channel (product over the block's
// tokens) and St = Diag(A_{t-1})^{-1} S_{t-1},
//   p = S'^T k = St^T (A_t o k),   r = S'^T q = St^T (A_t o q),
//   St <- St + (k / A_t) u^T,
// and at the end of the block S = Diag(A_last) St.  The per-token retain
// pass over the state (a multiply per element) becomes a scaling of the
// three staged vectors: a quarter of the arithmetic per token (verify of 7
// tokens for 256 x 96 states on MI355X: 0.468 -> 0.452 ms; the per-token
// lane exchanges and staging, not the arithmetic, take most of the rest).
// The library's input contract, log alpha in [-5, 0], keeps A above
// e^-40 over a block of 8 tokens, so 1 / A stays finite in fp32.
template <typename TIn, int NS>
__global__ __launch_bounds__(256 * NS) void decode_multi_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ log_alpha, const TIn* __restrict__ beta,
    float* __restrict__ S, const int32_t* __restrict__ n_tok, TIn* __restrict__ o,
    int32_t units, int32_t H, int32_t K, int32_t update_state) {
    constexpr int KB = 8;   // tokens per block of staged vectors

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int s = w >> 2;                 // state of this wavefront in the block
    const int c0 = 32 * (w & 3) + 4 * (lane & 7);   // this lane's first column
    const int r0 = 16 * (lane >> 3);               // this lane's first row
    const int first = NS * blockIdx.x;
    const int nvalid = min(NS, units - first);

    __shared__ __attribute__((aligned(16))) float sk[KB][NS][kHeadDim];
    __shared__ __attribute__((aligned(16))) float sq[KB][NS][kHeadDim];
    __shared__ __attribute__((aligned(16))) float sa[KB][NS][kHeadDim];
    __shared__ __attribute__((aligned(16))) float sv[KB][NS][kHeadDim];
    __shared__ __attribute__((aligned(16))) float sA[KB][NS][kHeadDim];
    __shared__ float sb[KB][NS], skq[KB][NS];

    // tokens to apply per state of the block; the block loop runs to the
    // largest (uniform over the workgroup), each wavefront to its own
    int tmax = 0, nt = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        int c = 0;
        if (j < nvalid) {
            c = n_tok ? n_tok[(first + j) / H] : K;
            c = c < 0 ? 0 : (c > K ? K : c);
        }
        tmax = max(tmax, c);
        if (j == s) nt = c;
    }
    tmax = __builtin_amdgcn_readfirstlane(tmax);
    nt = __builtin_amdgcn_readfirstlane(nt);

    const int unit = first + min(s, nvalid - 1);   // a valid state for addressing
    const size_t b = (size_t)(unit / H), h = (size_t)(unit % H);
    float* Sw = S + (size_t)unit * (kHeadDim * kHeadDim) + (size_t)r0 * kHeadDim + c0;
    floatx4 st[16];
#pragma unroll
    for (int m = 0; m < 16; ++m)
        st[m] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(Sw + m * kHeadDim));

    // staging: wavefront w takes (state, token) pairs w, w + 4 NS, ... of the
    // block; lane = channels 2 lane, 2 lane + 1
    constexpr int kPairs = KB * NS;
    for (int tb = 0; tb < tmax; tb += KB) {
        __syncthreads();   // the previous block's vectors are no longer read
        for (int pi = w; pi < kPairs; pi += 4 * NS) {
            const int js = pi % NS, jt = pi / NS;
            const int ju = first + min(js, nvalid - 1);
            const int tt = min(tb + jt, K - 1);   // always a valid token row
            const size_t row = ((size_t)(ju / H) * K + tt) * H + (size_t)(ju % H);
            const size_t off = row * kHeadDim + 2 * lane;
            const float k0 = to_f32(k[off]), k1 = to_f32(k[off + 1]);
            const float q0 = to_f32(q[off]), q1 = to_f32(q[off + 1]);
            sk[jt][js][2 * lane] = k0;
            sk[jt][js][2 * lane + 1] = k1;
            sq[jt][js][2 * lane] = q0;
            sq[jt][js][2 * lane + 1] = q1;
            sa[jt][js][2 * lane] = expf(to_f32(log_alpha[off]));
            sa[jt][js][2 * lane + 1] = expf(to_f32(log_alpha[off + 1]));
            sv[jt][js][2 * lane] = to_f32(v[off]);
            sv[jt][js][2 * lane + 1] = to_f32(v[off + 1]);
            const float kq = wave_sum(k0 * q0 + k1 * q1);
            if (lane == 0) {
                skq[jt][js] = kq;
                sb[jt][js] = to_f32(beta[row]);
            }
        }
        __syncthreads();
        // running decay over the block's tokens, one thread per (state,
        // channel): sa <- A o k, sq <- A o q, sk <- k / A, sA <- A
        if (t < NS * kHeadDim) {
            const int js = t / kHeadDim, ch = t % kHeadDim;
            float A = 1.f;
#pragma unroll
            for (int jt = 0; jt < KB; ++jt) {
                A *= sa[jt][js][ch];
                const float kv = sk[jt][js][ch], qv = sq[jt][js][ch];
                sa[jt][js][ch] = A * kv;
                sq[jt][js][ch] = A * qv;
                sk[jt][js][ch] = kv / A;
                sA[jt][js][ch] = A;
            }
        }
        __syncthreads();

        const int nb = min(KB, nt - tb);   // this wavefront's tokens in the block
        for (int i = 0; i < nb; ++i) {
            const int tt = tb + i;
            // recall p = S'^T k and read r = S'^T q on the rescaled state,
            // four rows at a time
            floatx4 p = zero4(), r = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const floatx4 ka = *reinterpret_cast<const floatx4*>(&sa[i][s][r0 + 4 * e]);
                const floatx4 qa = *reinterpret_cast<const floatx4*>(&sq[i][s][r0 + 4 * e]);
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    p += ka[x] * st[4 * e + x];
                    r += qa[x] * st[4 * e + x];
                }
            }
            // over the 8 row slices of the wavefront
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int x = 8; x < 64; x <<= 1) {
                    p[c] += __shfl_xor(p[c], x, 64);
                    r[c] += __shfl_xor(r[c], x, 64);
                }
            }
            // u = beta (v - p); read-out o = r + u (k . q); St += (k / A) u^T
            const floatx4 vv = *reinterpret_cast<const floatx4*>(&sv[i][s][c0]);
            const floatx4 u = sb[i][s] * (vv - p);
            if (lane < 8 && s < nvalid) {
                const floatx4 ov = r + u * skq[i][s];
                TIn* dst = o + ((b * K + tt) * H + h) * kHeadDim + c0;
#pragma unroll
                for (int c = 0; c < 4; ++c) dst[c] = from_f32<TIn>(ov[c]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const floatx4 ki = *reinterpret_cast<const floatx4*>(&sk[i][s][r0 + 4 * e]);
#pragma unroll
                for (int x = 0; x < 4; ++x) st[4 * e + x] += ki[x] * u;
            }
        }
        // back to the state itself: S = Diag(A of the block's last token) St
        if (nb > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const floatx4 al = *reinterpret_cast<const floatx4*>(&sA[nb - 1][s][r0 + 4 * e]);
#pragma unroll
                for (int x = 0; x < 4; ++x) st[4 * e + x] *= al[x];
            }
        }
    }

    if (update_state && s < nvalid && nt > 0) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
            __builtin_nontemporal_store(st[m], reinterpret_cast<floatx4*>(Sw + m * kHeadDim));
    }
}

}  // namespace

hipError_t launch_decode_multi(const DecodeMultiArgs& a, int dtype, hipStream_t stream) {
    const int64_t units = (int64_t)a.B * a.H;
    if (units == 0) return hipSuccess;
    constexpr int NS = 1;   // one state (four wavefronts) per workgroup: three workgroups per CU
    const dim3 grid((unsigned)((units + NS - 1) / NS)), block(256 * NS);
    if (dtype == 0) {
        decode_multi_kernel<float, NS><<<grid, block, 0, stream>>>(
            (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.log_alpha,
            (const float*)a.beta, a.S, a.n_tok, (float*)a.o, (int32_t)units, a.H, a.K,
            a.update_state);
    } else {
        decode_multi_kernel<bf16, NS><<<grid, block, 0, stream>>>(
            (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (const bf16*)a.log_alpha,
            (const bf16*)a.beta, a.S, a.n_tok, (bf16*)a.o, (int32_t)units, a.H, a.K,
            a.update_state);
    }
    return hipGetLastError();
}

}  // namespace kda
