// kda_decode.hip -- single-token KDA step for a batch of cached states.
//
// The fused recurrent decode path ("From GPT-2 to Kimi K3, from first
// principles", ch. 6 "Training, prefill, and decode use different paths"):
// for every (sequence, head) state S (128 x 128 fp32, row = key channel)
//
//     S'  = Diag(alpha) S,           alpha = exp(log_alpha)
//     p   = S'^T k,  r = S'^T q      (one pass over S', reductions over rows)
//     u   = beta (v - p)
//     S  <- S' + k u^T               (= (I - beta k k^T) S' + beta k v^T)
//     o   = S^T q = r + u (k . q)
//
// which is the KDA equation ("Kimi K3 Architecture Explained", Step 3) with
// the read after the update.  The step is pure HBM streaming: 64 KiB of
// state in and 64 KiB out per (sequence, head), 0.87 flop per byte.
//
// Mapping: a workgroup of 256 * NS threads owns NS adjacent states, i.e. a
// contiguous block of 128 * NS rows of 512 bytes.  Thread t owns columns
// 4 (t % 32) .. +3 of rows  t / 32 + 8 NS m  (m = 0 .. 15) of that block, so
// each of its 16 loads and stores is one 16-byte piece of a workgroup-wide
// access covering 4 NS KiB of consecutive memory; on MI355X that streams
// faster than splitting the workgroup's accesses over its states.  Load m
// falls in state m / (16 / NS) of the block.  The 64 floats stay in
// registers between the read and the write; the column sums over the 128
// rows of a state reduce across the two row groups of a wavefront
// (lane ^ 32), then across the wavefronts through LDS, where one thread per
// (state, sum, column) adds the per-wavefront partials.  The state is touched
// exactly once, so its loads and stores are non-temporal.
//
// The multi-token step (kda_decode_multi) is in kda_decode_multi.hip: this
// unit is built with LLVM's iterative ILP machine scheduler (set in
// build.py), which on MI355X streams the 256 x 96-state step 2.4% faster,
// while it slows the multi-token kernel (one wavefront fewer per SIMD).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kStateLoads = 16;     // 16-byte state pieces per thread
constexpr int kDecodeStates = 2;    // states per workgroup used by launch_decode

template <typename TIn, int NS>
__global__ __launch_bounds__(256 * NS) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ log_alpha, const TIn* __restrict__ beta,
    float* __restrict__ S, TIn* __restrict__ o, int32_t units) {
    constexpr int kWaves = 4 * NS;
    constexpr int kRowStep = 8 * NS;                 // rows per workgroup-wide access
    constexpr int kLoadsPerState = kStateLoads / NS;
    static_assert(kRowStep * kLoadsPerState == kHeadDim, "a state is 128 rows");

    const int t = threadIdx.x;
    const int cg = t & 31;
    const int rg = t >> 5;
    const int first = NS * blockIdx.x;               // first (b * H + h) of the block
    const int nvalid = min(NS, units - first);       // the last block may hold fewer

    __shared__ float sk[NS][kHeadDim], sq[NS][kHeadDim], sa[NS][kHeadDim], sv[NS][kHeadDim];
    __shared__ float su[NS][kHeadDim];
    __shared__ float skq[NS][2];
    __shared__ floatx4 sred[kWaves][NS][2][kHeadDim / 4];

    // 1. issue the per-token vectors first, so that waiting for them does not
    //    wait for the state loads behind them: thread t serves state t / 256;
    //    its first 128 threads take k, q, log alpha, the other 128 take v,
    //    q, log alpha.  The stage is branch-free so that no load sinks below
    //    the state loads (equal values stored twice are harmless).
    const int ms = t >> 8;
    const int j = t & 255;
    const int jc = j & (kHeadDim - 1);
    const bool kside = j < kHeadDim;
    const int unit_v = first + min(ms, nvalid - 1);  // clamped to a valid state
    const size_t vo = (size_t)unit_v * kHeadDim;
    const TIn r0 = (kside ? k : v)[vo + jc];
    const TIn r1 = q[vo + jc];
    const TIn r2 = log_alpha[vo + jc];
    const TIn rb = beta[unit_v];

    // 2. the state; pieces of states past the end re-read state 0 of the block
    const float* Sb = S + (size_t)first * (kHeadDim * kHeadDim);
    floatx4 st[kStateLoads];
#pragma unroll
    for (int m = 0; m < kStateLoads; ++m) {
        const int s = m / kLoadsPerState;
        const int row = rg + kRowStep * m;
        const int src = s < nvalid ? row : (row & (kHeadDim - 1));
        st[m] = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(Sb + src * kHeadDim + 4 * cg));
    }

    const float x0 = to_f32(r0), x1 = to_f32(r1), b = to_f32(rb);
    (kside ? sk[ms] : sv[ms])[jc] = x0;
    sq[ms][jc] = x1;
    sa[ms][jc] = expf(to_f32(r2));
    const float kq_part = wave_sum(x0 * x1);
    if (kside && (j & 63) == 0) skq[ms][j >> 6] = kq_part;
    __syncthreads();

    // 3. retain (scale rows), then partial recall p = S'^T k and read r = S'^T q
    floatx4 p[NS], r[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) p[s] = r[s] = zero4();
#pragma unroll
    for (int m = 0; m < kStateLoads; ++m) {
        const int s = m / kLoadsPerState;
        const int i = (rg + kRowStep * m) & (kHeadDim - 1);
        st[m] *= sa[s][i];
        p[s] += sk[s][i] * st[m];
        r[s] += sq[s][i] * st[m];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            p[s][c] += __shfl_xor(p[s][c], 32, 64);
            r[s][c] += __shfl_xor(r[s][c], 32, 64);
        }
    }
    if ((t & 32) == 0) {
        const int w = t >> 6;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            sred[w][s][0][cg] = p[s];
            sred[w][s][1][cg] = r[s];
        }
    }
    __syncthreads();

    // 4. column sums: thread t -> state t / 256, sum (t / 128) % 2, column t % 128;
    //    the recall sums give u = beta (v - p)
    const int pr = (t >> 7) & 1;
    const int col = t & (kHeadDim - 1);
    const float* red = reinterpret_cast<const float*>(&sred[0][0][0][0]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) acc += red[((w * NS + ms) * 2 + pr) * kHeadDim + col];
    if (pr == 0) su[ms][col] = b * (sv[ms][col] - acc);
    __syncthreads();

    // 5. read-out o = r + u (k . q) by the read-sum threads
    if (pr == 1 && ms < nvalid) {
        const float kq = skq[ms][0] + skq[ms][1];
        o[vo + col] = from_f32<TIn>(acc + su[ms][col] * kq);
    }

    // 6. erase + write: S = S' + k u^T, streamed back out
    floatx4 uu[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) uu[s] = *reinterpret_cast<const floatx4*>(&su[s][4 * cg]);
    float* Sw = S + (size_t)first * (kHeadDim * kHeadDim);
#pragma unroll
    for (int m = 0; m < kStateLoads; ++m) {
        const int s = m / kLoadsPerState;
        const int row = rg + kRowStep * m;
        const int i = row & (kHeadDim - 1);
        if (s < nvalid)
            __builtin_nontemporal_store(st[m] + sk[s][i] * uu[s],
                                        reinterpret_cast<floatx4*>(Sw + row * kHeadDim + 4 * cg));
    }
}

template <int NS>
void launch_decode_ns(const DecodeArgs& a, int dtype, int32_t units, hipStream_t stream) {
    const dim3 grid((unsigned)((units + NS - 1) / NS)), block(256 * NS);
    if (dtype == 0) {
        decode_kernel<float, NS><<<grid, block, 0, stream>>>(
            (const float*)a.q, (const float*)a.k, (const float*)a.v,
            (const float*)a.log_alpha, (const float*)a.beta, a.S, (float*)a.o, units);
    } else {
        decode_kernel<bf16, NS><<<grid, block, 0, stream>>>(
            (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
            (const bf16*)a.log_alpha, (const bf16*)a.beta, a.S, (bf16*)a.o, units);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const int64_t units = (int64_t)a.B * a.H;
    if (units == 0) return hipSuccess;
    launch_decode_ns<kDecodeStates>(a, dtype, (int32_t)units, stream);
    return hipGetLastError();
}

}  // namespace kda
