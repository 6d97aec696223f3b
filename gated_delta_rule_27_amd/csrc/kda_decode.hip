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
// Mapping: one 256-thread workgroup per state.  Thread (cg, rg) with
// cg = tid % 32, rg = tid / 32 owns columns 4cg .. 4cg+3 of rows rg + 8m
// (m = 0..15): every load and store is a fully coalesced 16-byte access
// (a wavefront covers two whole 512-byte rows per instruction), the 64
// floats stay in registers between the read and the write, and the column
// sums over the 128 rows reduce first across the two row groups of a
// wavefront (lane ^ 32) and then across the four wavefronts through LDS.
// The state is touched exactly once, so its loads and stores are
// non-temporal.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kDecodeThreads = 256;
constexpr int kRowsPerThread = kHeadDim / 8;  // 16

template <typename TIn>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const TIn* __restrict__ log_alpha, const TIn* __restrict__ beta,
    float* __restrict__ S, TIn* __restrict__ o) {
    const int unit = blockIdx.x;  // b * H + h
    const int tid = threadIdx.x;
    const int cg = tid & 31;
    const int rg = tid >> 5;

    __shared__ float sk[kHeadDim], sq[kHeadDim], sa[kHeadDim], sv[kHeadDim];
    __shared__ float sred[4][2][kHeadDim];
    __shared__ float skq[2];

    float* Su = S + (size_t)unit * (kHeadDim * kHeadDim);

    // 1. stream the state in first: it does not depend on the small vectors
    floatx4 st[kRowsPerThread];
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m)
        st[m] = __builtin_nontemporal_load(
            reinterpret_cast<const floatx4*>(Su + (rg + 8 * m) * kHeadDim + 4 * cg));

    // 2. per-token vectors: k, q, alpha = exp(log alpha), v; and k . q
    const size_t vo = (size_t)unit * kHeadDim;
    if (tid < kHeadDim) {
        const float kk = to_f32(k[vo + tid]);
        const float qq = to_f32(q[vo + tid]);
        sk[tid] = kk;
        sq[tid] = qq;
        sa[tid] = expf(to_f32(log_alpha[vo + tid]));
        const float s = wave_sum(kk * qq);
        if ((tid & 63) == 0) skq[tid >> 6] = s;
    } else {
        sv[tid - kHeadDim] = to_f32(v[vo + tid - kHeadDim]);
    }
    const float b = to_f32(beta[unit]);
    __syncthreads();

    // 3. retain (scale rows), then partial recall p = S'^T k and read r = S'^T q
    floatx4 p = zero4(), r = zero4();
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
        const int i = rg + 8 * m;
        st[m] *= sa[i];
        p += sk[i] * st[m];
        r += sq[i] * st[m];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        p[c] += __shfl_xor(p[c], 32, 64);
        r[c] += __shfl_xor(r[c], 32, 64);
    }
    if ((tid & 32) == 0) {
        const int w = tid >> 6;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sred[w][0][4 * cg + c] = p[c];
            sred[w][1][4 * cg + c] = r[c];
        }
    }
    __syncthreads();

    // 4. correction u = beta (v - p) and read-out o = r + u (k . q)
    const float kq = skq[0] + skq[1];
    floatx4 u, oc;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int col = 4 * cg + c;
        const float P = sred[0][0][col] + sred[1][0][col] + sred[2][0][col] + sred[3][0][col];
        const float R = sred[0][1][col] + sred[1][1][col] + sred[2][1][col] + sred[3][1][col];
        u[c] = b * (sv[col] - P);
        oc[c] = R + u[c] * kq;
    }

    // 5. erase + write: S = S' + k u^T, streamed back out
#pragma unroll
    for (int m = 0; m < kRowsPerThread; ++m) {
        const int i = rg + 8 * m;
        const floatx4 nv = st[m] + sk[i] * u;
        __builtin_nontemporal_store(
            nv, reinterpret_cast<floatx4*>(Su + (rg + 8 * m) * kHeadDim + 4 * cg));
    }
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) o[vo + 4 * cg + c] = from_f32<TIn>(oc[c]);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const int64_t units = (int64_t)a.B * a.H;
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)units), block(kDecodeThreads);
    if (dtype == 0) {
        decode_kernel<float><<<grid, block, 0, stream>>>(
            (const float*)a.q, (const float*)a.k, (const float*)a.v,
            (const float*)a.log_alpha, (const float*)a.beta, a.S, (float*)a.o);
    } else {
        decode_kernel<bf16><<<grid, block, 0, stream>>>(
            (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
            (const bf16*)a.log_alpha, (const bf16*)a.beta, a.S, (bf16*)a.o);
    }
    return hipGetLastError();
}

}  // namespace kda
