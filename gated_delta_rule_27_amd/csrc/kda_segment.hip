// kda_segment.hip -- the exclusive scan of KDA context parallelism.
//
// A segment of a sequence maps its incoming state affinely,
// S_out = M S_in + B ("An infra-oriented diagram of Kimi K3", "KDA Context
// Parallelism"; "From GPT-2 to Kimi K3", ch. 6): M (d_k x d_k) is the
// product of the segment's per-chunk transitions and B the state it reaches
// from a zero start; both come from prefill passes (kda_api.cpp).  Given the
// summaries of R consecutive segments, the state entering each one is
//   S_in[0] = h0,   S_in[r + 1] = M_r S_in[r] + B_r,
// a sequential chain of R small fp32 matrix products per head.
//
// Mapping: one workgroup per (head, 16-column slice of the state), 256
// threads; thread t owns row t / 2 and 8 columns of the slice.  The slice
// of the current state sits in LDS (one buffer per parity of r, so a step's
// reads and the next step's writes never meet); M_r rows stream from global
// memory (all slices of a head read the same M_r, from L2).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kScanCols = 16;          // state columns per workgroup
constexpr int kScanPad = kScanCols + 4;

__global__ __launch_bounds__(256) void segment_scan_kernel(const float* __restrict__ M,
                                                           const float* __restrict__ B,
                                                           const float* __restrict__ h0,
                                                           int32_t R, int32_t H,
                                                           float* __restrict__ S_in,
                                                           float* __restrict__ S_final) {
    constexpr int kState = kHeadDim * kHeadDim;
    const int h = blockIdx.x;
    const int col0 = blockIdx.y * kScanCols;
    const int t = threadIdx.x;
    const int i = t >> 1;               // row (key channel)
    const int c8 = (t & 1) * 8;         // first of this thread's 8 columns in the slice
    const size_t head = (size_t)h * kState;
    const size_t step = (size_t)H * kState;

    __shared__ float Ss[2][kHeadDim][kScanPad];

    float cur[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        cur[e] = h0 ? h0[head + (size_t)i * kHeadDim + col0 + c8 + e] : 0.f;

    for (int r = 0; r < R; ++r) {
        const int par = r & 1;
        float* out = S_in + (size_t)r * step + head + (size_t)i * kHeadDim + col0 + c8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            out[e] = cur[e];
            Ss[par][i][c8 + e] = cur[e];
        }
        __syncthreads();
        const float* Mr = M + (size_t)r * step + head + (size_t)i * kHeadDim;
        const float* Br = B + (size_t)r * step + head + (size_t)i * kHeadDim + col0 + c8;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = Br[e];
        for (int kk = 0; kk < kHeadDim; kk += 4) {
            const floatx4 m = *reinterpret_cast<const floatx4*>(Mr + kk);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += m[u] * Ss[par][kk + u][c8 + e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) cur[e] = acc[e];
    }
    if (S_final) {
#pragma unroll
        for (int e = 0; e < 8; ++e) S_final[head + (size_t)i * kHeadDim + col0 + c8 + e] = cur[e];
    }
}

}  // namespace

hipError_t launch_segment_scan(const float* M, const float* B, const float* h0, int32_t R,
                               int32_t H, float* S_in, float* S_final, hipStream_t stream) {
    if (H == 0) return hipSuccess;
    segment_scan_kernel<<<dim3((unsigned)H, kHeadDim / kScanCols), dim3(256), 0, stream>>>(
        M, B, h0, R, H, S_in, S_final);
    return hipGetLastError();
}

}  // namespace kda
