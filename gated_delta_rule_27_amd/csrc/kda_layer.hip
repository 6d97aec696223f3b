// kda_layer.hip -- the elementwise prologue and epilogue around the KDA core.
//
// Prologue ("From GPT-2 to Kimi K3", ch. 6, "Where q, k, v, alpha, and beta
// come from"; "An infra-oriented diagram of Kimi K3", Kimi Delta Attention
// card), on the outputs of the input projections:
//   q, k, v   = Swish(depthwise causal conv of width 4 over tokens), q and k
//               then L2-normalised per head;
//   log alpha = -5 sigmoid(a + bias), channel-wise, bounded to (-5, 0);
//   beta      = sigmoid(b), one per head;
// plus the convolution history (last three inputs of each sequence) for the
// next segment or decode step.
// Epilogue ("A third gate: control what leaves the module"; "Inside a KDA
// Layer"): y = RMSNorm_head(o) * w * sigmoid(g).
//
// Both are HBM-bound streams (a few flops per byte).  Mapping of the
// prologue: one wave per (tensor, 512-channel slice of a token row = 4
// heads, block of consecutive tokens).  Lane l holds channels 8 (l % 16) ..
// +7 of head 4 slice + l / 16, so every wave-wide load is 1 KiB contiguous
// (bf16) and all 64 lanes sit at the same token: the sequence bookkeeping of
// a packed batch (where a sequence starts, where it ends) is wave-uniform
// scalar work.  Each lane walks its token block in order, keeping the last
// three inputs in registers (the convolution window), so every input is
// loaded once, plus three rows of history per block.  The L2 norm of a head
// is a 16-lane butterfly.  The epilogue maps one 16-lane group per (token,
// head) row in the same way.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kConvW = 4;            // short-convolution width
constexpr int kHist = kConvW - 1;    // inputs of history per sequence
constexpr int kPU = kPrologueLookahead;   // tokens loaded ahead per lane

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
    const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<floatx4*>(p + 4) = floatx4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)x[e];  // RNE
    *reinterpret_cast<bf16x8*>(p) = a;
}

// 8 consecutive elements as loaded (kept packed until used, so a lane can
// hold many tokens in flight in few registers)
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
    __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <>
struct Raw8<float> {
    floatx4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const floatx4*>(p);
        b = *reinterpret_cast<const floatx4*>(p + 4);
    }
    __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// sigmoid(z) = 1 / (1 + e^-z); saturates cleanly to 0 and 1
__device__ __forceinline__ float sigmoid(float z) {
    return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// sum over the 16 lanes of a lane's row (lanes 16r .. 16r + 15)
__device__ __forceinline__ float row16_sum(float s) {
    s += __shfl_xor(s, 8, 16);
    s += __shfl_xor(s, 4, 16);
    s += __shfl_xor(s, 2, 16);
    s += __shfl_xor(s, 1, 16);
    return s;
}

template <typename TIn>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
    const int HD = a.H * kHeadDim;
    const int nslice = (a.H + 3) / 4;
    const int64_t per_tensor = (int64_t)a.n_tblocks * nslice;

    if (wid >= 4 * per_tensor) {
        // ---- history of empty sequences: carried over (or zero) ----
        const int64_t n = wid - 4 * per_tensor;
        if (n >= a.N || !a.state_out) return;
        const int64_t bos = a.cu_seqlens ? a.cu_seqlens[n] : 0;
        const int64_t eos = a.cu_seqlens ? a.cu_seqlens[n + 1] : a.T_total;
        if (eos != bos) return;
        const size_t base = (size_t)n * 3 * kHist * HD;
        const TIn* si = static_cast<const TIn*>(a.state_in);
        TIn* so = static_cast<TIn*>(a.state_out);
        for (int idx = lane; idx < 3 * kHist * HD; idx += 64)
            so[base + idx] = si ? si[base + idx] : from_f32<TIn>(0.f);
        return;
    }

    const int tensor = (int)(wid / per_tensor);            // 0 q, 1 k, 2 v, 3 decay
    const int64_t rest = wid % per_tensor;
    const int64_t tblock = rest / nslice;
    const int slice = (int)(rest % nslice);
    const int row = lane >> 4;
    const int h = 4 * slice + row;
    const int c8 = 8 * (lane & 15);
    const bool live = h < a.H;
    const int hc = live ? h * kHeadDim + c8 : c8;           // channel offset in a token row

    const int64_t t0 = tblock * a.tb;
    const int64_t t1 = t0 + a.tb < a.T_total ? t0 + a.tb : a.T_total;
    const TIn* x = static_cast<const TIn*>(a.x[tensor]);
    TIn* out = static_cast<TIn*>(a.out[tensor]);

    if (tensor == 3) {
        // ---- log alpha = -5 sigmoid(a + bias); beta = sigmoid(b) ----
        float bias[8];
        {
            const floatx4 b0 = *reinterpret_cast<const floatx4*>(a.a_bias + hc);
            const floatx4 b1 = *reinterpret_cast<const floatx4*>(a.a_bias + hc + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bias[e] = b0[e];
                bias[4 + e] = b1[e];
            }
        }
        const TIn* braw = static_cast<const TIn*>(a.b_raw);
        TIn* beta = static_cast<TIn*>(a.beta);
        const bool blane = live && c8 == 0;
        for (int64_t tb = t0; tb < t1; tb += kPU) {
            Raw8<TIn> xv[kPU];
            float bv[kPU];
#pragma unroll
            for (int u = 0; u < kPU; ++u) {
                const int64_t t = tb + u;
                if (t < t1 && live) xv[u].load(x + (size_t)t * HD + hc);
                bv[u] = (t < t1 && blane) ? to_f32(braw[(size_t)t * a.H + h]) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < kPU; ++u) {
                const int64_t t = tb + u;
                if (t < t1 && live) {
                    float y[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] = -5.f * sigmoid(xv[u][e] + bias[e]);
                    store8(out + (size_t)t * HD + hc, y);
                    if (blane) beta[(size_t)t * a.H + h] = from_f32<TIn>(sigmoid(bv[u]));
                }
            }
        }
        return;
    }

    // ---- q, k, v: convolution window, Swish, L2 norm (q, k) ----
    float w[4][8];  // w[j][e]: tap j multiplies the input 3 - j tokens back
    {
        const float* wp = a.conv_w + ((size_t)tensor * HD + hc) * kConvW;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const floatx4 t = *reinterpret_cast<const floatx4*>(wp + e * kConvW);
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j][e] = t[j];
        }
    }
    const bool norm = tensor < 2;
    const TIn* si = static_cast<const TIn*>(a.state_in);
    TIn* so = static_cast<TIn*>(a.state_out);
    // history entry p (0 = oldest) of sequence n for this lane's channels
    auto hist_off = [&](int64_t n, int p) {
        return (((size_t)n * 3 + tensor) * kHist + p) * HD + hc;
    };

    // the sequence holding token t0 (wave-uniform binary search)
    int64_t n = 0, bos = 0, eos = a.T_total;
    if (a.cu_seqlens) {
        int64_t lo = 0, hi = a.N - 1;   // last n with cu[n] <= t0 and cu[n+1] > t0
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (a.cu_seqlens[mid] <= t0) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        bos = a.cu_seqlens[n];
        eos = a.cu_seqlens[n + 1];
    }
    float win[kHist][8];   // inputs t-3, t-2, t-1
#pragma unroll
    for (int p = 0; p < kHist; ++p) {
        const int64_t tp = t0 - kHist + p;
        if (tp >= bos) {
            if (live) load8(x + (size_t)tp * HD + hc, win[p]);
        } else if (si) {
            if (live) load8(si + hist_off(n, (int)(tp - bos + kHist)), win[p]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[p][e] = 0.f;
        }
    }

    for (int64_t tb = t0; tb < t1; tb += kPU) {
        Raw8<TIn> xv[kPU];
#pragma unroll
        for (int u = 0; u < kPU; ++u)
            if (tb + u < t1 && live) xv[u].load(x + (size_t)(tb + u) * HD + hc);
#pragma unroll
        for (int u = 0; u < kPU; ++u) {
            const int64_t t = tb + u;
            if (t >= t1) break;
            while (t == eos) {   // a new sequence starts here (skipping empty ones)
                ++n;
                bos = eos;
                eos = a.cu_seqlens[n + 1];
#pragma unroll
                for (int p = 0; p < kHist; ++p) {
                    if (si && live) load8(si + hist_off(n, p), win[p]);
                    else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) win[p][e] = 0.f;
                    }
                }
            }
            float y[8], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float c = w[3][e] * xv[u][e] + w[2][e] * win[2][e] + w[1][e] * win[1][e] +
                                w[0][e] * win[0][e];
                y[e] = c * sigmoid(c);
                ss += y[e] * y[e];
                win[0][e] = win[1][e];
                win[1][e] = win[2][e];
                win[2][e] = xv[u][e];
            }
            if (norm) {
                const float r = __builtin_amdgcn_rsqf(row16_sum(ss) + a.l2_eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= r;
            }
            if (live) {
                store8(out + (size_t)t * HD + hc, y);
                if (t == eos - 1 && so) {
#pragma unroll
                    for (int p = 0; p < kHist; ++p) store8(so + hist_off(n, p), win[p]);
                }
            }
        }
    }
}

template <typename TIn>
__global__ __launch_bounds__(256) void epilogue_kernel(EpilogueArgs a) {
    // rows = (token, head) pairs; a wave covers 4 rows per step, kEU steps
    constexpr int kEU = 4;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t rows = a.T_total * a.H;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * (4 * kEU) + (lane >> 4);
    const int c8 = 8 * (lane & 15);
    const TIn* o = static_cast<const TIn*>(a.o);
    const TIn* g = static_cast<const TIn*>(a.g);
    TIn* y = static_cast<TIn*>(a.y);
    float ov[kEU][8], gv[kEU][8];
#pragma unroll
    for (int u = 0; u < kEU; ++u) {
        const int64_t r = r0 + 4 * u;
        if (r < rows) {
            load8(o + (size_t)r * kHeadDim + c8, ov[u]);
            load8(g + (size_t)r * kHeadDim + c8, gv[u]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[u][e] = gv[u][e] = 0.f;
        }
    }
#pragma unroll
    for (int u = 0; u < kEU; ++u) {
        const int64_t r = r0 + 4 * u;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += ov[u][e] * ov[u][e];
        const float inv = __builtin_amdgcn_rsqf(row16_sum(ss) * (1.f / kHeadDim) + a.eps);
        if (r < rows) {
            const int h = (int)(r % a.H);
            const float* wp = a.norm_w + (size_t)h * kHeadDim + c8;
            const floatx4 w0 = *reinterpret_cast<const floatx4*>(wp);
            const floatx4 w1 = *reinterpret_cast<const floatx4*>(wp + 4);
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wt = e < 4 ? w0[e] : w1[e - 4];
                out[e] = ov[u][e] * inv * wt * sigmoid(gv[u][e]);
            }
            store8(y + (size_t)r * kHeadDim + c8, out);
        }
    }
}

template <typename TIn>
hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t stream) {
    const int64_t nslice = (a.H + 3) / 4;
    const int64_t waves = 4 * (int64_t)a.n_tblocks * nslice + (a.state_out ? a.N : 0);
    const int64_t wgs = (waves + 3) / 4;
    if (wgs == 0) return hipSuccess;
    prologue_kernel<TIn><<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_epilogue_t(const EpilogueArgs& a, hipStream_t stream) {
    const int64_t rows = a.T_total * a.H;
    const int64_t wgs = (rows + 63) / 64;   // 4 waves x 16 rows
    if (wgs == 0) return hipSuccess;
    epilogue_kernel<TIn><<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, int dtype, hipStream_t stream) {
    return dtype == 0 ? launch_prologue_t<float>(a, stream) : launch_prologue_t<bf16>(a, stream);
}

hipError_t launch_epilogue(const EpilogueArgs& a, int dtype, hipStream_t stream) {
    return dtype == 0 ? launch_epilogue_t<float>(a, stream) : launch_epilogue_t<bf16>(a, stream);
}

}  // namespace kda
