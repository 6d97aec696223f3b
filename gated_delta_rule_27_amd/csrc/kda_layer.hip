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
// Both are HBM-bound streams (a few flops per byte), addressed through
// buffer resources with 32-bit offsets.  Prologue, one launch: gate waves
// (decay and write gates: one wave per 4 heads of a token block, lane = 8
// channels), then convolution waves: one per (tensor q / k / v, 256-channel
// slice of a token row = 2 heads, block of consecutive tokens).  Lane l
// holds channels 4 (l % 32) .. +3 of head 2 slice + l / 32, so every
// wave-wide load is 512 contiguous bytes (bf16) and all 64 lanes sit at the
// same token: the sequence bookkeeping of a packed batch (where a sequence
// starts, where it ends) is wave-uniform scalar work.  Each lane walks its
// token block in order, keeping the last three inputs in registers (the
// convolution window), in runs of 8 tokens whose loads are issued one run
// ahead, so every input is loaded once, plus three rows of history per
// block.  The L2 norm of a head is a DPP row sum plus a 16-lane swizzle.
// Epilogue: persistent waves over batches of 16 (token, head) rows, one
// 16-lane group per row, the next batch's loads in flight.
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

__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = a[e];
}
__device__ __forceinline__ void load4(const bf16* p, float (&x)[4]) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)a[e];
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4]) {
    *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void store4(bf16* p, const float (&x)[4]) {
    bf16x4 a;
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = (bf16)x[e];  // RNE
    *reinterpret_cast<bf16x4*>(p) = a;
}

// 4 consecutive elements as loaded (kept packed until used, so a lane can
// hold many tokens in flight in few registers)
template <typename T>
struct Raw4;
template <>
struct Raw4<bf16> {
    bf16x4 v;
    __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x4*>(p); }
    __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <>
struct Raw4<float> {
    floatx4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const floatx4*>(p); }
    __device__ __forceinline__ float operator[](int e) const { return v[e]; }
};
// tokens of loads in flight per lane of the convolution kernel
template <typename T>
constexpr int conv_lookahead() { return 8; }

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

// sum over the 16 lanes of a lane's row (lanes 16r .. 16r + 15), in every
// lane of the row: a DPP prefix sum, then lane 15 broadcast along the row
__device__ __forceinline__ float row16_sum(float s) {
    s += row_shr0<1>(s);
    s += row_shr0<2>(s);
    s += row_shr0<4>(s);
    s += row_shr0<8>(s);
    return row_bcast<15>(s);
}

// sum over the 32 lanes of a lane's half-wave: the two row sums, exchanged
// between the rows of the half by a swizzle (swap groups of 16 lanes)
__device__ __forceinline__ float row32_sum(float s) {
    s = row16_sum(s);
    return s + __builtin_bit_cast(float,
                                  __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, s), 0x401f));
}

// raw loads and stores of 4 / 8 elements through a buffer resource (32-bit
// offsets; out-of-range loads read 0 and out-of-range stores are dropped)
__device__ __forceinline__ Raw4<bf16> buf_raw4(rsrc_t r, uint32_t off, const bf16*) {
    Raw4<bf16> x;
    x.v = buf_load_bf16x4(r, off);
    return x;
}
__device__ __forceinline__ Raw4<float> buf_raw4(rsrc_t r, uint32_t off, const float*) {
    Raw4<float> x;
    x.v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    return x;
}
__device__ __forceinline__ Raw8<bf16> buf_raw8(rsrc_t r, uint32_t off, const bf16*) {
    Raw8<bf16> x;
    x.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    return x;
}
__device__ __forceinline__ Raw8<float> buf_raw8(rsrc_t r, uint32_t off, const float*) {
    Raw8<float> x;
    x.a = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
    x.b = __builtin_bit_cast(floatx4,
                             __builtin_amdgcn_raw_buffer_load_b128(r, (int)off + 16, 0, 0));
    return x;
}
__device__ __forceinline__ bf16 buf_elem(rsrc_t r, uint32_t off, const bf16*) {
    return buf_load_bf16(r, off);
}
__device__ __forceinline__ float buf_elem(rsrc_t r, uint32_t off, const float*) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
// Every output of these kernels is written once and not read again by
// them, so the stores carry the non-temporal cache policy (the streaming
// hint of gfx950 buffer stores): measured on MI355X, the epilogue of the
// 4096-token, 96-head prefill 55 -> 46 us and the prologue 160 -> 154 us.
constexpr int kStreamStore = 2;
typedef unsigned int uintx2_t __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buf_store_elem(rsrc_t r, uint32_t off, float x, bf16*) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, (bf16)x), r, (int)off, 0,
                                          kStreamStore);
}
__device__ __forceinline__ void buf_store_elem(rsrc_t r, uint32_t off, float x, float*) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, (int)off, 0, kStreamStore);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, const float (&x)[8], bf16*) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];  // RNE
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4_t, v), r, (int)off, 0,
                                           kStreamStore);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, const float (&x)[8], float*) {
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(uintx4_t, floatx4{x[0], x[1], x[2], x[3]}), r, (int)off, 0, kStreamStore);
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(uintx4_t, floatx4{x[4], x[5], x[6], x[7]}), r, (int)off + 16, 0,
        kStreamStore);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, const float (&x)[4], bf16*) {
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];  // RNE
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uintx2_t, v), r, (int)off, 0,
                                          kStreamStore);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, const float (&x)[4], float*) {
    __builtin_amdgcn_raw_buffer_store_b128(
        __builtin_bit_cast(uintx4_t, floatx4{x[0], x[1], x[2], x[3]}), r, (int)off, 0, kStreamStore);
}

// log alpha = -5 sigmoid(a + bias) and beta = sigmoid(b)
template <typename TIn>
__device__ __forceinline__ void prologue_gate(const PrologueArgs& a, int64_t wid, int lane) {
    const int HD = a.H * kHeadDim;
    const int nslice = (a.H + 3) / 4;
    if (wid >= (int64_t)a.n_tblocks * nslice) return;
    const int64_t tblock = wid / nslice;
    const int slice = (int)(wid % nslice);
    const int row = lane >> 4;
    const int h = 4 * slice + row;
    const int c8 = 8 * (lane & 15);
    const bool live = h < a.H;
    const int hc = live ? h * kHeadDim + c8 : c8;           // channel offset in a token row
    const int64_t t0 = tblock * a.tb;
    const int64_t t1 = t0 + a.tb < a.T_total ? t0 + a.tb : a.T_total;
    const TIn* x = static_cast<const TIn*>(a.x[3]);
    TIn* out = static_cast<TIn*>(a.out[3]);
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
    // the block's rows as buffer resources (32-bit offsets; lanes past the
    // last head read 0 and their stores are dropped)
    const uint32_t es = (uint32_t)sizeof(TIn);
    const uint32_t blk_bytes = (uint32_t)((t1 - t0) * HD) * es;
    const rsrc_t xr = make_rsrc_u32(x + (size_t)t0 * HD, blk_bytes);
    const rsrc_t outr = make_rsrc_u32(out + (size_t)t0 * HD, blk_bytes);
    const uint32_t lane_off = live ? (uint32_t)hc * es : 0x80000000u;
    const uint32_t row_b = (uint32_t)HD * es;
    const TIn* braw = static_cast<const TIn*>(a.b_raw);
    TIn* beta = static_cast<TIn*>(a.beta);
    const uint32_t bblk = (uint32_t)((t1 - t0) * a.H) * es;
    const rsrc_t br = make_rsrc_u32(braw + (size_t)t0 * a.H, bblk);
    const rsrc_t bw = make_rsrc_u32(beta + (size_t)t0 * a.H, bblk);
    // one lane per head writes beta; the others point past the end
    const uint32_t blane_off = (live && c8 == 0) ? (uint32_t)h * es : 0x80000000u;
    const uint32_t brow_b = (uint32_t)a.H * es;
    for (int64_t tb = t0; tb < t1; tb += kPU) {
        Raw8<TIn> xv[kPU];
        TIn bv[kPU];
        const uint32_t to = (uint32_t)(tb - t0);
#pragma unroll
        for (int u = 0; u < kPU; ++u) {
            xv[u] = buf_raw8(xr, lane_off + (to + u) * row_b, (const TIn*)nullptr);
            bv[u] = buf_elem(br, blane_off + (to + u) * brow_b, (const TIn*)nullptr);
        }
#pragma unroll
        for (int u = 0; u < kPU; ++u) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = -5.f * sigmoid(xv[u][e] + bias[e]);
            buf_store8(outr, lane_off + (to + u) * row_b, y, (TIn*)nullptr);
            buf_store_elem(bw, blane_off + (to + u) * brow_b, sigmoid(to_f32(bv[u])),
                           (TIn*)nullptr);
            // one token's arithmetic live at a time (the loads stay in flight)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// q, k, v: short convolution, Swish, L2 norm (q, k); conv history
template <typename TIn>
__device__ __forceinline__ void prologue_conv(const PrologueArgs& a, int64_t wid, int lane) {
    constexpr int kLA = conv_lookahead<TIn>();
    const int HD = a.H * kHeadDim;
    const int nslice = (a.H + 1) / 2;
    const int64_t per_tensor = (int64_t)a.n_tblocks * nslice;

    if (wid >= 3 * per_tensor) {
        // ---- history of empty sequences: carried over (or zero) ----
        const int64_t n = wid - 3 * per_tensor;
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

    const int tensor = (int)(wid / per_tensor);            // 0 q, 1 k, 2 v
    const int64_t rest = wid % per_tensor;
    const int64_t tblock = rest / nslice;
    const int slice = (int)(rest % nslice);
    const int h = 2 * slice + (lane >> 5);
    const int c4 = 4 * (lane & 31);
    const bool live = h < a.H;
    const int hc = live ? h * kHeadDim + c4 : c4;           // channel offset in a token row

    const int64_t t0 = tblock * a.tb;
    const int64_t t1 = t0 + a.tb < a.T_total ? t0 + a.tb : a.T_total;
    const TIn* x = static_cast<const TIn*>(a.x[tensor]);
    TIn* out = static_cast<TIn*>(a.out[tensor]);

    float w[4][4];  // w[j][e]: tap j multiplies the input 3 - j tokens back
    {
        const float* wp = a.conv_w + ((size_t)tensor * HD + hc) * kConvW;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
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
    float win[kHist][4];   // inputs t-3, t-2, t-1
#pragma unroll
    for (int p = 0; p < kHist; ++p) {
        const int64_t tp = t0 - kHist + p;
        if (tp >= bos) {
            if (live) load4(x + (size_t)tp * HD + hc, win[p]);
        } else if (si) {
            if (live) load4(si + hist_off(n, (int)(tp - bos + kHist)), win[p]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) win[p][e] = 0.f;
        }
    }

    // the block's rows of x and of the output as buffer resources (32-bit
    // offsets; a lane past the last head gets an offset past the end, so its
    // loads read 0 and its stores are dropped)
    const uint32_t blk_bytes = (uint32_t)((t1 - t0) * HD * (int64_t)sizeof(TIn));
    const rsrc_t xr = make_rsrc_u32(x + (size_t)t0 * HD, blk_bytes);
    const rsrc_t outr = make_rsrc_u32(out + (size_t)t0 * HD, blk_bytes);
    const uint32_t lane_off = live ? (uint32_t)(hc * (int)sizeof(TIn)) : 0x80000000u;
    const uint32_t row_b = (uint32_t)(HD * (int)sizeof(TIn));
    // one token: convolution window, Swish, L2 norm, store
    // (every multiply-add spelled out as one fused operation: the pipelined
    // and the single-token paths must round identically, so that a sequence
    // run in pieces reproduces the whole bit for bit)
    auto token = [&](int64_t t, const Raw4<TIn>& xt) {
        float y[4], ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float c = __builtin_fmaf(
                w[3][e], xt[e],
                __builtin_fmaf(w[2][e], win[2][e],
                               __builtin_fmaf(w[1][e], win[1][e], w[0][e] * win[0][e])));
            y[e] = c * sigmoid(c);
            ss = __builtin_fmaf(y[e], y[e], ss);
            win[0][e] = win[1][e];
            win[1][e] = win[2][e];
            win[2][e] = xt[e];
        }
        if (norm) {
            const float r = __builtin_amdgcn_rsqf(row32_sum(ss) + a.l2_eps);
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] *= r;
        }
        buf_store4(outr, lane_off + (uint32_t)(t - t0) * row_b, y, (TIn*)nullptr);
    };
    auto store_hist = [&]() {
        if (so && live) {
#pragma unroll
            for (int p = 0; p < kHist; ++p) store4(so + hist_off(n, p), win[p]);
        }
    };
    // runs of kLA tokens inside one sequence are software-pipelined: the
    // next run's loads are issued before the current run is computed
    auto run_ok = [&](int64_t tt) { return tt + kLA <= t1 && tt + kLA <= eos; };
    auto load_run = [&](int64_t tt, Raw4<TIn> (&buf)[kLA]) {
        const uint32_t ob = lane_off + (uint32_t)(tt - t0) * row_b;
#pragma unroll
        for (int u = 0; u < kLA; ++u) buf[u] = buf_raw4(xr, ob + u * row_b, (const TIn*)nullptr);
    };
    Raw4<TIn> cur[kLA];
    bool have = false;   // cur holds the run starting at tb (wave-uniform)
    for (int64_t tb = t0; tb < t1;) {
        if (run_ok(tb)) {
            if (!have) load_run(tb, cur);
            const int64_t tn = tb + kLA;
            const bool pre = run_ok(tn);
            Raw4<TIn> nxt[kLA];
            if (pre) load_run(tn, nxt);
            // the tokens in order, one token's arithmetic live at a time
#pragma unroll
            for (int u = 0; u < kLA; ++u) {
                token(tb + u, cur[u]);
                __builtin_amdgcn_sched_barrier(0);
            }
            tb = tn;
            if (tb == eos) store_hist();
            have = pre;
            if (pre) {
#pragma unroll
                for (int u = 0; u < kLA; ++u) cur[u] = nxt[u];
            }
        } else {
            have = false;
            // a sequence boundary or the block's end is near: one token
            while (tb == eos) {   // a new sequence starts here (skipping empty ones)
                ++n;
                bos = eos;
                eos = a.cu_seqlens[n + 1];
#pragma unroll
                for (int p = 0; p < kHist; ++p) {
                    if (si && live) load4(si + hist_off(n, p), win[p]);
                    else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) win[p][e] = 0.f;
                    }
                }
            }
            token(tb, buf_raw4(xr, lane_off + (uint32_t)(tb - t0) * row_b, (const TIn*)nullptr));
            ++tb;
            if (tb == eos) store_hist();
        }
    }
}

// One launch: the gate waves first (fewer and shorter), then the
// convolution waves (q, k, v and the history of empty sequences), so that
// the launch does not end on a tail of gate waves.
template <typename TIn>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a, int64_t gate_waves) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + wave;
    if (wid < gate_waves) prologue_gate<TIn>(a, wid, lane);
    else prologue_conv<TIn>(a, wid - gate_waves, lane);
}

// Epilogue rows per 16-lane group of a wave and batch (rows 4 u + group)
constexpr int kEU = 4;
constexpr int kEpiRows = 4 * kEU;   // rows per wave and batch

template <typename TIn>
__global__ __launch_bounds__(256) void epilogue_kernel(EpilogueArgs a) {
    // rows = (token, head) pairs, in batches of kEpiRows consecutive rows;
    // persistent waves take batches w, w + waves, ... with the next batch's
    // loads in flight while the current one is computed.  A batch's o, g
    // and y are buffer resources (32-bit offsets; rows past the end read 0
    // and drop their stores).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t rows = a.T_total * a.H;
    const int64_t nb = (rows + kEpiRows - 1) / kEpiRows;
    const int64_t nw = (int64_t)gridDim.x * 4;
    int64_t b = (int64_t)blockIdx.x * 4 + wave;
    if (b >= nb) return;
    const uint32_t es = (uint32_t)sizeof(TIn);
    const int grp = lane >> 4, c8 = 8 * (lane & 15);
    const uint32_t lane_off = (uint32_t)(grp * kHeadDim + c8) * es;
    const uint32_t step = 4u * kHeadDim * es;
    const TIn* o = static_cast<const TIn*>(a.o);
    const TIn* g = static_cast<const TIn*>(a.g);
    TIn* y = static_cast<TIn*>(a.y);
    auto rsrcs = [&](int64_t bb, rsrc_t& ro, rsrc_t& rg, rsrc_t& ry) {
        const int64_t r0 = bb * kEpiRows;
        const int64_t n = rows - r0 < kEpiRows ? rows - r0 : kEpiRows;
        const uint32_t nbytes = (uint32_t)n * kHeadDim * es;
        const size_t base = (size_t)r0 * kHeadDim;
        ro = make_rsrc_u32(o + base, nbytes);
        rg = make_rsrc_u32(g + base, nbytes);
        ry = make_rsrc_u32(y + base, nbytes);
    };
    Raw8<TIn> ov[kEU], gv[kEU];
    rsrc_t ro, rg, ry;
    rsrcs(b, ro, rg, ry);
#pragma unroll
    for (int u = 0; u < kEU; ++u) {
        ov[u] = buf_raw8(ro, lane_off + u * step, (const TIn*)nullptr);
        gv[u] = buf_raw8(rg, lane_off + u * step, (const TIn*)nullptr);
    }
    for (; b < nb; b += nw) {
        // the next batch's loads first
        const int64_t bn = b + nw;
        Raw8<TIn> ov2[kEU], gv2[kEU];
        rsrc_t ro2, rg2, ry2;
        if (bn < nb) {
            rsrcs(bn, ro2, rg2, ry2);
#pragma unroll
            for (int u = 0; u < kEU; ++u) {
                ov2[u] = buf_raw8(ro2, lane_off + u * step, (const TIn*)nullptr);
                gv2[u] = buf_raw8(rg2, lane_off + u * step, (const TIn*)nullptr);
            }
        }
        int h = (int)((b * kEpiRows + grp) % a.H);   // head of this lane's first row
#pragma unroll
        for (int u = 0; u < kEU; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += ov[u][e] * ov[u][e];
            const float inv = __builtin_amdgcn_rsqf(row16_sum(ss) * (1.f / kHeadDim) + a.eps);
            const float* wp = a.norm_w + (size_t)h * kHeadDim + c8;
            const floatx4 w0 = *reinterpret_cast<const floatx4*>(wp);
            const floatx4 w1 = *reinterpret_cast<const floatx4*>(wp + 4);
            float out[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float wt = e < 4 ? w0[e] : w1[e - 4];
                out[e] = ov[u][e] * inv * wt * sigmoid(gv[u][e]);
            }
            buf_store8(ry, lane_off + u * step, out, (TIn*)nullptr);
            h += 4;
            while (h >= a.H) h -= a.H;
        }
        if (bn < nb) {
#pragma unroll
            for (int u = 0; u < kEU; ++u) {
                ov[u] = ov2[u];
                gv[u] = gv2[u];
            }
            ro = ro2;
            rg = rg2;
            ry = ry2;
        }
    }
}

template <typename TIn>
hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t stream) {
    const int64_t gw = prologue_gate_waves(a.n_tblocks, a.H);
    const int64_t waves = gw + prologue_conv_waves(a.n_tblocks, a.H, a.state_out ? a.N : 0);
    const int64_t wgs = (waves + 3) / 4;
    if (wgs == 0) return hipSuccess;
    prologue_kernel<TIn><<<dim3((unsigned)wgs), dim3(256), 0, stream>>>(a, gw);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_epilogue_t(const EpilogueArgs& a, hipStream_t stream) {
    const int64_t rows = a.T_total * a.H;
    // persistent: at most 5 workgroups (20 waves) per compute unit
    const int64_t need = (rows + 4 * kEpiRows - 1) / (4 * kEpiRows);
    const int64_t wgs = need < 256 * 5 ? need : 256 * 5;
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
