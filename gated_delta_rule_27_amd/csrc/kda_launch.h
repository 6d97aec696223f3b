// kda_launch.h -- internal interface between the C ABI (kda_api.cpp) and the
// kernel launchers (kda_chunk.hip, kda_decode.hip).  Arguments arrive here
// already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kda {

// Raises a kernel's dynamic LDS limit once per device (64 devices at most
// are remembered; past that the attribute is set on every launch).  The
// attribute belongs to the function, not to stream work, so later launches,
// including launches recorded into a HIP graph, make no attribute calls.
// `done` is one flag word per kernel instantiation.
inline hipError_t raise_lds_limit_once(const void* kern, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

constexpr int kHeadDim = 128;  // d_k = d_v of the K3 KDA head
constexpr int kSnapUnit = 16;  // prefix-snapshot intervals are multiples of this

// Prefix snapshots: the state after every `every_chunks` units of kSnapUnit
// tokens of a sequence, i.e. after j * kSnapUnit * every_chunks tokens (j = 1, 2, ...), goes to
// snap[(base_n + j - 1), h] with base_n = snap_cu[n] (0 without snap_cu);
// indices at or past n_snap are not written.  snap == nullptr disables them.
struct SnapArgs {
    float* snap;              // [n_snap, H, 128, 128] fp32 (bf16 [.., 128 j, 128 i] under kChunkSnapBf16)
    const int32_t* snap_cu;   // device [N + 1], may be null (one sequence)
    int64_t n_snap;
    int32_t every_chunks;     // >= 1
};

// Variants of a prefill pass used for segment summaries (context
// parallelism): the affine map S_out = M S_in + B of a segment is B = the
// final state from a zero start, and M = the final state when V is zero and
// the initial state is the identity (the recurrence acts on each value
// column separately, so columns of the identity evolve into columns of M).
enum ChunkFlags : int32_t {
    kChunkNoOutput = 1,     // o is not written (may be null)
    kChunkVZero = 2,        // V is taken as zero (v may be null)
    kChunkH0Identity = 4,   // the initial state of every sequence is I
    kChunkSnapBf16 = 16,    // snapshots stored as bf16 and transposed: entry element
                            // (i, j) at j * 128 + i, so that the four consecutive rows
                            // of one column an MFMA lane holds go out as one 8-byte
                            // store (the bf16 pipelined kernel only; read by the
                            // backward's per-chunk gradient kernel)
    kChunkDualBM = 32,      // both segment-summary passes in one launch over shared
                            // operands: B (zero start, V) into h_T and M (identity
                            // start, V = 0) into h_T2; no outputs or snapshots (the
                            // bf16 pipelined kernel, split 2 only)
    kChunkSnapSlots = 8,    // snapshot j of sequence n goes to entry chunk_slot(n) + j
                            // (with a snapshot after every chunk: the per-chunk
                            // state store of the backward pass)
};

constexpr int kChunk = 16;  // tokens per chunk of the chunk kernels and the backward pass

// Entry of chunk c of sequence n (first token bos) in a per-chunk table:
// bos / 16 + n + c.  Strictly increasing over (n, c) without a scan over
// the sequence lengths; a table of T / 16 + N + 1 entries holds every chunk.
__host__ __device__ inline int64_t chunk_slot(int64_t bos, int64_t n) { return bos / kChunk + n; }
__host__ __device__ inline int64_t chunk_slots(int64_t T_total, int64_t N) {
    return T_total / kChunk + N + 1;
}

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* log_alpha;
    const void* beta;
    const float* h0;          // may be null (zero state)
    const int32_t* cu_seqlens;  // device, may be null (one sequence)
    int32_t N;
    int64_t T_total;
    int32_t H;
    void* o;
    float* h_T;               // may be null
    SnapArgs snap;            // snap.snap == nullptr: no snapshots
    int32_t flags;            // ChunkFlags
    float* h_T2 = nullptr;    // kChunkDualBM: the M pass's final states
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* log_alpha;
    const void* beta;
    float* S;
    int32_t B;
    int32_t H;
    void* o;
};

struct DecodeMultiArgs {
    const void* q;            // [B, K, H, 128]
    const void* k;
    const void* v;
    const void* log_alpha;
    const void* beta;         // [B, K, H]
    float* S;                 // [B, H, 128, 128]
    const int32_t* n_tok;     // device [B] or null (K for every sequence)
    int32_t B;
    int32_t K;
    int32_t H;
    int32_t update_state;
    void* o;                  // [B, K, H, 128]
};

// dtype: 0 = fp32, 1 = bf16 (kda_dtype values).
// chunk in {16, 32}; split = workgroups per head (value-column slices).
// bf16 with chunk 16 and split 1 or 2 runs the wave-specialised pipelined
// kernel (kda_chunk_ws2.hip), bf16 with chunk 32 and split 2 the pipelined
// 32-token kernel (kda_chunk_ws3.hip); every other combination runs the
// phase-serial kernel (kda_chunk.hip).
// (host-only choices, inline so that the C ABI's validation builds without
// the kernels, e.g. for the host sanitizer tests)
inline bool chunk_config_supported(int dtype, int chunk, int split) {
    (void)dtype;
    return (chunk == 16 || chunk == 32) && (split == 1 || split == 2 || split == 4);
}
inline void chunk_default_config(int dtype, int64_t T_total, int32_t N, int32_t H, int* chunk,
                                 int* split) {
    (void)T_total;
    const int64_t chains = (int64_t)N * H;
    if (dtype == 0) {
        *chunk = 16;
        *split = chains >= 512 ? 1 : (chains >= 256 ? 2 : 4);
    } else {
        *chunk = 16;
        *split = chains >= 256 ? 1 : 2;
    }
}
// the bf16 16-token prefill at split 1 or 2, with snapshots, pass flags and
// (split 2 only, no snapshots) the paired summary passes (kda_chunk_ws2.hip)
bool chunk_ws2_supports(const ChunkArgs& a, int split);
hipError_t launch_chunk_ws2(const ChunkArgs& a, int split, hipStream_t stream);
// its split-2 launch with outputs (kda_chunk_ws2_s2.hip), arguments already checked
hipError_t launch_chunk_ws2_split2(const ChunkArgs& a, hipStream_t stream);
// the same cases with 32-token chunks of two 16-token sub-tiles
// (kda_chunk_ws3.hip)
bool chunk_ws3_supports(const ChunkArgs& a, int split);
hipError_t launch_chunk_ws3(const ChunkArgs& a, int split, hipStream_t stream);
hipError_t launch_chunk(const ChunkArgs& a, int dtype, int chunk, int split,
                        hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, int dtype, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeMultiArgs& a, int dtype, hipStream_t stream);
hipError_t launch_segment_scan(const float* M, const float* B, const float* h0, int32_t R,
                               int32_t H, float* S_in, float* S_final, hipStream_t stream);

// Prologue of a KDA layer: projections in, core inputs out (kda_layer.hip).
struct PrologueArgs {
    const void* x[4];          // x_q, x_k, x_v, decay logits a: [T, H, 128]
    const void* b_raw;         // [T, H]
    const float* conv_w;       // [3 (q, k, v), H, 128, 4]
    const float* a_bias;       // [H, 128]
    const int32_t* cu_seqlens; // device, may be null (one sequence)
    int32_t N;
    int64_t T_total;
    int32_t H;
    const void* state_in;      // [N, 3, 3, H, 128] or null (zero history)
    void* state_out;           // same layout or null
    float l2_eps;
    void* out[4];              // q, k, v, log_alpha: [T, H, 128]
    void* beta;                // [T, H]
    int32_t tb;                // tokens per wave (prologue_tokens_per_wave)
    int32_t n_tblocks;         // ceil(T / tb)
};

// Epilogue: y = RMSNorm_head(o) * w * sigmoid(g).
struct EpilogueArgs {
    const void* o;             // [T, H, 128]
    const void* g;             // [T, H, 128]
    const float* norm_w;       // [H, 128]
    int64_t T_total;
    int32_t H;
    float eps;
    void* y;                   // [T, H, 128]
};

// Backward pass (kda_bwd.hip): all tensors in the forward's layouts.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* log_alpha;
    const void* beta;
    const float* h0;           // may be null
    const int32_t* cu_seqlens; // may be null
    int32_t N;
    int64_t T_total;
    int32_t H;
    const void* dout;          // dLoss / do
    const float* dhT;          // dLoss / dh_T, may be null
    void* dq;
    void* dk;
    void* dv;
    void* dlog_alpha;
    void* dbeta;
    float* dh0;                // may be null
    // per-chunk tables, in the input dtype (bf16 tables for bf16 inputs):
    const void* states;        // [n_slots, H, 128, 128]: state after chunk (slot)
    void* dstates;             // [n_slots, H, 128, 128]: dLoss / d(state after chunk)
    int64_t n_slots;
};

hipError_t launch_bwd(const BwdArgs& a, int dtype, hipStream_t stream);
// its two parts: the reverse recursion (split = workgroups per (sequence,
// head), 0 = by the number of chains; bf16 only, fp32 chooses its own) and
// the per-chunk gradients
hipError_t launch_bwd_rev(const BwdArgs& a, int dtype, int split, hipStream_t stream);
hipError_t launch_bwd_grad(const BwdArgs& a, int dtype, hipStream_t stream);
// Work on a side stream of the current device: bwd_fork makes the side
// stream wait for `stream`'s work so far and returns it (null if it cannot
// be had: then run everything on `stream`); bwd_join makes `stream` wait for
// the side stream's work so far.  A successful fork must be joined, on the
// same host thread, before the next fork on that device.
hipStream_t bwd_fork(hipStream_t stream);
hipError_t bwd_join(hipStream_t stream);
// The current device's address of the library's static scratch array of
// KDA_BWD_NOALLOC_MAX_BYTES (kda_noalloc.hip), looked up once per device.
hipError_t noalloc_scratch(void** ptr);
// the reverse recursion for bf16 inputs, pipelined (kda_bwd_ws.hip)
hipError_t launch_bwd_dh_ws(const BwdArgs& a, int split, hipStream_t stream);

constexpr int kPrologueLookahead = 8;   // tokens the prologue loads ahead per lane

// Tokens per prologue wave: enough waves to cover the chip several times,
// blocks long enough that the three rows of history per block stay a small
// overhead.
inline int32_t prologue_tokens_per_wave(int64_t T_total, int32_t H) {
    const int64_t nslice = (H + 3) / 4;
    int32_t tb = 64;
    while (tb > kPrologueLookahead && 4 * nslice * ((T_total + tb - 1) / tb) < 8192) tb /= 2;
    return tb;
}
// Waves of the prologue's convolution kernel: q, k, v x token blocks x
// two-head slices, plus one per sequence for the history of empty ones.
inline int64_t prologue_conv_waves(int64_t n_tblocks, int32_t H, int64_t n_hist) {
    return 3 * n_tblocks * (int64_t)((H + 1) / 2) + n_hist;
}
// Waves of its gate part: token blocks x four-head slices.
inline int64_t prologue_gate_waves(int64_t n_tblocks, int32_t H) {
    return n_tblocks * (int64_t)((H + 3) / 4);
}
hipError_t launch_prologue(const PrologueArgs& a, int dtype, hipStream_t stream);
hipError_t launch_epilogue(const EpilogueArgs& a, int dtype, hipStream_t stream);

}  // namespace kda
