// kda_device.h -- device-side building blocks shared by the KDA kernels
// (gfx950 / CDNA4).  Internal header of libkda.so.
//
// MFMA fragments.  All matrix products use 16x16 output tiles held as four
// fp32 per lane: lane l holds column (l % 16) and rows 4*(l/16) .. +3.
// For a contraction over k, lane group g = l/16 of the A operand (row
// l % 16) and of the B operand (column l % 16) must hold the SAME k indices;
// which ones is free.  This library assigns, per k-block:
//   bf16 16x16x32 : elements 0..3 -> k = kb + 4g + 0..3,
//                   elements 4..7 -> k = kb + 16 + 4g + 0..3;
//   bf16 16x16x16 : elements 0..3 -> k = kb + 4g + 0..3;
//   fp32 16x16x4  : four MFMAs j = 0..3, MFMA j uses k = kb + 4g + j.
// With that choice an fp32 accumulator tile (rows 4g..4g+3 in the lane) is
// directly a B operand over its 16 rows, so products that chain (state ->
// pseudo-values -> new state) never leave registers.  An A operand is read
// from LDS as a row with k contiguous.
//
// Invariant for every kernel of the library: an accumulator chain uses one
// MFMA opcode.  A bf16 16x16x16 product accumulated straight onto the result
// of a 16x16x32 chain (or the reverse) gave run-to-run wrong outputs on
// MI355X; the hazard between different MFMA opcodes writing and reading one
// accumulator was not characterised further.  Where a k = 16 product joins
// a k = 32 chain it is issued as the k = 32 instruction with a zero upper
// half (mma_bf16_k16_as_k32), or it starts a fresh accumulator that is added
// on the VALU; fp32 16x16x4 products likewise keep accumulators of their own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// ---- MFMA wrappers ---------------------------------------------------------

__device__ __forceinline__ floatx4 mma_bf16_k32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mma_bf16_k16(bf16x4 a, bf16x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(shortx4, a), __builtin_bit_cast(shortx4, b), c, 0, 0, 0);
}

// k = 16 in fp32: four 16x16x4 MFMAs, MFMA j on element j of a and b.
__device__ __forceinline__ floatx4 mma_f32_k16(floatx4 a, floatx4 b, floatx4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// A k = 16 bf16 product issued as the k = 32 instruction with the upper half
// of k zero.  Used where the accumulator comes straight from a chain of
// 16x16x32 products: an accumulator chain then stays on one MFMA opcode,
// whose back-to-back dependent accumulation the hardware forwards, instead
// of mixing opcodes on one accumulator, which needs software wait states
// between the two MFMAs.
__device__ __forceinline__ floatx4 mma_bf16_k16_as_k32(bf16x4 a, bf16x4 b, floatx4 c) {
    const bf16 z = (bf16)0.f;
    return mma_bf16_k32(bf16x8{a[0], a[1], a[2], a[3], z, z, z, z},
                        bf16x8{b[0], b[1], b[2], b[3], z, z, z, z}, c);
}

// ---- fragments -------------------------------------------------------------

// bf16 operand over k-block [kb, kb+32) from an LDS row (k contiguous).
__device__ __forceinline__ bf16x8 frag_k32(const bf16* row, int kb, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + kb + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + kb + 16 + 4 * g);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// bf16 operand over k-block [kb, kb+16).
__device__ __forceinline__ bf16x4 frag_k16(const bf16* row, int kb, int g) {
    return *reinterpret_cast<const bf16x4*>(row + kb + 4 * g);
}

// fp32 operand over k-block [kb, kb+16).
__device__ __forceinline__ floatx4 frag_k16(const float* row, int kb, int g) {
    return *reinterpret_cast<const floatx4*>(row + kb + 4 * g);
}

// B operand from accumulator tiles: rows kb..kb+15 (lo) and kb+16..kb+31 (hi).
__device__ __forceinline__ bf16x8 acc_frag_k32(floatx4 lo, floatx4 hi) {
    return bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                  (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}
__device__ __forceinline__ bf16x4 acc_frag_k16(floatx4 t) {
    return bf16x4{(bf16)t[0], (bf16)t[1], (bf16)t[2], (bf16)t[3]};
}

// ---- transposed LDS reads (ds_read_b64_tr_b16) -------------------------------
// In each group of 16 lanes, lane j names 4 consecutive 16-bit elements and
// lane i receives element i % 4 of the pieces named by lanes i / 4, i / 4 + 4,
// i / 4 + 8 and i / 4 + 12 (layout measured on gfx950).  col4 points lane j
// at row j / 4, columns 4 (j % 4) .. +3 of a row-major tile at `base` (row
// stride ld elements), so lane l16 receives rows 0..3 of column l16: four
// consecutive k of one column, the B-operand layout, in one instruction.
// Every lane of the wave must execute it; addresses are 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_col4(const bf16* base, int ld, int l16) {
    typedef short shortx4_t __attribute__((ext_vector_type(4)));
    const bf16* p = base + (l16 >> 2) * ld + 4 * (l16 & 3);
    const shortx4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) shortx4_t*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// ---- DPP lane shifts within a row of 16 lanes --------------------------------
// row_shr:n (lane r reads lane r - n of its row) and row_shl:n (lane r reads
// lane r + n); lanes whose source falls outside the row keep `fill`.
template <int N>
__device__ __forceinline__ float row_shr(float src, float fill) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                           __builtin_bit_cast(int, src), 0x110 + N, 0xF, 0xF,
                                           false));
}
template <int N>
__device__ __forceinline__ float row_shl(float src, float fill) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                           __builtin_bit_cast(int, src), 0x100 + N, 0xF, 0xF,
                                           false));
}

// Lane N of each row of 16 lanes, broadcast to the whole row (row_newbcast).
// Every lane reads a valid source, so no "old" value is passed: the result
// needs no copy of x in its register, and the compiler may fold the
// broadcast into the consuming VALU instruction.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, true));
}

// One step of forward elimination on a column held down a row of 16 lanes:
// x += x[I] * a (the pivot x[I] broadcast from lane I of the row), issued as
// one VALU instruction with the broadcast folded into its first operand.
// The leading two wait states cover the write of x by the previous step.
template <int I>
__device__ __forceinline__ void row_bcast_fmac(float& x, float a) {
    asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
                 : "+v"(x)
                 : "v"(a), "i"(I));
}
// The same pivot applied to a second column y from column x: y += x[I] * a.
template <int I>
__device__ __forceinline__ void row_bcast_fmac2(float& y, float x, float a) {
    asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(y)
                 : "v"(x), "v"(a), "i"(I));
}

// Two independent columns x, y eliminated by the same pivot I (each with its
// own pivot value): x += x[I] * a, y += y[I] * a, so that the two chains
// interleave.  Not volatile: the statement only reads and writes its
// operands, so the compiler may schedule the wave's other work around the
// chain (the register dependencies keep the steps in order, and anything it
// places between two steps only adds wait states).
template <int I>
__device__ __forceinline__ void row_bcast_fmac_x2(float& x, float& y, float a) {
    asm(
        "s_nop 1\n\tv_fmac_f32_dpp %0, %0, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(x), "+v"(y)
        : "v"(a), "i"(I));
}

// Shift with zero fill (lanes whose source is outside the row read 0); the
// compiler fuses these into the consuming add (v_add_f32_dpp).
template <int N>
__device__ __forceinline__ float row_shr0(float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src),
                                                                 0x110 + N, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float row_shl0(float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, src),
                                                                 0x100 + N, 0xF, 0xF, true));
}

// Inclusive prefix sum over the 16 lanes of a row (lane r: x_0 + ... + x_r).
__device__ __forceinline__ float row_prefix_sum(float x) {
    x += row_shr0<1>(x);
    x += row_shr0<2>(x);
    x += row_shr0<4>(x);
    x += row_shr0<8>(x);
    return x;
}
// Exclusive suffix sum over the 16 lanes of a row (lane r: x_{r+1} + ... + x_15).
__device__ __forceinline__ float row_suffix_sum_excl(float x) {
    x += row_shl0<1>(x);
    x += row_shl0<2>(x);
    x += row_shl0<4>(x);
    x += row_shl0<8>(x);
    return row_shl0<1>(x);
}

// Inclusive prefix product over the 16 lanes of a row (lane r: x_0 ... x_r).
__device__ __forceinline__ float row_prefix_prod(float x) {
    x *= row_shr<1>(x, 1.f);
    x *= row_shr<2>(x, 1.f);
    x *= row_shr<4>(x, 1.f);
    x *= row_shr<8>(x, 1.f);
    return x;
}
// Inclusive suffix product over the 16 lanes of a row (lane r: x_r ... x_15).
__device__ __forceinline__ float row_suffix_prod(float x) {
    x *= row_shl<1>(x, 1.f);
    x *= row_shl<2>(x, 1.f);
    x *= row_shl<4>(x, 1.f);
    x *= row_shl<8>(x, 1.f);
    return x;
}

// ---- wavefront reductions ---------------------------------------------------

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---- buffer resources ---------------------------------------------------------
// A raw buffer resource (stride 0) covers `bytes` bytes from `base`; loads at
// byte offsets at or past the end return 0 and stores there are dropped by
// the hardware.  The chunk kernels use one per chunk of tokens, sized to the
// rows of that chunk inside its sequence, so partial and out-of-range chunks
// need neither branches nor 64-bit address arithmetic per element.

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// word 3 of a gfx9-family raw buffer descriptor: 32-bit data format, no swizzle
constexpr int kBufWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, kBufWord3);
}
// the same for a size already known to fit 32 bits (no clamping: cheaper
// scalar code where a resource is made per chunk)
__device__ __forceinline__ rsrc_t make_rsrc_u32(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ bf16 buf_load_bf16(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16, (short)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}
__device__ __forceinline__ bf16x4 buf_load_bf16x4(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_store_bf16(bf16 x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, x), r, (int)off, 0, 0);
}
// bf16 store at voff (per lane) + soff (uniform)
__device__ __forceinline__ void buf_store_bf16(bf16 x, rsrc_t r, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(short, x), r, (int)voff, soff, 0);
}
// four bf16 (8 bytes) at voff (per lane) + soff (uniform)
__device__ __forceinline__ void buf_store_bf16x4(bf16x4 x, rsrc_t r, uint32_t voff, int soff) {
    typedef unsigned int uintx2_t __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uintx2_t, x), r, (int)voff, soff, 0);
}
// 16 bytes at voff (per lane) + soff (uniform)
__device__ __forceinline__ void buf_store_b128(bf16x8 x, rsrc_t r, uint32_t voff, int soff) {
    typedef unsigned int uintx4_t __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4_t, x), r, (int)voff, soff, 0);
}
// fp32 store at voff (per lane) + soff (uniform, e.g. a compile-time constant:
// it travels in the instruction's scalar offset, not in a vector register)
__device__ __forceinline__ void buf_store_f32(float x, rsrc_t r, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, x), r, (int)voff, soff, 0);
}

// ---- a wave's 128 x 16 accumulator tile out to memory, transposed ----------
// Lane (l16, g) of the wave holds rows 16 it + 4 g + e of column l16 (it =
// 0..7, e = 0..3): a 128 x 16 column block of a state in MFMA accumulators.
// Its transpose (16 rows of 128, 4 KB, contiguous in a transposed table
// entry) goes out through a wave-private LDS tile of 16 x kTileTP bf16:
// eight 8-byte LDS writes, four 16-byte LDS reads, four 1-KB stores, so
// every store instruction covers whole cache lines.  r / voff0: the block's
// first byte.  Only this wave touches `tile`; its LDS operations execute in
// order, and the fence keeps the compiler from moving them across.
constexpr int kTileTP = 128 + 8;   // a 128-channel row plus 16 bytes of padding
// The first half of store_tile_t: the transposed tile into LDS only (16 rows
// of kTileTP bf16), for other waves to store after a barrier.
__device__ __forceinline__ void tile_to_lds(const floatx4 (&T)[8], bf16* tile, int lane) {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        *reinterpret_cast<bf16x4*>(tile + l16 * kTileTP + 16 * it + 4 * g) = acc_frag_k16(T[it]);
        __builtin_amdgcn_sched_barrier(0);
    }
}
__device__ __forceinline__ void store_tile_t(const floatx4 (&T)[8], bf16* tile, rsrc_t r,
                                             uint32_t voff0, int lane) {
    const int l16 = lane & 15, g = lane >> 4;
    // (one conversion live at a time: the scheduler may not hoist them all)
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        *reinterpret_cast<bf16x4*>(tile + l16 * kTileTP + 16 * it + 4 * g) = acc_frag_k16(T[it]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // piece 64 s + lane: row 4 s + lane / 16, columns 8 (lane % 16) .. +7;
    // one base address each (re-derived here, not kept live across the
    // caller's loop), the rest immediate offsets
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const bf16* rb = tile + (ln >> 4) * kTileTP + (ln & 15) * 8;
    const uint32_t vb = voff0 + (uint32_t)ln * 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(rb + 4 * s * kTileTP);
        buf_store_b128(v, r, vb, 1024 * s);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// ---- vector global loads of 4 or 8 elements ----------------------------------

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    typedef floatx4 type;
};
template <>
struct Vec16<bf16> {
    static constexpr int N = 8;
    typedef bf16x8 type;
};

}  // namespace kda
