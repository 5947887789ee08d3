// Shared device helpers for the gfx950 (CDNA4) kernels of libmedusa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace medusa {

typedef uint16_t bf16_t;  // raw bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// Two values packed as one 32-bit word, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ float load(const float* p) { return *p; }
    __device__ static __forceinline__ float to_f32(float v) { return v; }
    __device__ static __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    __device__ static __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
    __device__ static __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Eight consecutive elements of T: the per-lane operand slice of one 32-deep MFMA step
// (16x16x32 bf16, or eight 16x16x4 fp32 instructions).
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    u32x4 v;  // 16 bytes
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float at(int i) const {
        uint32_t w = v[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};
template <> struct Frag<float> {
    u32x4 lo, hi;  // 32 bytes
    __device__ __forceinline__ void load(const float* p) {
        lo = reinterpret_cast<const u32x4*>(p)[0];
        hi = reinterpret_cast<const u32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { lo = u32x4{0u, 0u, 0u, 0u}; hi = lo; }
    __device__ __forceinline__ float at(int i) const { return __uint_as_float(i < 4 ? lo[i] : hi[i - 4]); }
};

// acc[16x16] += A[16 x 32] * B[32 x 16], where lane l supplies row (l % 16) of A and column
// (l % 16) of B at contraction slots 8*(l/16) .. 8*(l/16)+7.  Both operands use the same
// slot -> index map, so any permutation of the contraction index is allowed as long as A
// and B agree.  Result: lane l holds acc[4*(l/16) + r][l % 16], r = 0..3.
__device__ __forceinline__ void mma(floatx4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                  __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(floatx4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.at(i), b.at(i), acc, 0, 0, 0);
}

// ---------------------------------------------------------------- cross-lane helpers
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, kWave); }

// (value, index) ordering used by every top-k / argmax: larger value first, then lower id.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// Reduce (v, i) to the best pair over lanes that differ only in the bits of `mask_bits`
// (e.g. 15 -> the 16 lanes sharing l/16).
template <int kSpan>
__device__ __forceinline__ void reduce_best(float& v, int& i) {
#pragma unroll
    for (int m = 1; m < kSpan; m <<= 1) {
        float ov = shfl_xor_f(v, m);
        int oi = shfl_xor_i(i, m);
        if (better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// ---------------------------------------------------------------- DPP reductions
// Within a row of 16 lanes: quad_perm [1,0,3,2] (lane ^ 1), quad_perm [2,3,0,1] (lane ^ 2),
// row_half_mirror (lane i <- 7-i within 8) and row_mirror (lane i <- 15-i within 16) pair
// every lane with one from the other half at each step, so four steps reduce a row; the
// four row results are then read with readlane.  DPP moves stay in the VALU (no LDS
// crossbar round trip), and the order of the additions / comparisons is fixed.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
    const float ov = dpp_f<CTRL>(v);
    const int oi = dpp_i<CTRL>(i);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Best (value, id) over each row of 16 lanes; every lane of the row gets it.
__device__ __forceinline__ void row_best(float& v, int& i) {
    best_step<kDppXor1>(v, i);
    best_step<kDppXor2>(v, i);
    best_step<kDppHalfMirror>(v, i);
    best_step<kDppMirror>(v, i);
}

// Sum over each row of 16 lanes in a fixed order; every lane of the row gets it.
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return v;
}

// Best (value, id) over the whole wave; every lane gets it.
__device__ __forceinline__ void wave_best(float& v, int& i) {
    row_best(v, i);
    float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
        const int ri = __builtin_amdgcn_readlane(i, 16 * r);
        if (better(rv, ri, bv, bi)) { bv = rv; bi = ri; }
    }
    v = bv;
    i = bi;
}

// Sum over the whole wave in a fixed order; every lane gets it.
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// Blocks are dispatched round robin over the 8 XCDs (block i on XCD i % 8).  Map the
// hardware block id to a logical id so that logical neighbours share an XCD (and its L2).
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    const int full = nblocks & ~7;
    if (bid >= full) return bid;
    const int per = full >> 3;
    return (bid & 7) * per + (bid >> 3);
}

}  // namespace medusa
