// sse_device.h -- device helpers shared by the gfx950 kernels of this library:
// input loads, bf16 level splitting, MFMA wrappers, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sse {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---- storage types ---------------------------------------------------------
// bf16 inputs arrive as raw 16-bit patterns.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = (__bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (RNE) packed low/high in one 32-bit word (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Split a pair (a, b) into L packed bf16 terms: level l holds the RNE bf16 of
// what the previous levels left (every subtraction is exact in fp32).
template <int L>
__device__ __forceinline__ void split_pair(float a, float b, uint32_t (&out)[L]) {
#pragma unroll
    for (int l = 0; l < L; l++) {
        const uint32_t p = pack_bf16x2(a, b);
        out[l] = p;
        if (l + 1 < L) {
            a -= bf16_lo_f32(p);
            b -= bf16_hi_f32(p);
        }
    }
}

// Split x into L bf16 terms x ~= t0 + t1 + ... (each term is the RNE bf16 of
// what the previous terms left; every subtraction is exact in fp32).
template <int L>
__device__ __forceinline__ void split_levels(float x, uint16_t (&t)[L]) {
    float r = x;
#pragma unroll
    for (int i = 0; i < L; i++) {
        t[i] = f32_to_bf16_bits(r);
        if (i + 1 < L) r = r - bf16_bits_to_f32(t[i]);
    }
}

// ---- MFMA wrappers (gfx950) --------------------------------------------------
// 32x32x16 bf16 -> fp32: A 32 rows x 16 k, B 16 k x 32 cols.  Lane l supplies
// A[l%32][k-group l/32] and B[k-group l/32][l%32], 8 values each; the output
// tile gives lane l column l%32 and rows 8*(i/4) + 4*(l/32) + i%4, i = 0..15.
__device__ __forceinline__ f32x16 mfma32(const u16x8& a, const u16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16x16x32 bf16 -> fp32: lane l supplies row/column l%16 of k-group l/16; the
// output gives lane l column l%16 and rows 4*(l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4 mfma16(const u16x8& a, const u16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- wave reductions -----------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

// Reduce x over groups of L consecutive lanes (L a power of two <= 64; every
// lane gets its group's result).  A 16-lane group is one DPP row: four row
// rotations, no LDS traffic.
template <int L, typename Op>
__device__ __forceinline__ float row_reduce(float x, Op op) {
    if constexpr (L == 16) {
        x = op(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false)));
        x = op(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false)));
        x = op(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false)));
        x = op(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false)));
        return x;
    } else {
#pragma unroll
        for (int o = L / 2; o >= 1; o >>= 1) x = op(x, __shfl_xor(x, o, kWave));
        return x;
    }
}

}  // namespace sse
