// chunk_common.h -- pieces shared by the chunked gated-linear-attention
// kernels of this library: modes, input vectors, the element-wise
// preparation layout, bf16 term splitting, LDS helpers, MFMA term sums.
#pragma once

#include <type_traits>

#include "sse_launch.h"

namespace sse {

// Warp-specialised kernel for bf16 inputs (chunk_ws.hip); mode is
// kModeShared or kModeRouted (bf16 piece states come from piece_state.hip).
// Returns hipErrorInvalidValue for another mode or a shape it has no
// instance for.
hipError_t launch_chunk_ws(int mode, const ChunkArgs& a, int c, int d, hipStream_t st);

namespace {

constexpr int kNW = 4;        // waves per block
constexpr int kThreads = kNW * kWave;
constexpr int kPC = 4;        // columns per lane in the preparation layout

// Four consecutive input values of one row.
template <typename TIn>
struct Vec4;
template <>
struct Vec4<bf16_t> {
    uint2 u;
    __device__ __forceinline__ void load(const void* base, uint32_t byte_off) {
        u = *reinterpret_cast<const uint2*>(static_cast<const char*>(base) + byte_off);
    }
    // buffer load: an offset past the resource's size reads zeros
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
        u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
    }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = (e < 2) ? u.x : u.y;
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ uint16_t bits(int e) const {
        const uint32_t w = (e < 2) ? u.x : u.y;
        return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
    }
};
template <>
struct Vec4<float> {
    float4 f;
    __device__ __forceinline__ void load(const void* base, uint32_t byte_off) {
        f = *reinterpret_cast<const float4*>(static_cast<const char*>(base) + byte_off);
    }
    __device__ __forceinline__ float get(int e) const {
        return e == 0 ? f.x : e == 1 ? f.y : e == 2 ? f.z : f.w;
    }
    __device__ __forceinline__ uint16_t bits(int) const { return 0; }
};

// Raw buffer resource over [base, base + bytes): loads at offsets past the
// end return zeros (gfx9 descriptor word 3: 32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Preparation layout: CW columns per wave, NCG groups of 4 columns, NG
// groups of RPG consecutive records.
template <int C, int CKD>
struct Geo {
    static constexpr int CW = CKD / kNW;
    static constexpr int NCG = CW / kPC;
    static constexpr int NG = kWave / NCG;
    static constexpr int RPG = C / NG;
    static_assert(CW % kPC == 0 && RPG >= 1 && C % NG == 0, "unsupported shape");
};

template <int L>
__device__ __forceinline__ void split4(const float (&x)[kPC], uint2 (&out)[L]) {
    uint32_t lo[L], hi[L];
    split_pair<L>(x[0], x[1], lo);
    split_pair<L>(x[2], x[3], hi);
#pragma unroll
    for (int l = 0; l < L; l++) out[l] = make_uint2(lo[l], hi[l]);
}

__device__ __forceinline__ u16x8 lds8(const uint16_t* p) {
    return *reinterpret_cast<const u16x8*>(p);
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16): in each 16-lane group,
// lane i = 4b + k receives element k of the 8 bytes addressed by lanes
// 4e + b of the group, e = 0..3 (layout measured on the hardware).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
__device__ __forceinline__ u16x8 cat_tr(const s16x4& a, const s16x4& b) {
    return __builtin_bit_cast(u16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// sum over term pairs (x, y) with x + y < max(LA, LB) of A_x B_y
template <int LA, int LB>
__device__ __forceinline__ void mma32_terms(const u16x8 (&a)[LA], const u16x8 (&b)[LB], f32x16& c) {
    constexpr int L = LA > LB ? LA : LB;
#pragma unroll
    for (int x = 0; x < LA; x++)
#pragma unroll
        for (int y = 0; y < LB; y++)
            if (x + y < L) c = mfma32(a[x], b[y], c);
}
template <int LA, int LB>
__device__ __forceinline__ void mma16_terms(const u16x8 (&a)[LA], const u16x8 (&b)[LB], f32x4& c) {
    constexpr int L = LA > LB ? LA : LB;
#pragma unroll
    for (int x = 0; x < LA; x++)
#pragma unroll
        for (int y = 0; y < LB; y++)
            if (x + y < L) c = mfma16(a[x], b[y], c);
}

// f(std::integral_constant<int, i>) for i = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Barrier for LDS hazards only: global loads and stores may stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace

}  // namespace sse
