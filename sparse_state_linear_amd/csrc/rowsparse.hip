// rowsparse.hip -- the row-sparse key variant for gfx950: per (token, head),
// mask the key logits to their k largest entries and the log decay to the
// rows that are written.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.2 eqs. (7)-(8): the key is the softmax over the k largest key logits
// (the others are masked to -inf, so they get an exact zero write), and rows
// that are not written keep their state only if their transition is the
// identity.  With kl' = kl on the selected rows and -inf elsewhere, and
// la' = la on the selected rows and 0 elsewhere (identity form; la' = la in
// the plain form), the layer is a single-state gated linear attention over
// (q, kl', v, la') -- the shared-partition kernels of this library with no
// routed partitions.
//
// A row of c <= 128 logits is spread over c/32 lanes, 32 consecutive
// columns each (16-byte loads and stores).  The k-th largest logit is found
// exactly by a bitwise select on order-preserving keys, most significant
// bit first: the threshold keeps a bit when at least k keys are at or above
// it (each lane counts its own keys, the row's lanes add their counts by
// shuffles).  bf16 logits use 16-bit keys (16 steps), fp32 logits 32-bit
// keys.  Equal logits at the threshold are taken lowest row first.
#include "sse_launch.h"

namespace sse {

namespace {

// Larger values map to larger keys (finite values and -inf; -0 and +0 get
// the same key, so they tie like equal values).  A bf16 value's 16-bit key
// orders bf16 values exactly as the 32-bit key of the same value as fp32.
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key(bf16_t x) {
    const uint32_t u = x.bits == 0x8000u ? 0u : x.bits;
    return (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
}

template <typename TIn>
__device__ __forceinline__ TIn neg_inf();
template <>
__device__ __forceinline__ float neg_inf<float>() { return -INFINITY; }
template <>
__device__ __forceinline__ bf16_t neg_inf<bf16_t>() { return bf16_t{0xff80u}; }
template <typename TIn>
__device__ __forceinline__ TIn zero_val() { return TIn{}; }

constexpr int kRsWaves = 4;
constexpr int kRsCols = 32;   // columns per lane

template <typename T>
struct alignas(16) Vec16 {
    T x[16 / sizeof(T)];
};

// sum of v over the L lanes of this lane's row (L a power of two)
template <int L>
__device__ __forceinline__ int row_sum(int v) {
#pragma unroll
    for (int m = L / 2; m >= 1; m /= 2) v += __shfl_xor(v, m, L);
    return v;
}

// sum of v over the lanes of this lane's row before it
template <int L>
__device__ __forceinline__ int row_prefix(int v) {
    const int sub = (int)(threadIdx.x % L);
    int incl = v;
#pragma unroll
    for (int m = 1; m < L; m *= 2) {
        const int y = __shfl_up(incl, m, L);
        if (sub >= m) incl += y;
    }
    return incl - v;
}

template <int CK, typename TIn>
__global__ __launch_bounds__(kRsWaves * kWave) void rowsparse_mask_kernel(
    const TIn* __restrict__ kl, const TIn* __restrict__ la, int64_t rows, int k, int identity,
    TIn* __restrict__ kl_out, TIn* __restrict__ la_out) {
    static_assert(CK % kRsCols == 0 && CK / kRsCols <= kWave, "unsupported row length");
    constexpr int L = CK / kRsCols;                        // lanes per row
    constexpr int KB = sizeof(TIn) == 2 ? 16 : 32;         // key bits
    constexpr int VEC = 16 / (int)sizeof(TIn);             // values per 16-byte access
    constexpr int NV = kRsCols / VEC;
    using V = Vec16<TIn>;
    const int sub = (int)(threadIdx.x % L);
    const int64_t row = ((int64_t)blockIdx.x * kRsWaves * kWave + threadIdx.x) / L;
    const bool live = row < rows;   // the same for the L lanes of a row
    const int64_t base = (live ? row : 0) * CK + sub * kRsCols;
    V x[NV], l[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
        x[i] = reinterpret_cast<const V*>(kl + base)[i];
        l[i] = reinterpret_cast<const V*>(la + base)[i];
    }
    uint32_t key[kRsCols];
#pragma unroll
    for (int i = 0; i < NV; i++)
#pragma unroll
        for (int j = 0; j < VEC; j++) key[i * VEC + j] = order_key(x[i].x[j]);
    // largest threshold with at least k keys at or above it = the k-th key
    uint32_t thr = 0;
    for (int bit = KB - 1; bit >= 0; bit--) {
        const uint32_t cand = thr | (1u << bit);
        int n = 0;
#pragma unroll
        for (int e = 0; e < kRsCols; e++) n += key[e] >= cand ? 1 : 0;
        if (row_sum<L>(n) >= k) thr = cand;
    }
    int above = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kRsCols; e++) {
        above += key[e] > thr ? 1 : 0;
        eq += key[e] == thr ? 1 : 0;
    }
    // equal keys still to take, lowest rows first: those of earlier lanes
    // of the row come first
    int left = k - row_sum<L>(above) - row_prefix<L>(eq);
#pragma unroll
    for (int i = 0; i < NV; i++) {
#pragma unroll
        for (int j = 0; j < VEC; j++) {
            const uint32_t kk = key[i * VEC + j];
            bool sel = kk > thr;
            if (kk == thr) {
                sel = left > 0;
                left--;
            }
            if (!sel) {
                x[i].x[j] = neg_inf<TIn>();
                if (identity) l[i].x[j] = zero_val<TIn>();
            }
        }
    }
    if (live) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            reinterpret_cast<V*>(kl_out + base)[i] = x[i];
            reinterpret_cast<V*>(la_out + base)[i] = l[i];
        }
    }
}

template <typename TIn>
hipError_t launch_mask_t(const void* kl, const void* la, int64_t rows, int c, int k, int identity,
                         void* kl_out, void* la_out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const int64_t rows_per_block = (int64_t)kRsWaves * kWave / (c / kRsCols);
    const unsigned grid = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
    const TIn* a = static_cast<const TIn*>(kl);
    const TIn* b = static_cast<const TIn*>(la);
    TIn* ao = static_cast<TIn*>(kl_out);
    TIn* bo = static_cast<TIn*>(la_out);
    if (c == 32)
        rowsparse_mask_kernel<32, TIn><<<grid, kRsWaves * kWave, 0, st>>>(a, b, rows, k, identity, ao, bo);
    else if (c == 64)
        rowsparse_mask_kernel<64, TIn><<<grid, kRsWaves * kWave, 0, st>>>(a, b, rows, k, identity, ao, bo);
    else if (c == 128)
        rowsparse_mask_kernel<128, TIn><<<grid, kRsWaves * kWave, 0, st>>>(a, b, rows, k, identity, ao, bo);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rowsparse_mask(const void* kl, const void* la, int dtype, int64_t rows, int c,
                                 int k, int identity, void* kl_out, void* la_out, hipStream_t st) {
    return dtype == kF32 ? launch_mask_t<float>(kl, la, rows, c, k, identity, kl_out, la_out, st)
                         : launch_mask_t<bf16_t>(kl, la, rows, c, k, identity, kl_out, la_out, st);
}

}  // namespace sse
