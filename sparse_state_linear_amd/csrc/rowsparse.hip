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
// One wave per row, c <= 128 logits, lane = column (two columns per lane at
// c = 128).  The k-th largest logit is found exactly by a bitwise select on
// order-preserving 32-bit keys, most significant bit first: the threshold
// keeps a bit when at least k keys are at or above it (one ballot per bit).
// Equal logits at the threshold are taken lowest row first (ballot ranks).
#include "sse_launch.h"

namespace sse {

namespace {

// Larger floats map to larger keys (finite values and -inf; -0 and +0 get
// the same key, so they tie like equal values).
__device__ __forceinline__ uint32_t order_key(float x) {
    const uint32_t u = x == 0.f ? 0u : __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

template <int CK, typename TIn>
__global__ __launch_bounds__(kRsWaves * kWave) void rowsparse_mask_kernel(
    const TIn* __restrict__ kl, const TIn* __restrict__ la, int64_t rows, int k, int identity,
    TIn* __restrict__ kl_out, TIn* __restrict__ la_out) {
    constexpr int E = CK > kWave ? CK / kWave : 1;   // columns per lane
    const int lane = threadIdx.x % kWave;
    const int64_t row = (int64_t)blockIdx.x * kRsWaves + threadIdx.x / kWave;
    if (row >= rows) return;  // wave-uniform
    const int64_t base = row * CK;
    TIn x[E], l[E];
    uint32_t key[E];
    bool in[E];
#pragma unroll
    for (int e = 0; e < E; e++) {
        const int col = lane + kWave * e;
        in[e] = col < CK;
        x[e] = in[e] ? kl[base + col] : zero_val<TIn>();
        l[e] = in[e] ? la[base + col] : zero_val<TIn>();
        key[e] = order_key(to_f32(x[e]));
    }
    auto count_at_least = [&](uint32_t t) {
        int n = 0;
#pragma unroll
        for (int e = 0; e < E; e++) n += __popcll(__ballot(in[e] && key[e] >= t));
        return n;
    };
    // largest threshold with at least k keys at or above it = the k-th key
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; bit--) {
        const uint32_t cand = thr | (1u << bit);
        if (count_at_least(cand) >= k) thr = cand;
    }
    int above = 0;
#pragma unroll
    for (int e = 0; e < E; e++) above += __popcll(__ballot(in[e] && key[e] > thr));
    const int need = k - above;   // equal keys to take, lowest rows first
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
    int eq_before = 0;
#pragma unroll
    for (int e = 0; e < E; e++) {
        const uint64_t eq = __ballot(in[e] && key[e] == thr);
        const bool sel = key[e] > thr || (key[e] == thr && eq_before + __popcll(eq & lt) < need);
        eq_before += __popcll(eq);
        if (in[e]) {
            const int col = lane + kWave * e;
            kl_out[base + col] = sel ? x[e] : neg_inf<TIn>();
            la_out[base + col] = (sel || !identity) ? l[e] : zero_val<TIn>();
        }
    }
}

template <typename TIn>
hipError_t launch_mask_t(const void* kl, const void* la, int64_t rows, int c, int k, int identity,
                         void* kl_out, void* la_out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const unsigned grid = (unsigned)((rows + kRsWaves - 1) / kRsWaves);
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
