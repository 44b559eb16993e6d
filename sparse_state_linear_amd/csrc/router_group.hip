// router_group.hip -- router softmax + top-k and the varlen grouping of
// records into (sequence, head, partition) segments, for gfx950.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. (9)-(10) (router) and §2.6 (varlen grouping: records gathered per
// sample and partition, time order kept, new segment offsets).
//
// Grouping is a stable counting sort done in three launches:
//   route_count  one block per (sequence*head, 256-token block): routes its
//                tokens, counts records per partition in LDS, and stores the
//                log2 normaliser of each token's key softmax (§2.3, eq. 11)
//                so that later passes need no row reduction;
//   block_scan   one block per (sequence, head): exclusive scan over its
//                N x blocks counts.  The records of (s, h) occupy a known
//                contiguous range (every token contributes exactly k
//                records), so no scan across (s, h) is needed;
//   scatter      one block per (sequence*head, token block): ranks each
//                record inside its block with wave ballots and writes it.
#include "sse_launch.h"

namespace sse {

constexpr int kTokBlock = 256;  // tokens per grouping block (one per thread)

// Router for one row of N logits: top-k by logit (descending, equal logits ->
// lower index) and the softmax probability of each chosen partition.
template <int NMAX, typename TIn>
__device__ __forceinline__ void route_row(const TIn* __restrict__ row, int N, int K,
                                          int (&sel)[kMaxTopK], float (&w)[kMaxTopK]) {
    float z[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; i++) z[i] = (i < N) ? to_f32(row[i]) : -INFINITY;
    float m = z[0];
#pragma unroll
    for (int i = 1; i < NMAX; i++) m = fmaxf(m, z[i]);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; i++)
        if (i < N) s += expf(z[i] - m);
    uint64_t taken = 0;
#pragma unroll
    for (int r = 0; r < kMaxTopK; r++) {
        if (r < K) {
            int best = -1;
            float bv = -INFINITY;
#pragma unroll
            for (int i = 0; i < NMAX; i++) {
                bool ok = (i < N) && !((taken >> i) & 1ull);
                if (ok && (best < 0 || z[i] > bv)) {
                    best = i;
                    bv = z[i];
                }
            }
            taken |= 1ull << best;
            sel[r] = best;
            w[r] = expf(bv - m) / s;
        }
    }
}

// One thread per row; rows = tokens x heads.
template <int NMAX, typename TIn>
__global__ __launch_bounds__(256) void router_rows_kernel(const TIn* __restrict__ z, int64_t rows,
                                                          int N, int K, int32_t* __restrict__ idx,
                                                          float* __restrict__ wout) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    int sel[kMaxTopK];
    float w[kMaxTopK];
    route_row<NMAX, TIn>(z + r * N, N, K, sel, w);
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++)
        if (j < K) {
            idx[r * K + j] = sel[j];
            wout[r * K + j] = w[j];
        }
}

// Loads CK consecutive input values of one row as fp32.
template <int CK>
__device__ __forceinline__ void load_row(const bf16_t* p, float (&x)[CK]) {
#pragma unroll
    for (int u = 0; u < CK / 8; u++) {
        const uint4 v = reinterpret_cast<const uint4*>(p)[u];
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            x[8 * u + 2 * e] = __uint_as_float(w4[e] << 16);
            x[8 * u + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
        }
    }
}
template <int CK>
__device__ __forceinline__ void load_row(const float* p, float (&x)[CK]) {
#pragma unroll
    for (int u = 0; u < CK / 4; u++) {
        const float4 v = reinterpret_cast<const float4*>(p)[u];
        x[4 * u] = v.x;
        x[4 * u + 1] = v.y;
        x[4 * u + 2] = v.z;
        x[4 * u + 3] = v.w;
    }
}

// Route the tokens of one (sequence, head, token block), count the records
// per partition, and store lnz2 = log2 of the key-softmax denominator
// sum_j 2^((kl_j - m) log2 e) plus m log2 e, so that kappa_j =
// 2^(kl_j log2 e - lnz2).  Blocks of one token block are adjacent in launch
// order across heads (they read neighbouring rows).
template <int NMAX, int CK, typename TIn>
__global__ __launch_bounds__(kTokBlock) void route_count_kernel(
    const TIn* __restrict__ z, const TIn* __restrict__ kl, const int32_t* __restrict__ cu, int H,
    int N, int K, int nblk, int32_t* __restrict__ idx, float* __restrict__ wout,
    int32_t* __restrict__ counts, float* __restrict__ lnz2) {
    __shared__ int cnt[kMaxN];
    const int h = blockIdx.x % H;
    const int rest = blockIdx.x / H;
    const int blk = rest % nblk, s = rest / nblk;
    const int sh = s * H + h;
    const int64_t t1 = cu[s + 1];
    const int64_t tb = cu[s] + (int64_t)blk * kTokBlock;
    if (threadIdx.x < kMaxN) cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t t = tb + threadIdx.x;
    if (t < t1) {
        int sel[kMaxTopK];
        float w[kMaxTopK];
        const int64_t row = t * H + h;
        route_row<NMAX, TIn>(z + row * N, N, K, sel, w);
#pragma unroll
        for (int j = 0; j < kMaxTopK; j++)
            if (j < K) {
                idx[row * K + j] = sel[j];
                wout[row * K + j] = w[j];
                atomicAdd(&cnt[sel[j]], 1);
            }
        if (lnz2) {
            float x[CK];
            load_row<CK>(kl + row * CK, x);
            float m = x[0];
#pragma unroll
            for (int j = 1; j < CK; j++) m = fmaxf(m, x[j]);
            const float m2 = m * kLog2e;
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < CK; j++) sum += exp2f(fmaf(x[j], kLog2e, -m2));
            lnz2[row] = m2 + log2f(sum);
        }
    }
    __syncthreads();
    if (counts && threadIdx.x < N)
        counts[((int64_t)sh * N + threadIdx.x) * nblk + blk] = cnt[threadIdx.x];
}

// Block-wide exclusive scan of one int per thread; returns the prefix and
// sets `total`.  `tmp` holds one int per wave.
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int& total) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
    int inc = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) tmp[wv] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < nw; i++) {
        int v = tmp[i];
        if (i < wv) before += v;
        total += v;
    }
    __syncthreads();
    return before + inc - x;
}

// counts[(sh*N + i)*nblk + blk] -> start position of that block's records of
// partition i (in place); seg_offsets[sh*N + i] = start of segment.
__global__ __launch_bounds__(256) void block_scan_kernel(const int32_t* __restrict__ cu, int H,
                                                         int N, int K, int nblk,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ seg_offsets,
                                                         int num_seqs) {
    __shared__ int tmp[256 / kWave];
    const int sh = blockIdx.x;
    const int s = sh / H, h = sh % H;
    const int64_t len = cu[s + 1] - cu[s];
    int carry = (int)((int64_t)K * ((int64_t)H * cu[s] + h * len));
    const int M = N * nblk;
    int32_t* c = counts + (int64_t)sh * M;
    for (int base = 0; base < M; base += blockDim.x) {
        const int e = base + threadIdx.x;
        const int x = e < M ? c[e] : 0;
        int total;
        const int ex = block_exclusive_scan(x, tmp, total);
        if (e < M) {
            c[e] = carry + ex;
            if (e % nblk == 0) seg_offsets[(int64_t)sh * N + e / nblk] = carry + ex;
        }
        carry += total;
    }
    if (sh == (int)gridDim.x - 1 && threadIdx.x == 0)
        seg_offsets[(int64_t)num_seqs * H * N] = (int32_t)(K * ((int64_t)H * cu[num_seqs]));
}

// Stable scatter of the records of one (sequence, head, token block).
// When lnz2 is given, seg_cr[p] = lnz2[t, h] - log2(w) is stored too: the
// exponent offset that turns 2^(kl log2 e - seg_cr) into w * kappa.
__global__ __launch_bounds__(kTokBlock) void scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ win, const int32_t* __restrict__ cu,
    int H, int N, int K, int nblk, const int32_t* __restrict__ pos, int32_t* __restrict__ seg_tok,
    int32_t* __restrict__ seg_slot, float* __restrict__ seg_w, const float* __restrict__ lnz2,
    float* __restrict__ seg_cr) {
    constexpr int NW = kTokBlock / kWave;
    __shared__ int wcnt[NW][kMaxN];
    const int sh = blockIdx.x, blk = blockIdx.y;
    const int s = sh / H, h = sh % H;
    const int64_t t1 = cu[s + 1];
    const int64_t tb = cu[s] + (int64_t)blk * kTokBlock;
    if (tb >= t1) return;  // whole block past the sequence end (uniform)
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int64_t t = tb + threadIdx.x;
    const bool valid = t < t1;
    int sel[kMaxTopK];
    uint64_t mine = 0;
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        sel[j] = -1;
        if (j < K && valid) {
            sel[j] = idx[(t * H + h) * K + j];
            mine |= 1ull << sel[j];
        }
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    int rank_in_wave[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) rank_in_wave[j] = 0;
    for (int i = 0; i < N; i++) {
        const uint64_t b = __ballot((mine >> i) & 1ull);
        if (lane == 0) wcnt[wv][i] = __popcll(b);
#pragma unroll
        for (int j = 0; j < kMaxTopK; j++)
            if (sel[j] == i) rank_in_wave[j] = __popcll(b & lt);
    }
    __syncthreads();
    if (!valid) return;
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j < K) {
            const int i = sel[j];
            int before = 0;
            for (int w2 = 0; w2 < wv; w2++) before += wcnt[w2][i];
            const int p = pos[((int64_t)sh * N + i) * nblk + blk] + before + rank_in_wave[j];
            seg_tok[p] = (int32_t)t;
            if (seg_slot) seg_slot[p] = j;
            if (seg_w || seg_cr) {
                const float wj = win[(t * H + h) * K + j];
                if (seg_w) seg_w[p] = wj;
                if (seg_cr) seg_cr[p] = lnz2[t * H + h] - log2f(wj);
            }
        }
    }
}

template <typename TIn>
static hipError_t launch_router_rows_t(const void* z, int64_t rows, int N, int K, int32_t* idx,
                                       float* w, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 255) / 256)), block(256);
    const TIn* zz = static_cast<const TIn*>(z);
    if (N <= 8)
        router_rows_kernel<8, TIn><<<grid, block, 0, st>>>(zz, rows, N, K, idx, w);
    else if (N <= 16)
        router_rows_kernel<16, TIn><<<grid, block, 0, st>>>(zz, rows, N, K, idx, w);
    else if (N <= 32)
        router_rows_kernel<32, TIn><<<grid, block, 0, st>>>(zz, rows, N, K, idx, w);
    else
        router_rows_kernel<64, TIn><<<grid, block, 0, st>>>(zz, rows, N, K, idx, w);
    return hipGetLastError();
}

hipError_t launch_router_rows(const void* z, int dtype, int64_t rows, int N, int K, int32_t* idx,
                              float* w, hipStream_t st) {
    return dtype == kF32 ? launch_router_rows_t<float>(z, rows, N, K, idx, w, st)
                         : launch_router_rows_t<bf16_t>(z, rows, N, K, idx, w, st);
}

int group_nblk(int max_seqlen) { return max_seqlen <= 0 ? 1 : (max_seqlen + kTokBlock - 1) / kTokBlock; }

template <int NMAX, typename TIn>
static void launch_rc_n(dim3 grid, const TIn* z, const TIn* kl, const int32_t* cu, int H, int c,
                        int N, int K, int nblk, int32_t* idx, float* w, int32_t* counts,
                        float* lnz2, hipStream_t st) {
    if (c == 32)
        route_count_kernel<NMAX, 32, TIn><<<grid, kTokBlock, 0, st>>>(z, kl, cu, H, N, K, nblk, idx, w, counts, lnz2);
    else if (c == 64)
        route_count_kernel<NMAX, 64, TIn><<<grid, kTokBlock, 0, st>>>(z, kl, cu, H, N, K, nblk, idx, w, counts, lnz2);
    else
        route_count_kernel<NMAX, 128, TIn><<<grid, kTokBlock, 0, st>>>(z, kl, cu, H, N, K, nblk, idx, w, counts, lnz2);
}

template <typename TIn>
static hipError_t launch_route_count_t(const void* z, const void* kl, const int32_t* cu,
                                       int num_seqs, int max_seqlen, int H, int c, int N, int K,
                                       int32_t* idx, float* w, int32_t* counts, float* lnz2,
                                       hipStream_t st) {
    const int nblk = group_nblk(max_seqlen);
    if ((int64_t)num_seqs * H == 0) return hipSuccess;
    dim3 grid((unsigned)((int64_t)num_seqs * nblk * H));
    const TIn* zz = static_cast<const TIn*>(z);
    const TIn* kk = static_cast<const TIn*>(kl);
    if (N <= 8)
        launch_rc_n<8, TIn>(grid, zz, kk, cu, H, c, N, K, nblk, idx, w, counts, lnz2, st);
    else if (N <= 16)
        launch_rc_n<16, TIn>(grid, zz, kk, cu, H, c, N, K, nblk, idx, w, counts, lnz2, st);
    else if (N <= 32)
        launch_rc_n<32, TIn>(grid, zz, kk, cu, H, c, N, K, nblk, idx, w, counts, lnz2, st);
    else
        launch_rc_n<64, TIn>(grid, zz, kk, cu, H, c, N, K, nblk, idx, w, counts, lnz2, st);
    return hipGetLastError();
}

hipError_t launch_route_count(const void* z, const void* kl, int dtype, const int32_t* cu,
                              int num_seqs, int max_seqlen, int H, int c, int N, int K,
                              int32_t* idx, float* w, int32_t* counts, float* lnz2,
                              hipStream_t st) {
    return dtype == kF32 ? launch_route_count_t<float>(z, kl, cu, num_seqs, max_seqlen, H, c, N,
                                                       K, idx, w, counts, lnz2, st)
                         : launch_route_count_t<bf16_t>(z, kl, cu, num_seqs, max_seqlen, H, c,
                                                        N, K, idx, w, counts, lnz2, st);
}

// Count records per (segment, token block) from an existing top-k choice.
__global__ __launch_bounds__(kTokBlock) void count_kernel(const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cu, int H,
                                                          int N, int K, int nblk,
                                                          int32_t* __restrict__ counts) {
    __shared__ int cnt[kMaxN];
    const int sh = blockIdx.x, blk = blockIdx.y;
    const int s = sh / H, h = sh % H;
    const int64_t t = cu[s] + (int64_t)blk * kTokBlock + threadIdx.x;
    if (threadIdx.x < kMaxN) cnt[threadIdx.x] = 0;
    __syncthreads();
    if (t < cu[s + 1])
        for (int j = 0; j < K; j++) atomicAdd(&cnt[idx[(t * H + h) * K + j]], 1);
    __syncthreads();
    if (threadIdx.x < N) counts[((int64_t)sh * N + threadIdx.x) * nblk + blk] = cnt[threadIdx.x];
}

__global__ void zero_int_kernel(int32_t* p) { *p = 0; }

hipError_t launch_group(const int32_t* idx, const float* w, const int32_t* cu, int num_seqs,
                        int max_seqlen, int H, int N, int K, bool counts_ready, int32_t* counts,
                        int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot, float* seg_w,
                        const float* lnz2, float* seg_cr, hipStream_t st) {
    const int nblk = group_nblk(max_seqlen);
    const unsigned SH = (unsigned)(num_seqs * H);
    if (SH == 0) {
        // no sequences: only the terminal offset exists
        zero_int_kernel<<<1, 1, 0, st>>>(seg_offsets);
        return hipGetLastError();
    }
    if (!counts_ready) {
        count_kernel<<<dim3(SH, nblk), kTokBlock, 0, st>>>(idx, cu, H, N, K, nblk, counts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    block_scan_kernel<<<SH, 256, 0, st>>>(cu, H, N, K, nblk, counts, seg_offsets, num_seqs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scatter_kernel<<<dim3(SH, nblk), kTokBlock, 0, st>>>(idx, w, cu, H, N, K, nblk, counts,
                                                         seg_tok, seg_slot, seg_w, lnz2, seg_cr);
    return hipGetLastError();
}

}  // namespace sse
