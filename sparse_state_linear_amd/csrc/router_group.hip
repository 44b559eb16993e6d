// router_group.hip -- router softmax + top-k and the varlen grouping of
// records into (sequence, head, partition) segments, for gfx950.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. (9)-(10) (router) and §2.6 (varlen grouping: records gathered per
// sample and partition, time order kept, new segment offsets).
//
// Grouping is a stable counting sort done in three launches:
//   route_count  one block per (sequence, 64-token block, group of 4
//                heads): routes the block's rows (one lane per row; more
//                blocks with shorter chains measured faster than one block
//                for all heads of a token block), then one wave per head
//                (lane = token) ranks every record among the block's records
//                of its partition with wave ballots (time order kept), writes
//                the per-(head, partition) block counts and a head-major
//                (partition, rank, weight) record per routed token; for fp32
//                inputs it also stores the log2 normaliser of each row's key
//                softmax (section 2.3, eq. 11; 16 lanes per row, coalesced
//                16-byte loads; the first head group's block does all heads)
//                so that later passes need no row reduction;
//   block_scan   one block per (sequence, head): exclusive scan over its
//                N x blocks counts.  The records of (s, h) occupy a known
//                contiguous range (every token contributes exactly k
//                records), so no scan across (s, h) is needed;
//   scatter      one wave per (sequence, head, token block): reads the
//                head-major records (contiguous) and writes each as one
//                16-byte segment record at its block start + rank.
// The standalone grouping entry point (from a given top-k choice) counts
// with LDS atomics and ranks with ballots in its scatter instead.
#include "sse_launch.h"

namespace sse {


// Router for one row of N logits: top-k by logit (descending, equal logits ->
// lower index) and the softmax probability of each chosen partition.
// Loads one row of N router logits as fp32 (-inf past N).
template <int NMAX, typename TIn>
__device__ __forceinline__ void load_router_row(const TIn* __restrict__ row, int N,
                                                float (&z)[NMAX]) {
    constexpr int kVec = 16 / (int)sizeof(TIn);  // values per 16-byte load
    if (N == NMAX && NMAX % kVec == 0) {
        // whole row in 16-byte loads (rows are 16-byte aligned when N is a
        // multiple of kVec)
#pragma unroll
        for (int u = 0; u < NMAX / kVec; u++) {
            const uint4 v = reinterpret_cast<const uint4*>(row)[u];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if constexpr (sizeof(TIn) == 2) {
                    z[kVec * u + 2 * e] = __uint_as_float(w4[e] << 16);
                    z[kVec * u + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
                } else {
                    z[kVec * u + e] = __uint_as_float(w4[e]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NMAX; i++) z[i] = (i < N) ? to_f32(row[i]) : -INFINITY;
    }
}

// Router for one row of N logits (entries past N are -inf): top-k by logit
// (descending, equal logits -> lower index: a strictly greater value is
// needed to replace the current best) and the softmax probability of each
// chosen partition.  Branch-free: every choice is a select.
template <int NMAX>
__device__ __forceinline__ void route_row(const float (&z)[NMAX], int N, int K,
                                          int (&sel)[kMaxTopK], float (&w)[kMaxTopK]) {
    float m = z[0];
#pragma unroll
    for (int i = 1; i < NMAX; i++) m = fmaxf(m, z[i]);
    const float m2 = m * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NMAX; i++) s += __builtin_amdgcn_exp2f(fmaf(z[i], kLog2e, -m2));
    const float inv_s = 1.f / s;
    float zz[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; i++) zz[i] = z[i];
#pragma unroll
    for (int r = 0; r < kMaxTopK; r++) {
        if (r < K) {
            float bv = -INFINITY;
            int best = 0;
#pragma unroll
            for (int i = 0; i < NMAX; i++) {
                const bool gt = zz[i] > bv;
                bv = gt ? zz[i] : bv;
                best = gt ? i : best;
            }
#pragma unroll
            for (int i = 0; i < NMAX; i++) zz[i] = (i == best) ? -INFINITY : zz[i];
            sel[r] = best;
            w[r] = __builtin_amdgcn_exp2f(fmaf(bv, kLog2e, -m2)) * inv_s;
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
    float zr[NMAX];
    load_router_row<NMAX, TIn>(z + r * N, N, zr);
    route_row<NMAX>(zr, N, K, sel, w);
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

// Route the rows of one (sequence, 64-token block) for all heads, in groups
// of kHG heads: phase 1 routes the group's rows (one lane per row; the rows of
// a token block are one contiguous range) into LDS, phase 2 gives each head
// to one wave (lane = token), ranks the records of every partition by ballot
// (stable: lower token first), writes the block counts counts[s, h, i, blk]
// and the head-major records rinfo[(h T + t) K + j] = (i | rank << 16, w).
// With lnz2 given, it also stores lnz2 = log2 of the key-softmax denominator
// sum_j 2^((kl_j - m) log2 e) plus m log2 e, so that kappa_j =
// 2^(kl_j log2 e - lnz2), for the rows of its tokens and heads; the key
// normaliser spreads each row over CK/8 (bf16) or CK/4 (fp32) lanes.
constexpr int kHG = 4;  // heads per block (one wave per head in the ranking phase)
template <int NMAX, int CK, typename TIn>
__global__ __launch_bounds__(256) void route_count_kernel(
    const TIn* __restrict__ z, const TIn* __restrict__ kl, const int32_t* __restrict__ cu,
    int64_t T, int H, int N, int K, int nblk, int32_t* __restrict__ idx, float* __restrict__ wout,
    int32_t* __restrict__ counts, uint2* __restrict__ rinfo, float* __restrict__ lnz2) {
    extern __shared__ float swt[];  // [kHG][kTokBlock][K] weights, then the choices as bytes
    uint8_t* ssel = reinterpret_cast<uint8_t*>(swt + kHG * kTokBlock * K);
    const int blk = blockIdx.x, s = blockIdx.y, hgb = blockIdx.z * kHG;  // this block's heads
    const int64_t t1 = cu[s + 1];
    const int64_t tb = cu[s] + (int64_t)blk * kTokBlock;
    const int ntok = (int)(t1 - tb < 0 ? 0 : (t1 - tb > kTokBlock ? kTokBlock : t1 - tb));
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
    if (ntok == 0) {
        // a block past the end of a shorter sequence: zero counts for its
        // heads (no rows to route or rank, no normalisers)
        const int hgc = H - hgb < kHG ? H - hgb : kHG;
        for (int x = threadIdx.x; x < hgc * N; x += blockDim.x)
            counts[(((int64_t)s * H + hgb + x / N) * N + x % N) * nblk + blk] = 0;
        return;  // uniform
    }
    // rows per thread and batch, loaded before any is routed (one with 256
    // threads for 64 tokens x 4 heads)
    constexpr int kRB = (kTokBlock * kHG + 255) / 256;
    for (int hg0 = hgb; hg0 < hgb + kHG && hg0 < H; hg0 += kHG) {
        const int hgc = H - hg0 < kHG ? H - hg0 : kHG;
        const int rows = ntok * hgc;
        for (int rb = threadIdx.x; rb < rows; rb += kRB * (int)blockDim.x) {
            float zr[kRB][NMAX];
#pragma unroll
            for (int b = 0; b < kRB; b++) {
                const int rl = rb + b * (int)blockDim.x;
                const int rr = rl < rows ? rl : rb;
                const int64_t row = (tb + rr / hgc) * H + hg0 + rr % hgc;
                load_router_row<NMAX, TIn>(z + row * N, N, zr[b]);
            }
#pragma unroll
            for (int b = 0; b < kRB; b++) {
                const int rl = rb + b * (int)blockDim.x;
                if (rl >= rows) break;
                const int tl = rl / hgc, hi = rl % hgc;
                const int64_t row = (tb + tl) * H + hg0 + hi;
                int sel[kMaxTopK];
                float w[kMaxTopK];
                route_row<NMAX>(zr[b], N, K, sel, w);
#pragma unroll
                for (int j = 0; j < kMaxTopK; j++)
                    if (j < K) {
                        idx[row * K + j] = sel[j];
                        wout[row * K + j] = w[j];
                        swt[(hi * kTokBlock + tl) * K + j] = w[j];
                        ssel[(hi * kTokBlock + tl) * K + j] = (uint8_t)sel[j];
                    }
            }
        }
        __syncthreads();
        const bool valid = lane < ntok;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
        for (int hi = wv; hi < hgc; hi += nw) {
            const int h = hg0 + hi;
            int sel[kMaxTopK], rank[kMaxTopK];
            uint64_t mine = 0;
#pragma unroll
            for (int j = 0; j < kMaxTopK; j++) {
                sel[j] = -1;
                rank[j] = 0;
                if (j < K && valid) {
                    sel[j] = ssel[(hi * kTokBlock + lane) * K + j];
                    mine |= 1ull << sel[j];
                }
            }
            int mycount = 0;
            for (int i = 0; i < N; i++) {
                const uint64_t bal = __ballot((mine >> i) & 1ull);
#pragma unroll
                for (int j = 0; j < kMaxTopK; j++)
                    if (sel[j] == i) rank[j] = __popcll(bal & lt);
                if (lane == i) mycount = __popcll(bal);
            }
            if (lane < N) counts[(((int64_t)s * H + h) * N + lane) * nblk + blk] = mycount;
            if (valid)
#pragma unroll
                for (int j = 0; j < kMaxTopK; j++)
                    if (j < K)
                        rinfo[((int64_t)h * T + tb + lane) * K + j] =
                            make_uint2((uint32_t)sel[j] | ((uint32_t)rank[j] << 16),
                                       __float_as_uint(swt[(hi * kTokBlock + lane) * K + j]));
        }
        __syncthreads();
    }
    if (lnz2) {  // the normalisers of this block's rows (its heads' rows of its tokens)
        const int hgc = H - hgb < kHG ? H - hgb : kHG;
        const int nrows = ntok * hgc;                // row rl: token rl / hgc, head hgb + rl % hgc
        auto row_of = [&](int rl) { return (tb + rl / hgc) * H + hgb + rl % hgc; };
        constexpr int VPL = 16 / (int)sizeof(TIn);  // values per lane
        constexpr int LPR = CK / VPL;                // lanes per row
        constexpr int RPW = kWave / LPR;             // rows per wave and pass
        const int sub = lane % LPR, rr = lane / LPR;
        // kB passes per batch: all their loads are issued before any of
        // them is reduced, so the batch waits for memory once
        constexpr int kB = 8;
        const int step = nw * RPW;
        for (int rb0 = wv * RPW; rb0 < nrows; rb0 += kB * step) {
        uint4 vb[kB];
#pragma unroll
        for (int b = 0; b < kB; b++) {
            const int rl = rb0 + b * step + rr;
            vb[b] = reinterpret_cast<const uint4*>(kl + row_of(rl < nrows ? rl : 0) * CK)[sub];
        }
#pragma unroll
        for (int b = 0; b < kB; b++) {
            const int rl = rb0 + b * step + rr;
            const bool ok = rl < nrows;
            const int64_t r = row_of(ok ? rl : 0);
            const uint4 v = vb[b];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            float x[VPL];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if constexpr (sizeof(TIn) == 2) {
                    x[2 * e] = __uint_as_float(w4[e] << 16);
                    x[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
                } else {
                    x[e] = __uint_as_float(w4[e]);
                }
            }
            float m = x[0];
#pragma unroll
            for (int j = 1; j < VPL; j++) m = fmaxf(m, x[j]);
            m = row_reduce<LPR>(m, [](float u, float v) { return fmaxf(u, v); });
            const float m2 = m * kLog2e;
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < VPL; j++) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -m2));
            sum = row_reduce<LPR>(sum, [](float u, float v) { return u + v; });
            if (ok && sub == 0) lnz2[r] = m2 + log2f(sum);
        }
        }
    }
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
// partition i (in place); seg_offsets[sh*N + i] = start of segment.  Each
// thread scans kScanE consecutive counts, so a tile of 256 kScanE counts
// costs one round of loads.
constexpr int kScanE = 8;
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
    // only the sequence's own token blocks hold records (blocks past its end
    // have zero counts and are never read): scan element e is partition
    // e / nb, block e % nb
    const int nb = (int)((len + kTokBlock - 1) / kTokBlock);
    const int M = N * nb;
    int32_t* c = counts + (int64_t)sh * N * nblk;
    if (nb == 0)
        for (int i = threadIdx.x; i < N; i += blockDim.x) seg_offsets[(int64_t)sh * N + i] = carry;
    for (int base = 0; base < M; base += (int)blockDim.x * kScanE) {
        const int e0 = base + (int)threadIdx.x * kScanE;
        int x[kScanE];
        int tsum = 0;
#pragma unroll
        for (int u = 0; u < kScanE; u++) {
            const int e = e0 + u;
            x[u] = e < M ? c[(e / nb) * nblk + e % nb] : 0;
            tsum += x[u];
        }
        int total;
        int run = carry + block_exclusive_scan(tsum, tmp, total);
#pragma unroll
        for (int u = 0; u < kScanE; u++) {
            const int e = e0 + u;
            if (e < M) {
                c[(e / nb) * nblk + e % nb] = run;
                if (e % nb == 0) seg_offsets[(int64_t)sh * N + e / nb] = run;
            }
            run += x[u];
        }
        carry += total;
    }
    if (sh == (int)gridDim.x - 1 && threadIdx.x == 0)
        seg_offsets[(int64_t)num_seqs * H * N] = (int32_t)(K * ((int64_t)H * cu[num_seqs]));
}

// Forward scatter: one wave per (sequence, head, 64-token block) reads the
// head-major records of route_count (lane = token) and writes each routed
// record as one 16-byte SegRec at its block start (after block_scan) + rank.
constexpr int kScatterWaves = 4;
__global__ __launch_bounds__(kScatterWaves * kWave) void scatter_fwd_kernel(
    const uint2* __restrict__ rinfo, const int32_t* __restrict__ cu, int64_t T, int H, int N,
    int K, int nblk, const int32_t* __restrict__ pos, const float* __restrict__ lnz2,
    SegRec* __restrict__ seg) {
    static_assert(kTokBlock == kWave, "one wave per token block");
    const int sh = blockIdx.x;
    const int blk = blockIdx.y * kScatterWaves + (int)(threadIdx.x / kWave);
    if (blk >= nblk) return;  // wave-uniform
    const int s = sh / H, h = sh % H;
    const int64_t t1 = cu[s + 1];
    const int64_t tb = cu[s] + (int64_t)blk * kTokBlock;
    if (tb >= t1) return;  // wave-uniform
    const int lane = threadIdx.x % kWave;
    const bool valid = tb + lane < t1;
    const int64_t t = valid ? tb + lane : tb;  // invalid lanes re-read a valid token
    const int start = lane < N ? pos[((int64_t)sh * N + lane) * nblk + blk] : 0;
    const uint32_t row = (uint32_t)t * (uint32_t)H + (uint32_t)h;
    const float l2 = lnz2[row];
    uint2 inf[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++)
        if (j < K) inf[j] = rinfo[((int64_t)h * T + t) * K + j];
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j < K) {
            const int i = (int)(inf[j].x & 0xffffu), rank = (int)(inf[j].x >> 16);
            const int p = __shfl(start, i, kWave) + rank;  // all lanes active here
            const float wj = __uint_as_float(inf[j].y);
            if (valid)
                *reinterpret_cast<uint4*>(seg + p) =
                    make_uint4(row, row * (uint32_t)K + (uint32_t)j,
                               __float_as_uint(l2 - log2f(wj)), inf[j].y);
        }
    }
}

// Stable scatter of the records of one (sequence, head, token block) for
// the standalone grouping entry point: one wave per 64-token block (a token
// block is exactly one wave, so a record's rank among the block's records of
// its partition is a ballot popcount), four token blocks per launch block.
__global__ __launch_bounds__(kScatterWaves * kWave) void scatter_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ win, const int32_t* __restrict__ cu,
    int H, int N, int K, int nblk, const int32_t* __restrict__ pos, int32_t* __restrict__ seg_tok,
    int32_t* __restrict__ seg_slot, float* __restrict__ seg_w) {
    static_assert(kTokBlock == kWave, "one wave per token block");
    const int sh = blockIdx.x;
    const int blk = blockIdx.y * kScatterWaves + (int)(threadIdx.x / kWave);
    if (blk >= nblk) return;  // wave-uniform
    const int s = sh / H, h = sh % H;
    const int64_t t1 = cu[s + 1];
    const int64_t tb = cu[s] + (int64_t)blk * kTokBlock;
    if (tb >= t1) return;  // wave-uniform
    const int lane = threadIdx.x % kWave;
    const int64_t t = tb + lane;
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
    int rank[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) rank[j] = 0;
    for (int i = 0; i < N; i++) {
        const uint64_t bal = __ballot((mine >> i) & 1ull);
#pragma unroll
        for (int j = 0; j < kMaxTopK; j++)
            if (sel[j] == i) rank[j] = __popcll(bal & lt);
    }
    if (!valid) return;
#pragma unroll
    for (int j = 0; j < kMaxTopK; j++) {
        if (j < K) {
            const int i = sel[j];
            const int p = pos[((int64_t)sh * N + i) * nblk + blk] + rank[j];
            seg_tok[p] = (int32_t)t;
            if (seg_slot) seg_slot[p] = j;
            if (seg_w) seg_w[p] = win[(t * H + h) * K + j];
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


template <int NMAX, typename TIn>
static void launch_rc_n(dim3 grid, const TIn* z, const TIn* kl, const int32_t* cu, int64_t T,
                        int H, int c, int N, int K, int nblk, int32_t* idx, float* w,
                        int32_t* counts, uint2* rinfo, float* lnz2, hipStream_t st) {
    const size_t lds = (sizeof(float) + 1) * (size_t)kHG * kTokBlock * K;  // <= 40 KB
    if (c == 32)
        route_count_kernel<NMAX, 32, TIn><<<grid, 256, lds, st>>>(z, kl, cu, T, H, N, K, nblk, idx, w, counts, rinfo, lnz2);
    else if (c == 64)
        route_count_kernel<NMAX, 64, TIn><<<grid, 256, lds, st>>>(z, kl, cu, T, H, N, K, nblk, idx, w, counts, rinfo, lnz2);
    else
        route_count_kernel<NMAX, 128, TIn><<<grid, 256, lds, st>>>(z, kl, cu, T, H, N, K, nblk, idx, w, counts, rinfo, lnz2);
}

template <typename TIn>
static hipError_t launch_route_count_t(const void* z, const void* kl, const int32_t* cu,
                                       int num_seqs, int max_seqlen, int64_t T, int H, int c,
                                       int N, int K, int32_t* idx, float* w, int32_t* counts,
                                       uint2* rinfo, float* lnz2, hipStream_t st) {
    const int nblk = group_nblk(max_seqlen);
    if ((int64_t)num_seqs * H == 0) return hipSuccess;
    if (H > kMaxH || N > kMaxN || K > kMaxTopK) return hipErrorInvalidValue;
    dim3 grid((unsigned)nblk, (unsigned)num_seqs, (unsigned)((H + kHG - 1) / kHG));
    const TIn* zz = static_cast<const TIn*>(z);
    const TIn* kk = static_cast<const TIn*>(kl);
    if (N <= 8)
        launch_rc_n<8, TIn>(grid, zz, kk, cu, T, H, c, N, K, nblk, idx, w, counts, rinfo, lnz2, st);
    else if (N <= 16)
        launch_rc_n<16, TIn>(grid, zz, kk, cu, T, H, c, N, K, nblk, idx, w, counts, rinfo, lnz2, st);
    else if (N <= 32)
        launch_rc_n<32, TIn>(grid, zz, kk, cu, T, H, c, N, K, nblk, idx, w, counts, rinfo, lnz2, st);
    else
        launch_rc_n<64, TIn>(grid, zz, kk, cu, T, H, c, N, K, nblk, idx, w, counts, rinfo, lnz2, st);
    return hipGetLastError();
}

hipError_t launch_route_count(const void* z, const void* kl, int dtype, const int32_t* cu,
                              int num_seqs, int max_seqlen, int64_t T, int H, int c, int N, int K,
                              int32_t* idx, float* w, int32_t* counts, uint2* rinfo, float* lnz2,
                              hipStream_t st) {
    return dtype == kF32
               ? launch_route_count_t<float>(z, kl, cu, num_seqs, max_seqlen, T, H, c, N, K, idx,
                                             w, counts, rinfo, lnz2, st)
               : launch_route_count_t<bf16_t>(z, kl, cu, num_seqs, max_seqlen, T, H, c, N, K,
                                              idx, w, counts, rinfo, lnz2, st);
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
                        int max_seqlen, int H, int N, int K, int32_t* counts,
                        int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot, float* seg_w,
                        hipStream_t st) {
    const int nblk = group_nblk(max_seqlen);
    const unsigned SH = (unsigned)(num_seqs * H);
    if (SH == 0) {
        // no sequences: only the terminal offset exists
        zero_int_kernel<<<1, 1, 0, st>>>(seg_offsets);
        return hipGetLastError();
    }
    count_kernel<<<dim3(SH, nblk), kTokBlock, 0, st>>>(idx, cu, H, N, K, nblk, counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    block_scan_kernel<<<SH, 256, 0, st>>>(cu, H, N, K, nblk, counts, seg_offsets, num_seqs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    scatter_kernel<<<dim3(SH, (nblk + kScatterWaves - 1) / kScatterWaves), kScatterWaves * kWave,
                     0, st>>>(idx, w, cu, H, N, K, nblk, counts, seg_tok, seg_slot, seg_w);
    return hipGetLastError();
}

// Key normalisers alone (used when the routed and shared partitions have
// different keys, or when no routing kernel runs): one (token, head) row per
// CK/8 (bf16) or CK/4 (fp32) lanes, 16-byte loads, max-shifted sum of exp2
// with row reductions in registers.
template <int CK, typename TIn>
__global__ __launch_bounds__(256) void key_norm_kernel(const TIn* __restrict__ kl, int64_t rows,
                                                       float* __restrict__ lnz2) {
    constexpr int VPL = 16 / (int)sizeof(TIn);   // values per lane
    constexpr int LPR = CK / VPL;                // lanes per row
    constexpr int RPB = 256 / LPR;               // rows per block
    const int sub = threadIdx.x % LPR;
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const bool ok = r < rows;
    const uint4 v = reinterpret_cast<const uint4*>(kl + (ok ? r : 0) * CK)[sub];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float x[VPL];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        if constexpr (sizeof(TIn) == 2) {
            x[2 * e] = __uint_as_float(w4[e] << 16);
            x[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
        } else {
            x[e] = __uint_as_float(w4[e]);
        }
    }
    float m = x[0];
#pragma unroll
    for (int j = 1; j < VPL; j++) m = fmaxf(m, x[j]);
    m = row_reduce<LPR>(m, [](float u, float w) { return fmaxf(u, w); });
    const float m2 = m * kLog2e;
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; j++) sum += __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -m2));
    sum = row_reduce<LPR>(sum, [](float u, float w) { return u + w; });
    if (ok && sub == 0) lnz2[r] = m2 + log2f(sum);
}

template <typename TIn>
static hipError_t launch_key_norm_t(const void* kl, int64_t rows, int c, float* lnz2,
                                    hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const TIn* k = static_cast<const TIn*>(kl);
    constexpr int VPL = 16 / (int)sizeof(TIn);
    const int64_t rpb = 256 / (c / VPL);
    const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
    if (c == 32)
        key_norm_kernel<32, TIn><<<grid, 256, 0, st>>>(k, rows, lnz2);
    else if (c == 64)
        key_norm_kernel<64, TIn><<<grid, 256, 0, st>>>(k, rows, lnz2);
    else if (c == 128)
        key_norm_kernel<128, TIn><<<grid, 256, 0, st>>>(k, rows, lnz2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_key_norm(const void* kl, int dtype, int64_t rows, int c, float* lnz2,
                           hipStream_t st) {
    return dtype == kF32 ? launch_key_norm_t<float>(kl, rows, c, lnz2, st)
                         : launch_key_norm_t<bf16_t>(kl, rows, c, lnz2, st);
}

// Debug copies of the forward's own grouping: the segment offsets as
// scanned, and the token and top-k rank of every record the chunk kernels
// read (decoded from its input row t*H + h and slot row (t*H + h)*K + rank).
__global__ __launch_bounds__(256) void seg_debug_kernel(const SegRec* __restrict__ seg,
                                                        const int32_t* __restrict__ seg_off,
                                                        int64_t nrec, int64_t noff, int H, int K,
                                                        int32_t* __restrict__ out_off,
                                                        int32_t* __restrict__ out_tok,
                                                        int32_t* __restrict__ out_slot) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (out_off && i < noff) out_off[i] = seg_off[i];
    if (i < nrec) {
        const uint2 r = *reinterpret_cast<const uint2*>(seg + i);
        if (out_tok) out_tok[i] = (int32_t)(r.x / (uint32_t)H);
        if (out_slot) out_slot[i] = (int32_t)(r.y % (uint32_t)K);
    }
}

hipError_t launch_seg_debug(const SegRec* seg, const int32_t* seg_off, int64_t nrec, int64_t nseg,
                            int H, int K, int32_t* out_off, int32_t* out_tok, int32_t* out_slot,
                            hipStream_t st) {
    const int64_t n = nrec > nseg + 1 ? nrec : nseg + 1;
    if (!out_off && !out_tok && !out_slot) return hipSuccess;
    seg_debug_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(seg, seg_off, nrec, nseg + 1, H,
                                                                  K, out_off, out_tok, out_slot);
    return hipGetLastError();
}

hipError_t launch_group_fwd(const uint2* rinfo, const int32_t* cu, int num_seqs, int max_seqlen,
                            int64_t T, int H, int N, int K, int32_t* counts, int32_t* seg_offsets,
                            const float* lnz2, SegRec* seg, hipStream_t st) {
    const int nblk = group_nblk(max_seqlen);
    const unsigned SH = (unsigned)(num_seqs * H);
    if (SH == 0) {
        zero_int_kernel<<<1, 1, 0, st>>>(seg_offsets);
        return hipGetLastError();
    }
    block_scan_kernel<<<SH, 256, 0, st>>>(cu, H, N, K, nblk, counts, seg_offsets, num_seqs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scatter_fwd_kernel<<<dim3(SH, (nblk + kScatterWaves - 1) / kScatterWaves),
                         kScatterWaves * kWave, 0, st>>>(rinfo, cu, T, H, N, K, nblk, counts, lnz2,
                                                         seg);
    return hipGetLastError();
}

}  // namespace sse
