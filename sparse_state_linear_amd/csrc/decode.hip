// decode.hip -- one SSE decode step for gfx950.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. (9)-(14) for a single token, with the shared partition of §2.5;
// §2.6 (decode recurs only on the selected states; unselected states keep an
// identity transition).
//
// One block per (sequence*head, 32-column slice of d), four waves; wave w
// owns rows [w c/4, (w+1) c/4) of the slice, lane = (4-column group, row
// group), so each row's 128 bytes are read and written by 8 lanes.  The step
// is HBM-bound (per (b, h) it moves 2 (k+1) c d fp32 values), so the kernel
// is arranged to put state loads in flight as early as possible:
//   1. the shared partition's slice does not depend on the routing and is
//      loaded first, together with the token's inputs;
//   2. every wave computes the key softmax (eq. 11) and the router (eqs.
//      9-10) by itself with wave reductions, so no block barrier stands
//      between the loads and the routing;
//   3. the routed slices are loaded two partitions at a time, the first pair
//      before the shared slice is processed.
// The N - k unselected states are never read or written.  The gated reads
// are reduced over rows inside each wave and across the four waves through
// LDS, in a fixed order (deterministic).
#include "sse_launch.h"

namespace sse {

constexpr int kDecCols = 32;     // columns of d per block
constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * kWave;

// State slices are read once and written once per step, and a step touches
// far more than the caches hold: nontemporal loads and stores (measured
// a few per cent faster than plain ones on gfx950).
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float* p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(float* p, const float4& y) {
    const f32x4v v = {y.x, y.y, y.z, y.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
}

template <int CK, typename TIn>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ kl, const TIn* __restrict__ v,
    const TIn* __restrict__ la, const TIn* __restrict__ z, int H, int d, int N, int K,
    float* __restrict__ states, float* __restrict__ o, int32_t* __restrict__ topk_idx) {
    constexpr int RW = CK / kDecWaves;         // rows per wave
    constexpr int RG = kWave / (kDecCols / 4); // row groups per wave (8)
    constexpr int RPT = RW / RG;               // rows per lane
    constexpr int KPL = (CK + kWave - 1) / kWave;  // key logits per lane
    static_assert(RPT >= 1 && RW % RG == 0, "rows must split evenly over the row groups");
    __shared__ float s_o[kDecWaves][kDecCols];

    const int bh = blockIdx.x, cb = blockIdx.y, d0 = cb * kDecCols;
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c4 = lane % (kDecCols / 4), rg = lane / (kDecCols / 4);
    const int64_t in_c = (int64_t)bh * CK;
    const int64_t cd = (int64_t)CK * d;
    // this lane's rows j = RW wv + rg + RG u and columns d0 + 4 c4 .. + 3
    float* const Sbh = states + (int64_t)bh * (N + 1) * cd + (int64_t)(wv * RW + rg) * d + d0 + 4 * c4;

    // ---- 1. shared slice and the token's inputs
    float4 xs[RPT];
    const float* Ssh = Sbh + (int64_t)N * cd;
#pragma unroll
    for (int u = 0; u < RPT; u++) xs[u] = load_nt(Ssh + (int64_t)(RG * u) * d);
    float qj[RPT], klj[RPT], laj[RPT];
#pragma unroll
    for (int u = 0; u < RPT; u++) {
        const int64_t j = in_c + wv * RW + rg + RG * u;
        qj[u] = to_f32(q[j]);
        klj[u] = to_f32(kl[j]);
        laj[u] = to_f32(la[j]);
    }
    float4 vv;
    {
        const int64_t vo = (int64_t)bh * d + d0 + 4 * c4;
        vv = make_float4(to_f32(v[vo]), to_f32(v[vo + 1]), to_f32(v[vo + 2]), to_f32(v[vo + 3]));
    }
    float kx[KPL];
#pragma unroll
    for (int i = 0; i < KPL; i++) kx[i] = lane + kWave * i < CK ? to_f32(kl[in_c + lane + kWave * i]) : -INFINITY;
    const float zi = lane < N ? to_f32(z[(int64_t)bh * N + lane]) : -INFINITY;

    // ---- 2. key softmax (eq. 11) and decay (eq. 6) of this lane's rows
    float km = kx[0];
#pragma unroll
    for (int i = 1; i < KPL; i++) km = fmaxf(km, kx[i]);
    km = wave_max(km);
    float ks = 0.f;
#pragma unroll
    for (int i = 0; i < KPL; i++) ks += lane + kWave * i < CK ? expf(kx[i] - km) : 0.f;
    const float kden = wave_sum(ks);
    float kap[RPT], alp[RPT];
#pragma unroll
    for (int u = 0; u < RPT; u++) {
        kap[u] = expf(klj[u] - km) / kden;
        alp[u] = expf(laj[u]);
    }
    // router softmax (eq. 9): max and denominator over the N logits
    const float zm = wave_max(zi);
    const float zden = wave_sum(lane < N ? expf(zi - zm) : 0.f);

    // S <- diag(alpha) S + w kappa^T v on this lane's rows, stored in place;
    // returns q S over those rows (eqs. 12-13 for one partition)
    auto update = [&](float* Sp, const float4 (&x)[RPT], float w) {
        float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < RPT; u++) {
            const float a = alp[u], wk = w * kap[u];
            float4 y;
            y.x = a * x[u].x + wk * vv.x;
            y.y = a * x[u].y + wk * vv.y;
            y.z = a * x[u].z + wk * vv.z;
            y.w = a * x[u].w + wk * vv.w;
            store_nt(Sp + (int64_t)(RG * u) * d, y);
            part.x += qj[u] * y.x;
            part.y += qj[u] * y.y;
            part.z += qj[u] * y.z;
            part.w += qj[u] * y.w;
        }
        return part;
    };

    // ---- 3. routed partitions, two at a time (eq. 10: descending logits,
    //         equal logits -> lower index)
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f), psh = acc;
    bool taken = false;
    for (int r0 = 0; r0 < K; r0 += 2) {
        int p[2] = {0, 0};
        float w[2] = {0.f, 0.f};
        float4 x[2][RPT];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int r = r0 + h2;
            if (r < K) {  // wave-uniform
                float bv = (lane < N && !taken) ? zi : -INFINITY;
                int bi = (lane < N && !taken) ? lane : kWave;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const float ov = __shfl_xor(bv, off, kWave);
                    const int oi = __shfl_xor(bi, off, kWave);
                    if (ov > bv || (ov == bv && oi < bi)) {
                        bv = ov;
                        bi = oi;
                    }
                }
                if (lane == bi) taken = true;
                // (bi < N for finite logits; the clamp keeps the address in
                // range whatever the logits hold)
                p[h2] = min(__builtin_amdgcn_readfirstlane(bi), N - 1);
                w[h2] = expf(bv - zm) / zden;
                if (topk_idx && cb == 0 && wv == 0 && lane == 0) topk_idx[(int64_t)bh * K + r] = bi;
                const float* Sp = Sbh + (int64_t)p[h2] * cd;
#pragma unroll
                for (int u = 0; u < RPT; u++)
                    x[h2][u] = load_nt(Sp + (int64_t)(RG * u) * d);
            }
        }
        if (r0 == 0) psh = update(Sbh + (int64_t)N * cd, xs, 1.f);  // shared partition, weight 1
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            if (r0 + h2 < K) {
                const float4 part = update(Sbh + (int64_t)p[h2] * cd, x[h2], w[h2]);
                acc.x += w[h2] * part.x;
                acc.y += w[h2] * part.y;
                acc.z += w[h2] * part.z;
                acc.w += w[h2] * part.w;
            }
        }
    }
    acc.x += psh.x;
    acc.y += psh.y;
    acc.z += psh.z;
    acc.w += psh.w;

    // ---- 4. o = sum of the gated reads: over the row groups of the wave,
    //         then over the waves
#pragma unroll
    for (int off = kDecCols / 4; off < kWave; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off, kWave);
        acc.y += __shfl_xor(acc.y, off, kWave);
        acc.z += __shfl_xor(acc.z, off, kWave);
        acc.w += __shfl_xor(acc.w, off, kWave);
    }
    if (lane < kDecCols / 4) *reinterpret_cast<float4*>(&s_o[wv][4 * lane]) = acc;
    __syncthreads();
    if (threadIdx.x < kDecCols) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < kDecWaves; i++) sum += s_o[i][threadIdx.x];
        o[(int64_t)bh * d + d0 + threadIdx.x] = sum;
    }
}

// General decode step: the shared partition's own query and key (q_sh,
// kl_sh; the routed ones when null) and a read set chosen by its own router
// logits zr (top-kr; the write set when null).  Same block layout as
// decode_kernel.  The write set is updated in place (eq. 12); every
// partition in the read set is read after the writes with its read weight
// (a partition read but not written is read from its unchanged state and
// not stored); the shared partition is written with kappa_sh and read with
// q_sh.  Each partition of the union of the two sets is loaded once.
template <int CK, typename TIn>
__global__ __launch_bounds__(kDecThreads) void decode_ex_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ kl, const TIn* __restrict__ v,
    const TIn* __restrict__ la, const TIn* __restrict__ z, const TIn* __restrict__ q_sh,
    const TIn* __restrict__ kl_sh, const TIn* __restrict__ zr, int H, int d, int N, int K, int KR,
    float* __restrict__ states, float* __restrict__ o, int32_t* __restrict__ topk_idx,
    int32_t* __restrict__ read_idx) {
    constexpr int RW = CK / kDecWaves;
    constexpr int RG = kWave / (kDecCols / 4);
    constexpr int RPT = RW / RG;
    constexpr int KPL = (CK + kWave - 1) / kWave;
    __shared__ float s_o[kDecWaves][kDecCols];

    const int bh = blockIdx.x, cb = blockIdx.y, d0 = cb * kDecCols;
    const int lane = threadIdx.x % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c4 = lane % (kDecCols / 4), rg = lane / (kDecCols / 4);
    const int64_t in_c = (int64_t)bh * CK;
    const int64_t cd = (int64_t)CK * d;
    float* const Sbh = states + (int64_t)bh * (N + 1) * cd + (int64_t)(wv * RW + rg) * d + d0 + 4 * c4;
    const TIn* qs = q_sh ? q_sh : q;
    const TIn* ks = kl_sh ? kl_sh : kl;

    float qj[RPT], qsj[RPT], alp[RPT];
    float4 vv;
    {
        const int64_t vo = (int64_t)bh * d + d0 + 4 * c4;
        vv = make_float4(to_f32(v[vo]), to_f32(v[vo + 1]), to_f32(v[vo + 2]), to_f32(v[vo + 3]));
    }
    // key softmax over the c rows (eq. 11) for a key-logit row
    auto key_rows = [&](const TIn* kr, float (&kap)[RPT]) {
        float kx[KPL];
#pragma unroll
        for (int i = 0; i < KPL; i++)
            kx[i] = lane + kWave * i < CK ? to_f32(kr[in_c + lane + kWave * i]) : -INFINITY;
        float km = kx[0];
#pragma unroll
        for (int i = 1; i < KPL; i++) km = fmaxf(km, kx[i]);
        km = wave_max(km);
        float ksum = 0.f;
#pragma unroll
        for (int i = 0; i < KPL; i++) ksum += lane + kWave * i < CK ? expf(kx[i] - km) : 0.f;
        const float kden = wave_sum(ksum);
#pragma unroll
        for (int u = 0; u < RPT; u++)
            kap[u] = expf(to_f32(kr[in_c + wv * RW + rg + RG * u]) - km) / kden;
    };
    float kap[RPT], kaps[RPT];
    key_rows(kl, kap);
    key_rows(ks, kaps);
#pragma unroll
    for (int u = 0; u < RPT; u++) {
        const int64_t j = in_c + wv * RW + rg + RG * u;
        qj[u] = to_f32(q[j]);
        qsj[u] = to_f32(qs[j]);
        alp[u] = expf(to_f32(la[j]));
    }
    // router softmax and top-k of a logit row (eqs. 9-10; ties -> lower index)
    auto route = [&](const TIn* zz, int KK, int (&sel)[kMaxTopK], float (&wsel)[kMaxTopK]) {
        const float zi = lane < N ? to_f32(zz[(int64_t)bh * N + lane]) : -INFINITY;
        const float zm = wave_max(zi);
        const float zden = wave_sum(lane < N ? expf(zi - zm) : 0.f);
        bool taken = false;
        for (int r = 0; r < KK; r++) {
            float bv = (lane < N && !taken) ? zi : -INFINITY;
            int bi = (lane < N && !taken) ? lane : kWave;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off, kWave);
                const int oi = __shfl_xor(bi, off, kWave);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == bi) taken = true;
            sel[r] = min(__builtin_amdgcn_readfirstlane(bi), N - 1);
            wsel[r] = expf(bv - zm) / zden;
        }
    };
    int wsel[kMaxTopK], rsel[kMaxTopK];
    float ww[kMaxTopK], wr[kMaxTopK];
    route(z, K, wsel, ww);
    if (zr) {
        route(zr, KR, rsel, wr);
    } else {
        for (int r = 0; r < K; r++) {
            rsel[r] = wsel[r];
            wr[r] = ww[r];
        }
    }
    const int nr = zr ? KR : K;
    if (cb == 0 && wv == 0 && lane == 0) {
        if (topk_idx)
            for (int r = 0; r < K; r++) topk_idx[(int64_t)bh * K + r] = wsel[r];
        if (read_idx)
            for (int r = 0; r < nr; r++) read_idx[(int64_t)bh * nr + r] = rsel[r];
    }

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // one partition: optional write (weight we, key kk), optional read
    // (weight wrd, query qq); the state is stored only when written
    auto visit = [&](int p, bool wr_on, float we, const float (&kk)[RPT], bool rd_on, float wrd,
                     const float (&qq)[RPT]) {
        float* Sp = Sbh + (int64_t)p * cd;
        float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < RPT; u++) {
            float4 y = load_nt(Sp + (int64_t)(RG * u) * d);
            if (wr_on) {
                const float a = alp[u], wk = we * kk[u];
                y.x = a * y.x + wk * vv.x;
                y.y = a * y.y + wk * vv.y;
                y.z = a * y.z + wk * vv.z;
                y.w = a * y.w + wk * vv.w;
                store_nt(Sp + (int64_t)(RG * u) * d, y);
            }
            part.x += qq[u] * y.x;
            part.y += qq[u] * y.y;
            part.z += qq[u] * y.z;
            part.w += qq[u] * y.w;
        }
        if (rd_on) {
            acc.x += wrd * part.x;
            acc.y += wrd * part.y;
            acc.z += wrd * part.z;
            acc.w += wrd * part.w;
        }
    };
    // the write set (read too when it is also in the read set)
    for (int r = 0; r < K; r++) {
        const int p = wsel[r];
        int jr = -1;
        for (int x = 0; x < nr; x++)
            if (rsel[x] == p) jr = x;
        visit(p, true, ww[r], kap, jr >= 0, jr >= 0 ? wr[jr] : 0.f, qj);
    }
    // partitions read but not written
    for (int x = 0; x < nr; x++) {
        const int p = rsel[x];
        bool written = false;
        for (int r = 0; r < K; r++) written = written || wsel[r] == p;
        if (!written) visit(p, false, 0.f, kap, true, wr[x], qj);
    }
    // the shared partition (weight 1, its own key and query)
    visit(N, true, 1.f, kaps, true, 1.f, qsj);

#pragma unroll
    for (int off = kDecCols / 4; off < kWave; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off, kWave);
        acc.y += __shfl_xor(acc.y, off, kWave);
        acc.z += __shfl_xor(acc.z, off, kWave);
        acc.w += __shfl_xor(acc.w, off, kWave);
    }
    if (lane < kDecCols / 4) *reinterpret_cast<float4*>(&s_o[wv][4 * lane]) = acc;
    __syncthreads();
    if (threadIdx.x < kDecCols) {
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < kDecWaves; i++) sum += s_o[i][threadIdx.x];
        o[(int64_t)bh * d + d0 + threadIdx.x] = sum;
    }
}

template <int CK, typename TIn>
static void launch_decode_ck(const void* q, const void* kl, const void* v, const void* la,
                             const void* z, int B, int H, int d, int N, int K, float* states,
                             float* o, int32_t* idx, hipStream_t st) {
    dim3 grid((unsigned)(B * H), (unsigned)(d / kDecCols)), block(kDecThreads);
    decode_kernel<CK, TIn><<<grid, block, 0, st>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(kl), static_cast<const TIn*>(v),
        static_cast<const TIn*>(la), static_cast<const TIn*>(z), H, d, N, K, states, o, idx);
}

template <typename TIn>
static void launch_decode_t(const void* q, const void* kl, const void* v, const void* la,
                            const void* z, int B, int H, int c, int d, int N, int K,
                            float* states, float* o, int32_t* idx, hipStream_t st) {
    if (c == 32)
        launch_decode_ck<32, TIn>(q, kl, v, la, z, B, H, d, N, K, states, o, idx, st);
    else if (c == 64)
        launch_decode_ck<64, TIn>(q, kl, v, la, z, B, H, d, N, K, states, o, idx, st);
    else
        launch_decode_ck<128, TIn>(q, kl, v, la, z, B, H, d, N, K, states, o, idx, st);
}

hipError_t launch_decode(const void* q, const void* kl, const void* v, const void* la,
                         const void* z, int dtype, int B, int H, int c, int d, int N, int K,
                         float* states, float* o, int32_t* topk_idx, hipStream_t st) {
    if ((int64_t)B * H == 0) return hipSuccess;
    if (dtype == kF32)
        launch_decode_t<float>(q, kl, v, la, z, B, H, c, d, N, K, states, o, topk_idx, st);
    else
        launch_decode_t<bf16_t>(q, kl, v, la, z, B, H, c, d, N, K, states, o, topk_idx, st);
    return hipGetLastError();
}

template <int CK, typename TIn>
static void launch_decode_ex_ck(const void* q, const void* kl, const void* v, const void* la,
                                const void* z, const void* qs, const void* ks, const void* zr,
                                int B, int H, int d, int N, int K, int KR, float* states, float* o,
                                int32_t* idx, int32_t* ridx, hipStream_t st) {
    dim3 grid((unsigned)(B * H), (unsigned)(d / kDecCols)), block(kDecThreads);
    decode_ex_kernel<CK, TIn><<<grid, block, 0, st>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(kl), static_cast<const TIn*>(v),
        static_cast<const TIn*>(la), static_cast<const TIn*>(z), static_cast<const TIn*>(qs),
        static_cast<const TIn*>(ks), static_cast<const TIn*>(zr), H, d, N, K, KR, states, o, idx,
        ridx);
}

template <typename TIn>
static void launch_decode_ex_t(const void* q, const void* kl, const void* v, const void* la,
                               const void* z, const void* qs, const void* ks, const void* zr,
                               int B, int H, int c, int d, int N, int K, int KR, float* states,
                               float* o, int32_t* idx, int32_t* ridx, hipStream_t st) {
    if (c == 32)
        launch_decode_ex_ck<32, TIn>(q, kl, v, la, z, qs, ks, zr, B, H, d, N, K, KR, states, o,
                                     idx, ridx, st);
    else if (c == 64)
        launch_decode_ex_ck<64, TIn>(q, kl, v, la, z, qs, ks, zr, B, H, d, N, K, KR, states, o,
                                     idx, ridx, st);
    else
        launch_decode_ex_ck<128, TIn>(q, kl, v, la, z, qs, ks, zr, B, H, d, N, K, KR, states, o,
                                      idx, ridx, st);
}

hipError_t launch_decode_ex(const void* q, const void* kl, const void* v, const void* la,
                            const void* z, const void* q_sh, const void* kl_sh, const void* zr,
                            int dtype, int B, int H, int c, int d, int N, int K, int KR,
                            float* states, float* o, int32_t* topk_idx, int32_t* read_idx,
                            hipStream_t st) {
    if ((int64_t)B * H == 0) return hipSuccess;
    if (dtype == kF32)
        launch_decode_ex_t<float>(q, kl, v, la, z, q_sh, kl_sh, zr, B, H, c, d, N, K, KR, states,
                                  o, topk_idx, read_idx, st);
    else
        launch_decode_ex_t<bf16_t>(q, kl, v, la, z, q_sh, kl_sh, zr, B, H, c, d, N, K, KR,
                                   states, o, topk_idx, read_idx, st);
    return hipGetLastError();
}

}  // namespace sse
