// decode.hip -- one SSE decode step for gfx950.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. (9)-(14) for a single token, with the shared partition of §2.5;
// §2.6 (decode recurs only on the selected states; unselected states keep an
// identity transition).
//
// One block per (sequence*head, 32-column slice of d).  Each block routes its
// token (wave 0), computes the key softmax and decay for the c rows, and then
// streams the c x 32 slices of the k+1 active states: read, decay, rank-one
// write, store back in place, and accumulate the gated read q S.  The other
// N-k routed states are never touched.  The step is HBM-bound: per (b, h) it
// moves 2 (k+1) c d fp32 values.
#include "sse_launch.h"

namespace sse {

constexpr int kDecCols = 32;     // columns of d per block
constexpr int kDecThreads = 256;

template <int CK, typename TIn>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ kl, const TIn* __restrict__ v,
    const TIn* __restrict__ la, const TIn* __restrict__ z, int H, int d, int N, int K,
    float* __restrict__ states, float* __restrict__ o, int32_t* __restrict__ topk_idx) {
    constexpr int RG = kDecThreads / (kDecCols / 4);  // row groups (32)
    constexpr int RPT = CK / RG > 0 ? CK / RG : 1;    // rows per thread
    __shared__ float s_kappa[CK], s_alpha[CK], s_q[CK], s_v[kDecCols];
    __shared__ float s_red[2][kDecThreads / kWave];
    __shared__ float s_w[kMaxTopK + 1];
    __shared__ int s_part[kMaxTopK + 1];
    __shared__ float s_opart[kDecThreads / kWave][kDecCols];

    const int bh = blockIdx.x, cb = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
    const int d0 = cb * kDecCols;

    // ---- router (wave 0): eq. (9) softmax over N, eq. (10) top-k on logits
    if (wv == 0) {
        const float zi = lane < N ? to_f32(z[(int64_t)bh * N + lane]) : -INFINITY;
        const float m = wave_max(zi);
        const float den = wave_sum(lane < N ? expf(zi - m) : 0.f);
        bool taken = false;
        for (int r = 0; r < K; r++) {
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
            if (lane == 0) {
                s_part[r] = bi;
                s_w[r] = expf(bv - m) / den;
                if (topk_idx && cb == 0) topk_idx[(int64_t)bh * K + r] = bi;
            }
        }
        if (lane == 0) {
            s_part[K] = N;   // shared partition, weight 1
            s_w[K] = 1.f;
        }
    }
    // ---- key softmax (eq. 11), decay (eq. 6), query, value slice
    float kx = -INFINITY;
    if (tid < CK) {
        const int64_t off = (int64_t)bh * CK + tid;
        kx = to_f32(kl[off]);
        s_alpha[tid] = expf(to_f32(la[off]));
        s_q[tid] = to_f32(q[off]);
    }
    if (tid < kDecCols) s_v[tid] = to_f32(v[(int64_t)bh * d + d0 + tid]);
    float m = wave_max(kx);
    if (lane == 0) s_red[0][wv] = m;
    __syncthreads();
    m = s_red[0][0];
    for (int i = 1; i < kDecThreads / kWave; i++) m = fmaxf(m, s_red[0][i]);
    const float ex = tid < CK ? expf(kx - m) : 0.f;
    const float ssum = wave_sum(ex);
    if (lane == 0) s_red[1][wv] = ssum;
    __syncthreads();
    float den = 0.f;
    for (int i = 0; i < kDecThreads / kWave; i++) den += s_red[1][i];
    if (tid < CK) s_kappa[tid] = ex / den;
    __syncthreads();

    // ---- stream the k+1 active state slices
    const int c4 = tid % (kDecCols / 4);   // float4 column group
    const int rg = tid / (kDecCols / 4);   // row group
    const float4 vv = *reinterpret_cast<const float4*>(&s_v[4 * c4]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t sbase = (int64_t)bh * (N + 1) * CK * d;
    for (int r = 0; r <= K; r++) {
        const int p = s_part[r];
        const float w = s_w[r];
        float* Sp = states + sbase + (int64_t)p * CK * d + d0 + 4 * c4;
        float4 x[RPT];
#pragma unroll
        for (int u = 0; u < RPT; u++) {
            const int j = rg + RG * u;
            if (j < CK) x[u] = *reinterpret_cast<const float4*>(Sp + (int64_t)j * d);
        }
        float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < RPT; u++) {
            const int j = rg + RG * u;
            if (j < CK) {
                const float a = s_alpha[j], wk = w * s_kappa[j], qj = s_q[j];
                float4 y;
                y.x = a * x[u].x + wk * vv.x;
                y.y = a * x[u].y + wk * vv.y;
                y.z = a * x[u].z + wk * vv.z;
                y.w = a * x[u].w + wk * vv.w;
                *reinterpret_cast<float4*>(Sp + (int64_t)j * d) = y;
                part.x += qj * y.x;
                part.y += qj * y.y;
                part.z += qj * y.z;
                part.w += qj * y.w;
            }
        }
        acc.x += w * part.x;
        acc.y += w * part.y;
        acc.z += w * part.z;
        acc.w += w * part.w;
    }
    // ---- reduce the partial reads over row groups
#pragma unroll
    for (int off = kDecCols / 4; off < kWave; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off, kWave);
        acc.y += __shfl_xor(acc.y, off, kWave);
        acc.z += __shfl_xor(acc.z, off, kWave);
        acc.w += __shfl_xor(acc.w, off, kWave);
    }
    if (lane < kDecCols / 4) {
        s_opart[wv][4 * lane + 0] = acc.x;
        s_opart[wv][4 * lane + 1] = acc.y;
        s_opart[wv][4 * lane + 2] = acc.z;
        s_opart[wv][4 * lane + 3] = acc.w;
    }
    __syncthreads();
    if (tid < kDecCols) {
        float sum = 0.f;
        for (int i = 0; i < kDecThreads / kWave; i++) sum += s_opart[i][tid];
        o[(int64_t)bh * d + d0 + tid] = sum;
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

}  // namespace sse
