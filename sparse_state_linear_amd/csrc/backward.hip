// backward.hip -- gradients of the SSE forward for gfx950: the chunked
// reverse pass over every partition segment, and the per-token combine.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. (9)-(14) (the same router probability e gates the write and the
// read, so the router logits get a continuous gradient through e; the top-k
// indices get none), §2.5 (shared partition, weight 1), §2.6 (each
// partition runs over its own records with an identity transition
// elsewhere, so the reverse pass runs over the same segments; an unselected
// partition's gradient state passes unchanged).
//
// The scalar whose gradient is taken is L = <do, o> + <dS_final, S_final>.
// One segment: records r in time order, gate w_r (= e, or 1 for the shared
// partition), chunks of C = 16 records.  In a chunk, with b the in-chunk
// cumulative log decay (per state row), D = diag(e^{b_C}),
//   Qt = q e^b,  K0 = kappa e^{-b},  Kh = w K0,  g_r = w_r do_r,
//   A  = (Qt Kh^T) masked to s <= r,  GV = (g V^T) masked to s <= r,
//   y  = Qt S_in + A V                 (the read before its gate)
// and, with G the gradient of the state after the chunk (G~ = D G),
//   dQt = g S_in^T + GV Kh,   dKh = GV^T Qt + V G~^T,
//   dV  = A^T g + Kh G~,      dS_in = Qt^T g + G~,
//   db  = Qt . dQt - Kh . dKh (per record and row), plus, at the chunk's
//         last record, sum_m S_out . G (the decay of the whole chunk);
//   dlog_alpha = reverse cumulative sum of db over the chunk's records,
//   dq = dQt e^b,  dkappa = w e^{-b} dKh,
//   dw = y . do + K0 . dKh   (the read gate and the write gate).
// S_in of every chunk comes from a forward sweep of the same block that
// stores it (checkpoints) before the reverse sweep.  The reverse sweep
// carries G in MFMA accumulator registers: wave w owns 16-column tiles
// w, w + 4, ... of the c x d state (all rows), like S_in.  Products that
// contract over state rows (Qt S_in, Kh G~, Qt^T g) use those registers as
// the MFMA B operand directly; products that contract over columns (g S_in^T,
// V G~^T) take them through a per-wave LDS transpose, 16 rows at a time, and
// the four waves' partial sums are added through LDS.  Every product runs on
// fp32 16x16x4 MFMA with fp32 operands.
//
// Each record's gradients (dq, dkappa turned into key-logit gradients, dv,
// dlog_alpha, dw) go to its own slot [token, head, rank] (rank = its place
// in the token's top-k list, k for the shared partition); the combine kernel
// sums a token's k + 1 slots and applies the router softmax Jacobian, so no
// atomics are used and every run gives the same bits.
#include "chunk_common.h"

namespace sse {

namespace {

typedef float f32x4b __attribute__((ext_vector_type(4)));

constexpr int kBC = 16;          // records per chunk
constexpr int kBW = 4;           // waves per block
constexpr int kBThreads = kBW * kWave;

// 16x16x4 fp32 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16]; the
// output gives lane l column l%16 and rows 4 (l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4b mf(float a, float b, f32x4b c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int drow(int g4, int i) { return 4 * g4 + i; }

// LDS writes of this wave complete before its next LDS reads are issued
// (for data exchanged between lanes of one wave).
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

template <int CK, int DV>
struct BwSmem {
    static constexpr int KS = CK + 1, VS = DV + 1;
    float qt[kBC][KS];           // Qt
    float k0[kBC][KS];           // K0 = kappa e^{-b}
    float bb[kBC][KS];           // b (natural log, in-chunk cumulative)
    float v[kBC][VS];
    float g[kBC][VS];            // g = w do
    float dob[kBC][VS];          // do
    float a[kBW][kBC][kBC + 1];  // partial A tiles (state-row quarters)
    float gv[kBW][kBC][kBC + 1]; // partial GV tiles (column quarters)
    float xp[kBW][16][33];       // per-wave transpose of 16 state rows x 32 columns
    float red[kBW][kBC][KS];     // per-wave partial of a column contraction
    float dqt[kBC][KS];
    float dkh[kBC][KS];
    float ebc[CK];               // e^{b_C}
    float dbc[kBW][CK];          // per-wave partial of sum_m S_out . G
    float dwp[kBW][kBC];         // per-wave partial of y . do
    float dww[kBC];              // K0 . dKh
    float lnz[kBC];
    float w[kBC];
    uint32_t row[kBC];           // input row t*H + h
    uint32_t slot[kBC];          // gradient slot row (t*H + h)*(k+1) + rank
    int valid[kBC];
};

}  // namespace

// Blocks [0, S*H) run the shared partition's chain of (s, h); blocks
// [S*H, S*H*(N+1)) run routed segment g = block - S*H.
template <int CK, int DV, typename TIn>
__global__ __launch_bounds__(kBThreads, 1) void bwd_kernel(const BwdArgs a) {
    using SM = BwSmem<CK, DV>;
    constexpr int RT = CK / 16;              // 16-row tiles of the state
    constexpr int NCT = DV / 16;             // 16-column tiles
    constexpr int CTW = NCT >= kBW ? NCT / kBW : 1;
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, g4 = lane / 16;
    const bool owner = wv < NCT;
    const int H = a.H, N = a.N, K = a.topk;
    const int SH = a.num_seqs * H;

    // ---------------- which records ----------------
    const bool shared = (int)blockIdx.x < SH;
    int s, h, part;
    int64_t lo, n, cbase;   // first record, count, first checkpoint
    if (shared) {
        const int u = blockIdx.x;
        s = u / H;
        h = u % H;
        part = N;
        lo = a.cu[s];
        n = a.cu[s + 1] - lo;
        cbase = ((int64_t)a.cu[s] * H + (int64_t)h * n) / kBC + 2 * (int64_t)u;
    } else {
        const int g = blockIdx.x - SH;
        part = g % N;
        s = g / N / H;
        h = g / N % H;
        lo = a.seg_offsets[g];
        n = a.seg_offsets[g + 1] - lo;
        cbase = a.ckpt_shared_chunks + lo / kBC + 2 * (int64_t)g;
    }
    const int64_t nchunks = (n + kBC - 1) / kBC;
    const int64_t sbase = (((int64_t)s * H + h) * (N + 1) + part) * CK * DV;
    const TIn* __restrict__ gq = static_cast<const TIn*>(a.q);
    const TIn* __restrict__ gk = static_cast<const TIn*>(a.kl);
    const TIn* __restrict__ gv = static_cast<const TIn*>(a.v);
    const TIn* __restrict__ gl = static_cast<const TIn*>(a.la);

    // register tiles (rt, ct = wv + 4 u): lane holds rows 16 rt + drow(g4, i)
    // and column 16 ct + l16
    auto tile_row = [&](int rt, int i) { return 16 * rt + drow(g4, i); };
    auto tile_col = [&](int u) { return 16 * (wv + kBW * u) + l16; };
    auto ckpt = [&](int64_t ci) { return a.ckpt + (cbase + ci) * (int64_t)(CK * DV); };
    auto store_state = [&](float* dst, const f32x4b (&X)[RT][CTW]) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int u = 0; u < CTW; u++)
#pragma unroll
                for (int i = 0; i < 4; i++) dst[tile_row(rt, i) * DV + tile_col(u)] = X[rt][u][i];
    };
    auto load_state = [&](const float* src, f32x4b (&X)[RT][CTW]) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int u = 0; u < CTW; u++)
#pragma unroll
                for (int i = 0; i < 4; i++) X[rt][u][i] = src[tile_row(rt, i) * DV + tile_col(u)];
    };

    // ---------------- per-chunk records and rows ----------------
    auto meta = [&](int64_t c) {
        if (tid < kBC) {
            const int64_t idx = c * kBC + tid;
            const bool valid = idx < n;
            const int64_t ci = valid ? idx : n - 1;   // a real row for padded records
            uint32_t row, slot;
            float w;
            if (shared) {
                row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
                slot = row * (uint32_t)(K + 1) + (uint32_t)K;
                w = 1.f;
            } else {
                const SegRec r = a.seg_rec[lo + ci];
                row = r.row;
                slot = row * (uint32_t)(K + 1) + r.orow % (uint32_t)K;
                w = r.w;
            }
            sm.row[tid] = row;
            sm.slot[tid] = slot;
            sm.w[tid] = valid ? w : 0.f;
            sm.valid[tid] = valid;
        }
    };
    // rows into LDS (fp32); padded records: no decay, no key, no gradient
    auto load_rows = [&](bool with_q) {
        for (int e = tid; e < kBC * CK; e += kBThreads) {
            const int r = e / CK, j = e % CK;
            const int64_t off = (int64_t)sm.row[r] * CK + j;
            const bool valid = sm.valid[r] != 0;
            if (with_q) sm.qt[r][j] = to_f32(gq[off]);
            sm.k0[r][j] = to_f32(gk[off]);
            sm.bb[r][j] = valid ? to_f32(gl[off]) : 0.f;
        }
        for (int e = tid; e < kBC * DV; e += kBThreads) {
            const int r = e / DV, m = e % DV;
            const int64_t off = (int64_t)sm.row[r] * DV + m;
            sm.v[r][m] = to_f32(gv[off]);
            if (with_q) {
                const float dov = sm.valid[r] ? a.dout[off] : 0.f;
                sm.dob[r][m] = dov;
                sm.g[r][m] = sm.w[r] * dov;
            }
        }
    };
    // key normalisers (wave wv: records 4 wv .. +3), in-chunk cumulative
    // decay (thread j: state row j), then K0 (and Qt)
    auto prep = [&](bool with_q) {
#pragma unroll
        for (int rr = 0; rr < kBC / kBW; rr++) {
            const int r = (kBC / kBW) * wv + rr;
            float m = -INFINITY;
            for (int j = lane; j < CK; j += kWave) m = fmaxf(m, sm.k0[r][j]);
            m = wave_max(m);
            float z = 0.f;
            for (int j = lane; j < CK; j += kWave) z += expf(sm.k0[r][j] - m);
            z = wave_sum(z);
            if (lane == 0) sm.lnz[r] = m + logf(z);
        }
        if (tid < CK) {
            float b = 0.f;
#pragma unroll
            for (int r = 0; r < kBC; r++) {
                b += sm.bb[r][tid];
                sm.bb[r][tid] = b;
            }
            sm.ebc[tid] = expf(b);
        }
        __syncthreads();
        for (int e = tid; e < kBC * CK; e += kBThreads) {
            const int r = e / CK, j = e % CK;
            const float b = sm.bb[r][j];
            if (with_q) sm.qt[r][j] *= expf(b);
            sm.k0[r][j] = sm.valid[r] ? expf(sm.k0[r][j] - sm.lnz[r] - b) : 0.f;
        }
    };

    // ================= forward sweep: checkpoints S_in of every chunk =================
    f32x4b S[RT][CTW];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int u = 0; u < CTW; u++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                S[rt][u][i] = (owner && a.init) ? a.init[sbase + (int64_t)tile_row(rt, i) * DV + tile_col(u)] : 0.f;
    for (int64_t c = 0; c < nchunks; c++) {
        meta(c);
        __syncthreads();
        load_rows(false);
        __syncthreads();
        prep(false);
        __syncthreads();
        if (owner) {
            store_state(ckpt(c), S);
            // S = D (S + Kh^T V)
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kBW * u;
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int ks = 0; ks < kBC / 4; ks++) {
                        const int rec = 4 * ks + g4;
                        S[rt][u] = mf(sm.w[rec] * sm.k0[rec][16 * rt + l16], sm.v[rec][16 * ct + l16],
                                      S[rt][u]);
                    }
            }
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float dd = sm.ebc[tile_row(rt, i)];
#pragma unroll
                    for (int u = 0; u < CTW; u++) S[rt][u][i] *= dd;
                }
        }
        __syncthreads();
    }
    if (owner) store_state(ckpt(nchunks), S);   // the final state (S_out of the last chunk)

    // ================= reverse sweep =================
    // G: gradient of the state after the current chunk
    f32x4b G[RT][CTW];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int u = 0; u < CTW; u++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                G[rt][u][i] = (owner && a.dfinal) ? a.dfinal[sbase + (int64_t)tile_row(rt, i) * DV + tile_col(u)] : 0.f;

    // out[r][j] (partial over this wave's columns) = sum_m X[r][m] Y[j][m],
    // Y given as the wave's register tiles, X in LDS: per 16-row tile of Y,
    // the wave writes its 16 x 32 slice to xp and reads it back transposed
    auto col_contract = [&](const float (*X)[SM::VS], const f32x4b (&Y)[RT][CTW]) {
#pragma unroll
        for (int jt = 0; jt < RT; jt++) {
#pragma unroll
            for (int u = 0; u < CTW; u++)
#pragma unroll
                for (int i = 0; i < 4; i++) sm.xp[wv][drow(g4, i)][16 * u + l16] = Y[jt][u][i];
            wave_lds_sync();
            f32x4b acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kBW * u;
#pragma unroll
                for (int kk = 0; kk < 4; kk++) {
                    const int mloc = 4 * kk + g4;
                    acc = mf(X[l16][16 * ct + mloc], sm.xp[wv][l16][16 * u + mloc], acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; i++) sm.red[wv][drow(g4, i)][16 * jt + l16] = acc[i];
            wave_lds_sync();
        }
    };
    // out[r][j] over records: sum_s Mt[r][s] B[s][j] with Mt from the sum of
    // the four partial tiles P (transposed when `tr`), B[s][j] in LDS scaled
    // by the record gate when `gate` (Kh = w K0)
    auto rec_contract = [&](const float (*P)[kBC][kBC + 1], bool tr, const float (*B)[SM::KS],
                            bool gate, int jt) {
        f32x4b acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kBC / 4; ks++) {
            const int sidx = 4 * ks + g4;
            float m = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < kBW; w2++) m += tr ? P[w2][sidx][l16] : P[w2][l16][sidx];
            const float bv = B[sidx][16 * jt + l16] * (gate ? sm.w[sidx] : 1.f);
            acc = mf(m, bv, acc);
        }
        return acc;
    };

    f32x4b Sin[RT][CTW];
    for (int64_t c = nchunks - 1; c >= 0; c--) {
        meta(c);
        __syncthreads();
        load_rows(true);
        __syncthreads();
        prep(true);
        __syncthreads();
        // ---- S_in of this chunk; sum_m S_out . G (before G is rescaled) ----
        if (owner) {
            load_state(ckpt(c), Sin);
            const float* so = ckpt(c + 1);
            float part[RT][4];
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float x = 0.f;
#pragma unroll
                    for (int u = 0; u < CTW; u++)
                        x += so[tile_row(rt, i) * DV + tile_col(u)] * G[rt][u][i];
                    part[rt][i] = row_reduce<16>(x, [](float p, float q) { return p + q; });
                }
            if (l16 == 0)
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) sm.dbc[wv][tile_row(rt, i)] = part[rt][i];
            // G~ = D G
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float dd = sm.ebc[tile_row(rt, i)];
#pragma unroll
                    for (int u = 0; u < CTW; u++) G[rt][u][i] *= dd;
                }
        } else {
            for (int j = lane; j < CK; j += kWave) sm.dbc[wv][j] = 0.f;
        }
        // ---- partial A (state rows [wv CK/4, (wv+1) CK/4)) and GV (columns
        //      [wv DV/4, (wv+1) DV/4)), masked to s <= r ----
        {
            f32x4b aa = {0.f, 0.f, 0.f, 0.f}, gg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < CK / (4 * kBW); kk++) {
                const int j = wv * (CK / kBW) + 4 * kk + g4;
                aa = mf(sm.qt[l16][j], sm.w[l16] * sm.k0[l16][j], aa);
            }
#pragma unroll
            for (int kk = 0; kk < DV / (4 * kBW); kk++) {
                const int m = wv * (DV / kBW) + 4 * kk + g4;
                gg = mf(sm.g[l16][m], sm.v[l16][m], gg);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = drow(g4, i);
                sm.a[wv][r][l16] = l16 <= r ? aa[i] : 0.f;
                sm.gv[wv][r][l16] = l16 <= r ? gg[i] : 0.f;
            }
        }
        __syncthreads();
        // ---- column-owned outputs: y (for y . do) and dV ----
        if (owner) {
            float dwpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kBW * u, col = 16 * ct + l16;
                f32x4b y = {0.f, 0.f, 0.f, 0.f}, dv = {0.f, 0.f, 0.f, 0.f};
                // y = Qt S_in + A V;  dV = A^T g + Kh G~
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int j = tile_row(rt, i);
                        y = mf(sm.qt[l16][j], Sin[rt][u][i], y);
                        dv = mf(sm.w[l16] * sm.k0[l16][j], G[rt][u][i], dv);
                    }
#pragma unroll
                for (int ks = 0; ks < kBC / 4; ks++) {
                    const int sidx = 4 * ks + g4;
                    float am = 0.f, at = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < kBW; w2++) {
                        am += sm.a[w2][l16][sidx];   // A[r = l16][s]
                        at += sm.a[w2][sidx][l16];   // A^T[r = l16][s] = A[s][r]
                    }
                    y = mf(am, sm.v[sidx][col], y);
                    dv = mf(at, sm.g[sidx][col], dv);
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = drow(g4, i);
                    dwpart[i] += y[i] * sm.dob[r][col];
                    if (sm.valid[r]) a.g_dv[(int64_t)sm.slot[r] * DV + col] = dv[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float x = row_reduce<16>(dwpart[i], [](float p, float q) { return p + q; });
                if (l16 == 0) sm.dwp[wv][drow(g4, i)] = x;
            }
        } else if (lane < kBC) {
            sm.dwp[wv][lane] = 0.f;
        }
        // ---- dQt = g S_in^T (column partials) + GV Kh ----
        if (owner) col_contract(sm.g, Sin);
        __syncthreads();
        for (int jt = wv; jt < RT; jt += kBW) {
            const f32x4b cpart = rec_contract(sm.gv, false, sm.k0, true, jt);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = drow(g4, i), j = 16 * jt + l16;
                float x = cpart[i];
#pragma unroll
                for (int w2 = 0; w2 < kBW; w2++)
                    if (w2 < NCT) x += sm.red[w2][r][j];
                sm.dqt[r][j] = x;
            }
        }
        __syncthreads();
        // ---- dKh = V G~^T (column partials) + GV^T Qt ----
        if (owner) col_contract(sm.v, G);
        __syncthreads();
        for (int jt = wv; jt < RT; jt += kBW) {
            const f32x4b cpart = rec_contract(sm.gv, true, sm.qt, false, jt);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = drow(g4, i), j = 16 * jt + l16;
                float x = cpart[i];
#pragma unroll
                for (int w2 = 0; w2 < kBW; w2++)
                    if (w2 < NCT) x += sm.red[w2][r][j];
                sm.dkh[r][j] = x;
            }
        }
        // ---- G = G~ + Qt^T g (gradient of S_in: G of the previous chunk) ----
        if (owner) {
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int col = tile_col(u);
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int ks = 0; ks < kBC / 4; ks++) {
                        const int rec = 4 * ks + g4;
                        G[rt][u] = mf(sm.qt[rec][16 * rt + l16], sm.g[rec][col], G[rt][u]);
                    }
            }
        }
        __syncthreads();
        // ---- K0 . dKh per record (wave wv: records 4 wv .. +3) ----
#pragma unroll
        for (int rr = 0; rr < kBC / kBW; rr++) {
            const int r = (kBC / kBW) * wv + rr;
            float x = 0.f;
            for (int j = lane; j < CK; j += kWave) x += sm.k0[r][j] * sm.dkh[r][j];
            x = wave_sum(x);
            if (lane == 0) sm.dww[r] = x;
        }
        __syncthreads();
        // ---- per record and state row: dq, key-logit gradient, dlog_alpha
        //      (reverse cumulative sum over the chunk), and dw ----
        if (tid < CK) {
            const int j = tid;
            float dbc = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < kBW; w2++) dbc += sm.dbc[w2][j];
            float run = dbc;   // the chunk decay acts at its last record
#pragma unroll
            for (int r = kBC - 1; r >= 0; r--) {
                const float b = sm.bb[r][j], w = sm.w[r];
                const float dqt = sm.dqt[r][j], dkh = sm.dkh[r][j];
                run += sm.qt[r][j] * dqt - w * sm.k0[r][j] * dkh;
                if (sm.valid[r]) {
                    const int64_t o = (int64_t)sm.slot[r] * CK + j;
                    const float kap = sm.k0[r][j] * expf(b);
                    // dkappa = w e^{-b} dKh; kappa . dkappa = w (K0 . dKh)
                    const float dkap = w * expf(-b) * dkh;
                    a.g_dq[o] = dqt * expf(b);
                    a.g_dkl[o] = kap * (dkap - w * sm.dww[r]);
                    a.g_dla[o] = run;
                }
            }
        }
        if (tid >= CK && tid < CK + kBC) {
            const int r = tid - CK;
            if (sm.valid[r]) {
                float x = sm.dww[r];
#pragma unroll
                for (int w2 = 0; w2 < kBW; w2++) x += sm.dwp[w2][r];
                a.g_dw[sm.slot[r]] = x;
            }
        }
        __syncthreads();
    }
    // gradient of the segment's initial state
    if (owner && a.dinit) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int u = 0; u < CTW; u++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    a.dinit[sbase + (int64_t)tile_row(rt, i) * DV + tile_col(u)] = G[rt][u][i];
    }
}

// Per (token, head): sum the k + 1 slots of every gradient; the router
// logits' gradient through e = softmax(z): dz = e * (de - e . de) with de
// the gate gradients of the k chosen partitions (zero elsewhere).
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_combine_kernel(const BwdArgs a, int c, int d,
                                                         int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x;   // one block per (token, head)
    if (row >= rows) return;
    const int K = a.topk, N = a.N, P = K + 1;
    const int64_t sb = row * P;
    for (int j = threadIdx.x; j < c; j += blockDim.x) {
        float q = 0.f, k = 0.f, l = 0.f;
        for (int p = 0; p < P; p++) {
            q += a.g_dq[(sb + p) * c + j];
            k += a.g_dkl[(sb + p) * c + j];
            l += a.g_dla[(sb + p) * c + j];
        }
        a.dq[row * c + j] = q;
        a.dkl[row * c + j] = k;
        a.dla[row * c + j] = l;
    }
    for (int m = threadIdx.x; m < d; m += blockDim.x) {
        float x = 0.f;
        for (int p = 0; p < P; p++) x += a.g_dv[(sb + p) * d + m];
        a.dv[row * d + m] = x;
    }
    if (threadIdx.x < kWave) {
        // router softmax over N (one wave; N <= 64)
        const int lane = threadIdx.x;
        const TIn* z = static_cast<const TIn*>(a.z);
        const float zi = lane < N ? to_f32(z[row * N + lane]) : -INFINITY;
        const float zm = wave_max(zi);
        const float ex = lane < N ? expf(zi - zm) : 0.f;
        const float e = ex / wave_sum(ex);
        float de = 0.f;
        for (int p = 0; p < K; p++)
            if (a.sel_idx[row * K + p] == lane) de = a.g_dw[sb + p];
        const float ede = wave_sum(e * de);
        if (lane < N) a.dz[row * N + lane] = e * (de - ede);
    }
}

namespace {

template <int CK, int DV, typename TIn>
void launch_bwd_cfg(const BwdArgs& a, hipStream_t st) {
    const unsigned grid = (unsigned)((int64_t)a.num_seqs * a.H * (a.N + 1));
    if (grid == 0) return;
    bwd_kernel<CK, DV, TIn><<<grid, kBThreads, 0, st>>>(a);
}

template <typename TIn>
bool launch_bwd_shape(const BwdArgs& a, int c, int d, hipStream_t st) {
#define SSE_BWD_CASE(CC, DD)                     \
    if (c == CC && d == DD) {                    \
        launch_bwd_cfg<CC, DD, TIn>(a, st);      \
        return true;                             \
    }
    SSE_BWD_CASE(32, 32) SSE_BWD_CASE(32, 64) SSE_BWD_CASE(32, 128)
    SSE_BWD_CASE(64, 32) SSE_BWD_CASE(64, 64) SSE_BWD_CASE(64, 128)
    SSE_BWD_CASE(128, 32) SSE_BWD_CASE(128, 64) SSE_BWD_CASE(128, 128)
#undef SSE_BWD_CASE
    return false;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, int dtype, int c, int d, hipStream_t st) {
    if ((int64_t)a.num_seqs * a.H == 0) return hipSuccess;
    const bool ok = dtype == kF32 ? launch_bwd_shape<float>(a, c, d, st)
                                  : launch_bwd_shape<bf16_t>(a, c, d, st);
    if (!ok) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.rows == 0) return hipSuccess;
    if (dtype == kF32)
        bwd_combine_kernel<float><<<(unsigned)a.rows, 256, 0, st>>>(a, c, d, a.rows);
    else
        bwd_combine_kernel<bf16_t><<<(unsigned)a.rows, 256, 0, st>>>(a, c, d, a.rows);
    return hipGetLastError();
}

}  // namespace sse
