// chunk_f64.hip -- chunked gated linear attention over partition segments for
// fp32 inputs on gfx950: every value after the load is fp64.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记".
// A routed partition's state moves only on the records that select it (§2.6:
// identity transition elsewhere; §2.4: each partition keeps its own clock), so
// each (sequence, head, partition) segment is a gated linear attention (§2.1
// eq. 6, diagonal decay) over its own records, with the router probability w
// gating the write and the read (§2.3, eqs. 12-14).  The shared partition
// (§2.5) is the segment of all tokens of a sequence with w = 1.
//
// Chunked form over C records r = 0..C-1, b_r = sum_{u<=r} log_alpha_u (per
// state row, within the chunk), b_C the chunk total:
//   Qt[r,j] = q[r,j] e^{b[r,j]},  Kh[s,j] = w_s kappa[s,j] e^{-b[s,j]}
//   A[r,s]  = (Qt Kh^T)[r,s] for s <= r, else 0     (the own write is read)
//   O       = A V + Qt S_in,  read = w_r O_r
//   S_out   = diag(e^{b_C}) (S_in + Kh^T V)
// which is the token recurrence unrolled over the chunk.
//
// Precision: fp32 inputs carry a parity bar of 1e-5 of the output rms, a few
// fp32 ulps.  Here the key softmax (max-shifted, per record), the cumulative
// decay, the exponentials (library fp64 exp) and every contraction (fp64
// MFMA, 16x16x4) run in fp64, and the state stays fp64 for the whole segment;
// the outputs are rounded to fp32 once.  The routed reads reach the shared
// pass through fp32 slots (one more rounding each), which the shared pass adds
// in fp64 before its single rounding of o.
//
// Block = 4 waves, one segment (routed) or one (sequence, head) chain
// (shared), chunks of 16 records.  Per chunk: the rows are loaded into LDS as
// fp64; each wave computes the key normalisers of 4 records, the first c
// threads run the cumulative decay of one state row each; the decayed
// operands replace the raw rows in LDS; each wave adds the product of its
// quarter of the state rows to A (four partial tiles, summed when read); the
// waves that own 16-column tiles of the state compute O = Qt S_in,
// S += Kh^T V, the decay, then O += A V, and store the gated reads.
#include "chunk_common.h"

namespace sse {

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kFC = 16;           // records per chunk
constexpr int kFW = 4;            // waves per block
constexpr int kFThreads = kFW * kWave;

// 16x16x4 fp64 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16]; the
// output gives lane l column l%16 and rows l/16 + 4 i, i = 0..3 (measured on
// gfx950; the fp32 and bf16 16x16 forms give rows 4 (l/16) + i instead).
__device__ __forceinline__ f64x4 mfma64(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int CK, int DV>
struct F64Smem {
    static constexpr int KS = CK + 1, VS = DV + 1;  // odd strides: 16 rows, 16 bank pairs
    double q[kFC][KS];       // q, then Qt
    double k[kFC][KS];       // key logits, then Kh
    double l[kFC][KS];       // log decay, then its in-chunk cumulative sum
    double v[kFC][VS];
    double a[kFW][kFC][kFC + 1];  // partial A tiles (one per wave's row quarter)
    double ebc[CK];          // e^{b_C} per state row
    double lnz[kFC];         // key-softmax normaliser per record
    double ww[kFC];          // write gate (0: the record writes nothing)
    double wr[kFC];          // read gate
    uint32_t row[kFC];       // input row t*H + h
    uint32_t orow[kFC];      // output row (slot row or o row)
    int dec[kFC];            // the record decays the state (it is a write)
    int rd[kFC];             // the record is read (its gated read is stored)
};

}  // namespace

template <int CK, int DV, int MODE>
__global__ __launch_bounds__(kFThreads, 1) void chunk_f64_kernel(const ChunkArgs a) {
    using SM = F64Smem<CK, DV>;
    constexpr int KS = SM::KS, VS = SM::VS;
    constexpr int RT = CK / 16;             // 16-row tiles of the state
    constexpr int NCT = DV / 16;            // 16-column tiles of the state
    constexpr int CTW = NCT >= kFW ? NCT / kFW : 1;   // column tiles per owning wave
    static_assert(MODE == kModeRouted || MODE == kModeShared || MODE == kModeMasked,
                  "routed, shared and masked passes");
    __shared__ SM sm;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, g4 = lane / 16;
    const bool owner = wv < NCT;             // owns column tiles wv, wv + 4, ...
    const int H = a.H, N = a.N;

    int s, h, part;
    int64_t lo, n;
    if constexpr (MODE != kModeShared) {
        const int g = blockIdx.x;
        part = g % N;
        s = g / N / H;
        h = g / N % H;
        if constexpr (MODE == kModeRouted) {
            lo = a.seg_offsets[g];
            n = a.seg_offsets[g + 1] - lo;
        } else {
            lo = a.cu[s];
            n = a.cu[s + 1] - lo;
        }
    } else {
        const int sh = blockIdx.x;
        s = sh / H;
        h = sh % H;
        part = N;
        lo = a.cu[s];
        n = a.cu[s + 1] - lo;
    }
    const int64_t sbase = (((int64_t)s * H + h) * (N + 1) + part) * CK * DV;
    const float* __restrict__ gq = static_cast<const float*>(a.q);
    const float* __restrict__ gk = static_cast<const float*>(a.kl);
    const float* __restrict__ gv = static_cast<const float*>(a.v);
    const float* __restrict__ gl = static_cast<const float*>(a.la);

    // state tiles (rt, ct = wv + 4 u): lane holds rows 16 rt + g4 + 4 i,
    // column 16 ct + l16
    f64x4 S[RT][CTW];
#pragma unroll
    for (int rt = 0; rt < RT; rt++)
#pragma unroll
        for (int u = 0; u < CTW; u++) {
            const int ct = wv + kFW * u;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int row = 16 * rt + g4 + 4 * i, col = 16 * ct + l16;
                S[rt][u][i] = (owner && a.init) ? (double)a.init[sbase + (int64_t)row * DV + col] : 0.0;
            }
        }

    const int64_t nchunks = (n + kFC - 1) / kFC;
    for (int64_t c = 0; c < nchunks; c++) {
        // ---- records of this chunk ----
        if (tid < kFC) {
            const int64_t idx = c * kFC + tid;
            const bool valid = idx < n;
            const int64_t ci = valid ? idx : n - 1;   // a real row for padded records
            uint32_t row, orow;
            double ww = 0.0, wr = 0.0;
            bool wrt = valid, rdd = valid;
            if constexpr (MODE == kModeRouted) {
                const SegRec r = a.seg_rec[lo + ci];
                row = r.row;
                orow = r.orow;
                ww = wr = r.w;
            } else if constexpr (MODE == kModeMasked) {
                // token lo + ci: written if the partition is in its write
                // set, read if it is in its read set (slot = read rank)
                row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
                wrt = rdd = false;
                int jr = 0;
                for (int j = 0; j < a.sel_k; j++)
                    if (a.sel_idx[row * (uint32_t)a.sel_k + j] == part) {
                        wrt = valid;
                        ww = a.sel_w[row * (uint32_t)a.sel_k + j];
                    }
                for (int j = 0; j < a.rd_k; j++)
                    if (a.rd_idx[row * (uint32_t)a.rd_k + j] == part) {
                        rdd = valid;
                        wr = a.rd_w[row * (uint32_t)a.rd_k + j];
                        jr = j;
                    }
                orow = row * (uint32_t)a.rd_k + (uint32_t)jr;
            } else {
                row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
                orow = row;
                ww = wr = 1.0;
            }
            sm.row[tid] = row;
            sm.orow[tid] = orow;
            sm.ww[tid] = wrt ? ww : 0.0;
            sm.wr[tid] = wr;
            sm.dec[tid] = wrt;
            sm.rd[tid] = rdd;
        }
        __syncthreads();
        // ---- raw rows as fp64 (records that do not write: no decay; their
        //      key is zeroed below) ----
        for (int e = tid; e < kFC * CK; e += kFThreads) {
            const int r = e / CK, j = e % CK;
            const int64_t off = (int64_t)sm.row[r] * CK + j;
            sm.q[r][j] = (double)gq[off];
            sm.k[r][j] = (double)gk[off];
            sm.l[r][j] = sm.dec[r] ? (double)gl[off] : 0.0;
        }
        for (int e = tid; e < kFC * DV; e += kFThreads) {
            const int r = e / DV, m = e % DV;
            sm.v[r][m] = (double)gv[(int64_t)sm.row[r] * DV + m];
        }
        __syncthreads();
        // ---- key normalisers (wave wv: records 4 wv .. 4 wv + 3) and the
        //      in-chunk cumulative decay (thread j: state row j) ----
#pragma unroll
        for (int rr = 0; rr < kFC / kFW; rr++) {
            const int r = (kFC / kFW) * wv + rr;
            double m = -INFINITY;
            for (int j = lane; j < CK; j += kWave) m = fmax(m, sm.k[r][j]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, kWave));
            double z = 0.0;
            for (int j = lane; j < CK; j += kWave) z += exp(sm.k[r][j] - m);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o, kWave);
            if (lane == 0) sm.lnz[r] = m + log(z);
        }
        if (tid < CK) {
            double b = 0.0;
#pragma unroll
            for (int r = 0; r < kFC; r++) {
                b += sm.l[r][tid];
                sm.l[r][tid] = b;
            }
            sm.ebc[tid] = exp(b);
        }
        __syncthreads();
        // ---- decayed operands: Qt = q e^b, Kh = w e^{kl - lnz - b} ----
        for (int e = tid; e < kFC * CK; e += kFThreads) {
            const int r = e / CK, j = e % CK;
            const double b = sm.l[r][j];
            sm.q[r][j] = sm.q[r][j] * exp(b);
            sm.k[r][j] = sm.dec[r] ? sm.ww[r] * exp(sm.k[r][j] - sm.lnz[r] - b) : 0.0;
        }
        __syncthreads();
        // ---- partial A over state rows [wv CK/4, (wv+1) CK/4): lane gets
        //      r = g4 + 4 i, s = l16 ----
        {
            f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int kk = 0; kk < CK / (4 * kFW); kk++) {
                const int j = wv * (CK / kFW) + 4 * kk + g4;
                acc = mfma64(sm.q[l16][j], sm.k[l16][j], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = g4 + 4 * i;
                sm.a[wv][r][l16] = l16 <= r ? acc[i] : 0.0;
            }
        }
        // ---- O = Qt S_in, then S = D (S + Kh^T V) ----
        f64x4 O[CTW];
        if (owner) {
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                O[u] = f64x4{0.0, 0.0, 0.0, 0.0};
                // k-step (rt, i) runs over state rows 16 rt + g + 4 i, g = 0..3:
                // the B operand is this lane's register i of tile (rt, u)
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        O[u] = mfma64(sm.q[l16][16 * rt + g4 + 4 * i], S[rt][u][i], O[u]);
            }
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kFW * u;
#pragma unroll
                for (int rt = 0; rt < RT; rt++)
#pragma unroll
                    for (int ks = 0; ks < kFC / 4; ks++)
                        S[rt][u] = mfma64(sm.k[4 * ks + g4][16 * rt + l16],
                                          sm.v[4 * ks + g4][16 * ct + l16], S[rt][u]);
            }
#pragma unroll
            for (int rt = 0; rt < RT; rt++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const double d = sm.ebc[16 * rt + g4 + 4 * i];
#pragma unroll
                    for (int u = 0; u < CTW; u++) S[rt][u][i] *= d;
                }
        }
        __syncthreads();  // partial A tiles complete
        if (owner) {
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kFW * u;
                // O += A V: lane supplies A[r = l16][s = 4 ks + g4]
#pragma unroll
                for (int ks = 0; ks < kFC / 4; ks++) {
                    const int sidx = 4 * ks + g4;
                    const double av = sm.a[0][l16][sidx] + sm.a[1][l16][sidx] +
                                      sm.a[2][l16][sidx] + sm.a[3][l16][sidx];
                    O[u] = mfma64(av, sm.v[sidx][16 * ct + l16], O[u]);
                }
                // gated reads: record r = g4 + 4 i, column 16 ct + l16
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int r = g4 + 4 * i, col = 16 * ct + l16;
                    if (!sm.rd[r]) continue;
                    const double val = sm.wr[r] * O[u][i];
                    const uint32_t orow = sm.orow[r];
                    if constexpr (MODE != kModeShared) {
                        a.part[(int64_t)orow * DV + col] = (float)val;
                    } else {
                        double sum = val;
                        for (int jk = 0; jk < a.topk; jk++)
                            sum += (double)a.part[((int64_t)orow * a.topk + jk) * DV + col];
                        a.o[(int64_t)orow * DV + col] = (float)sum;
                    }
                }
            }
        }
        __syncthreads();  // LDS rows of this chunk are free
    }

    // ---- final state (a segment without records keeps its initial state) ----
    if (owner) {
#pragma unroll
        for (int rt = 0; rt < RT; rt++)
#pragma unroll
            for (int u = 0; u < CTW; u++) {
                const int ct = wv + kFW * u;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int row = 16 * rt + g4 + 4 * i, col = 16 * ct + l16;
                    a.final_states[sbase + (int64_t)row * DV + col] = (float)S[rt][u][i];
                }
            }
    }
}

namespace {

template <int CK, int DV, int MODE>
void launch_f64_cfg(const ChunkArgs& a, hipStream_t st) {
    const unsigned grid = (unsigned)(a.num_seqs * a.H * (MODE != kModeShared ? a.N : 1));
    if (grid == 0) return;
    chunk_f64_kernel<CK, DV, MODE><<<grid, kFThreads, 0, st>>>(a);
}

template <int MODE>
bool launch_f64_shape(const ChunkArgs& a, int c, int d, hipStream_t st) {
#define SSE_F64_CASE(CC, DD)                  \
    if (c == CC && d == DD) {                 \
        launch_f64_cfg<CC, DD, MODE>(a, st);  \
        return true;                          \
    }
    SSE_F64_CASE(32, 32) SSE_F64_CASE(32, 64) SSE_F64_CASE(32, 128)
    SSE_F64_CASE(64, 32) SSE_F64_CASE(64, 64) SSE_F64_CASE(64, 128)
    SSE_F64_CASE(128, 32) SSE_F64_CASE(128, 64) SSE_F64_CASE(128, 128)
#undef SSE_F64_CASE
    return false;
}

}  // namespace

hipError_t launch_chunk_f64(int mode, const ChunkArgs& a, int c, int d, hipStream_t st) {
    if ((int64_t)a.num_seqs * a.H == 0) return hipSuccess;
    bool ok = false;
    if (mode == kModeRouted)
        ok = launch_f64_shape<kModeRouted>(a, c, d, st);
    else if (mode == kModeShared)
        ok = launch_f64_shape<kModeShared>(a, c, d, st);
    else if (mode == kModeMasked)
        ok = launch_f64_shape<kModeMasked>(a, c, d, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---- dispatch by input type: bf16 -> the warp-specialised kernels of
// chunk_ws.hip and piece_state.hip; fp32 -> the fp64 kernel above ----
hipError_t launch_chunk_local(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    if (dtype == kF32) return hipSuccess;
    return launch_piece_state(a, c, d, st);
}
hipError_t launch_chunk_shared(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    return dtype == kF32 ? launch_chunk_f64(kModeShared, a, c, d, st)
                         : launch_chunk_ws(kModeShared, a, c, d, st);
}
hipError_t launch_chunk_routed(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    return dtype == kF32 ? launch_chunk_f64(kModeRouted, a, c, d, st)
                         : launch_chunk_ws(kModeRouted, a, c, d, st);
}
hipError_t launch_chunk_masked(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    return dtype == kF32 ? launch_chunk_f64(kModeMasked, a, c, d, st)
                         : launch_chunk_ws(kModeMasked, a, c, d, st);
}

}  // namespace sse
