// backward.hip -- gradients of the SSE forward for gfx950: two sequential
// sweeps per partition segment give the states and state gradients at the
// chunk boundaries, then every chunk's record gradients run in parallel,
// then a per-token combine.
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
// partition), chunks of C = 32 records.  In a chunk, with b the in-chunk
// inclusive cumulative log decay (per state row), D = diag(e^{b_C}),
//   Qt = q e^b,  K0 = kappa e^{-b},  Kh = w K0,  g_r = w_r do_r,
//   A  = (Qt Kh^T) masked to s <= r,  GV = (g V^T) masked to s <= r,
//   y  = Qt S_in + A V                 (the read before its gate),
//   S_out = D S_in + Kt^T V,  Kt_r = w_r kappa_r e^{b_C - b_r} (exponents <= 0),
// and, with G the gradient of the state after the chunk and G~ = D G,
//   G_in = D G + Qt^T g                (the gradient of the state before it),
//   dQt = g S_in^T + GV Kh,   dKh = V G~^T + GV^T Qt,   dV = A^T g + Kh G~,
//   db  = Qt . dQt - Kh . dKh  (per record and row),
//   t   = sum_m S_out . G = rowsum(S_in . G~) + sum_s Kh_s . (V G~^T)_s
//         (the decay of the whole chunk, through S_out),
//   dlog_alpha_r = t + sum_{u >= r in the chunk} db_u,
//   dq = dQt e^b,  dkey_logits = kappa (dkappa - kappa . dkappa) with
//   dkappa = w e^{-b} dKh,  dw = y . do + K0 . dKh  (read and write gates).
//
// Launch 1 (sweeps): one block per segment and direction.  The forward
// sweep carries S from the initial state and stores S_in of every chunk;
// the reverse sweep carries G from dS_final and stores G~ = D G of every
// chunk (the form the chunk launch uses), and its last G is the gradient of
// the segment's initial state.  A step is
// one c x C by C x d product into the carried state tiles (registers), on
// fp32 MFMA (16x16x4) for fp32 inputs and on bf16 MFMA for bf16 inputs (the
// chunk's 32 records as one k-step; the A side in two bf16 terms, the B side
// V, exact in bf16, or g in two terms).  The forward sweep also writes
// every chunk's record list (input row, gradient slot, gate, key
// normaliser) for launch 2.
// Launch 2 (chunks): every chunk's gradients from its stored S_in and G~, so
// all chunks are independent; persistent 8-wave blocks, each walking every
// G-th checkpoint slot with the next slot's records and rows prefetched;
// wave w owning
// the 16-column block w of the d-side outputs (y, dV) and the 16-row block w
// of the c-side ones (dQt, dKh).  The state operands are read straight from
// the stored states in the MFMA operand layout (rows, or transposed for the
// products that contract over d).  With fp32 inputs every product runs on
// fp32 MFMA.  With bf16 inputs every product runs on bf16 MFMA with its
// operands in two bf16 terms (V is exact in bf16), the products of the two
// low terms left out: the four over state rows or columns (Qt S_in, Kh G~,
// g S_in^T, V G~^T), the A and GV tiles, and the four over the chunk's 32
// records (A V, A^T g, GV Kh, GV^T Qt) as one k-step each, their record-
// major operands gathered by LDS transpose reads.
// Launch 3 (combine): each record's gradients went to its own slot [token,
// head, rank] (rank = its place in the token's top-k list, k for the shared
// partition); one wave per (token, head) sums the token's k + 1 slots and
// applies the router softmax Jacobian.  No atomics: every run gives the
// same bits.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "chunk_common.h"

namespace sse {

namespace {

typedef float f32x4b __attribute__((ext_vector_type(4)));

constexpr int kBC = kBwdChunk;     // records per chunk
// waves of a sweep block: 8, or one per 16x16 state tile when fewer
template <int CK, int DV>
constexpr int sweep_waves() { return (CK / 16) * (DV / 16) < 8 ? (CK / 16) * (DV / 16) : 8; }
constexpr int kCW = 8;             // waves of a chunk block

// Row stride (floats) of the LDS operand arrays.  MFMA operands are read
// two ways: lane (l16, g4) reads row l16 and column g4 (A operands), or row
// g4 and column l16 (B operands).  A stride of 34 modulo 64 banks puts the
// 32 lanes of each half-wave on distinct banks in both patterns.
constexpr int lds_stride(int n) { return n + (n % 64 == 0 ? 34 : 2); }
static_assert(lds_stride(32) % 2 == 0 && lds_stride(64) % 2 == 0 && lds_stride(128) % 2 == 0,
              "even row strides: every row of an LDS operand array is 8-byte aligned");

// 16x16x4 fp32 MFMA: lane l supplies A[l%16][l/16] and B[l/16][l%16]; the
// output gives lane l column l%16 and rows 4 (l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4b mf(float a, float b, f32x4b c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One segment of the backward: the shared chain of unit u < S*H, or routed
// segment g = u - S*H (partition g % N of unit g / N).
struct Seg {
    int s, h, part;
    bool shared;
    int64_t lo, n;      // first record (token of a shared chain, grouping record
                        // of a routed segment) and record count
    int64_t base;       // checkpoint slot of its first chunk
    int64_t sbase;      // offset of its c x d state in [S, H, N+1, c, d]
};

template <int CK, int DV>
__device__ __forceinline__ Seg seg_of(const BwdArgs& a, int u) {
    Seg q;
    const int H = a.H, N = a.N, SH = a.num_seqs * H;
    if (u < SH) {
        q.s = u / H;
        q.h = u % H;
        q.part = N;
        q.shared = true;
        const int64_t t0 = a.cu[q.s];
        q.n = a.cu[q.s + 1] - t0;
        q.lo = t0;
        // shared chains numbered in a record space of their own: chain (s, h)
        // holds records [cu[s] H + h len_s, cu[s] H + (h + 1) len_s)
        q.base = bwd_slot_base(t0 * H + (int64_t)q.h * q.n, u);
    } else {
        const int g = u - SH;
        q.part = g % N;
        q.s = g / N / H;
        q.h = g / N % H;
        q.shared = false;
        q.lo = a.seg_offsets[g];
        q.n = a.seg_offsets[g + 1] - q.lo;
        q.base = a.sh_slots + bwd_slot_base(q.lo, g);
    }
    q.sbase = (((int64_t)q.s * H + q.h) * (N + 1) + q.part) * CK * DV;
    return q;
}

// Record r of segment q (r < n): input row t*H + h, gate w, gradient slot row.
struct Rec {
    uint32_t row, slot;
    float w;
};
__device__ __forceinline__ Rec rec_of(const BwdArgs& a, const Seg& q, int64_t r) {
    Rec x;
    const uint32_t K = (uint32_t)a.topk;
    if (q.shared) {
        x.row = (uint32_t)(q.lo + r) * (uint32_t)a.H + (uint32_t)q.h;
        x.slot = x.row * (K + 1) + K;
        x.w = 1.f;
    } else {
        const SegRec s = a.seg_rec[q.lo + r];
        x.row = s.row;
        x.slot = s.row * (K + 1) + s.orow % K;
        x.w = s.w;
    }
    return x;
}

// 8 consecutive elements of a row, loaded with 16-byte loads.
template <typename T>
struct Row8;
template <>
struct Row8<bf16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = i < 2 ? u.x : i < 4 ? u.y : i < 6 ? u.z : u.w;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <>
struct Row8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ float get(int i) const {
        const float4& h = i < 4 ? a : b;
        const int k = i & 3;
        return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    }
};

template <int CK, int DV>
struct SwSmem {
    static constexpr int KS = lds_stride(CK), VS = lds_stride(DV);
    float x[kBC][KS];        // A side: Kt (forward) or Qt (reverse)
    float la[kBC][KS];       // log decay, then its in-chunk sums
    float y[kBC][VS];        // B side: V (forward) or g = w do (reverse)
    float ebc[CK];           // e^{b_C}
    float btot[sweep_waves<CK, DV>() * kWave / CK][CK];   // per record group: its log decay total
    // bf16 inputs: the A side transposed [state row][record] in two bf16
    // terms (rows of 80 bytes: 16-byte aligned operand reads, and the 16
    // rows one read touches fall on distinct banks)
    alignas(16) uint16_t xh[CK][kBC + 8];
    alignas(16) uint16_t xl[CK][kBC + 8];
    // metadata of three chunks (the current one and the two ahead)
    float lnz[3][kBC];       // key normalisers (log2)
    float w[3][kBC];
    uint32_t row[3][kBC];
    int valid[3][kBC];
};

}  // namespace

// Blocks [0, 2 SH) run the shared chains (u < SH = sequences x heads),
// forward then reverse; blocks [2 SH, 2 NSEG) the routed segments, forward
// then reverse.
template <int CK, int DV, typename TIn>
__global__ __launch_bounds__((sweep_waves<CK, DV>() * kWave)) void bwd_sweep_kernel(const BwdArgs a) {
    using SM = SwSmem<CK, DV>;
    constexpr int kSW = sweep_waves<CK, DV>();
    constexpr int CT = DV / 16;
    constexpr int NTILE = (CK / 16) * CT;
    constexpr int TPW = NTILE / kSW;               // state tiles per wave
    static_assert(NTILE % kSW == 0, "every wave owns the same number of tiles");
    constexpr bool kBf = std::is_same<TIn, bf16_t>::value;   // bf16 MFMA for the products
    __shared__ SM sm;

    // Blocks are dispatched in index order: the shared chains (the longest
    // segments, every token of a sequence) come first in both directions,
    // so that they run beside the routed segments instead of after them
    const int nseg = a.num_seqs * a.H * (a.N + 1);
    const int SH = a.num_seqs * a.H, nrt = nseg - SH;
    const int b = (int)blockIdx.x;
    const bool rev = b < 2 * SH ? b >= SH : b - 2 * SH >= nrt;
    const int u = b < 2 * SH ? b % SH : SH + (b - 2 * SH) % nrt;
    const Seg q = seg_of<CK, DV>(a, u);
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, g4 = lane / 16;
    const int64_t nch = (q.n + kBC - 1) / kBC;
    const TIn* __restrict__ gq = static_cast<const TIn*>(a.q);
    const TIn* __restrict__ gk = static_cast<const TIn*>(a.kl);
    const TIn* __restrict__ gv = static_cast<const TIn*>(a.v);
    const TIn* __restrict__ gl = static_cast<const TIn*>(a.la);

    // the slots after this segment's chunks, up to the next segment's first
    // slot, hold no chunk: the forward sweep marks them (the chunk launch
    // skips a slot whose first record is marked)
    if (!rev) {
        const int64_t next = u + 1 < nseg ? seg_of<CK, DV>(a, u + 1).base : a.nslot;
        for (int64_t x = q.base + nch + tid; x < next; x += kSW * kWave)
            a.slot_meta[x * kBC] = BwdRec{0u, kNoSlot, 0.f, 0.f};
    }

    // both directions as one body with the direction fixed at compile time
    auto sweep = [&](auto revC) {
        constexpr bool REV = decltype(revC)::value;
        // state tiles of this wave: tile t = wv + kSW i holds rows
        // 16 (t / CT) + 4 g4 + e and column 16 (t % CT) + l16
        f32x4b X[TPW];
        const float* src0 = REV ? a.dfinal : a.init;
#pragma unroll
        for (int i = 0; i < TPW; i++) {
            const int t = wv + kSW * i;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                float v0 = 0.f;
                if (src0)
                    v0 = src0[q.sbase + (int64_t)(16 * (t / CT) + 4 * g4 + e) * DV + 16 * (t % CT) + l16];
                X[i][e] = v0;
            }
        }

        // Pipelined over chunks: the record list of chunk ci + 3 and the rows
        // of chunk ci + 2 are loaded while chunk ci is prepared and multiplied
        // (the rows into the register set chunk ci's rows just left).
        constexpr int NT = kSW * kWave;
        static_assert(kBC * CK / 8 <= NT && kBC * DV / 8 <= NT, "one 8-element piece per thread");
        auto order = [&](int64_t ci) { return REV ? nch - 1 - ci : ci; };
        // a chunk's record list: loaded into registers one step before it
        // is written to LDS, so no barrier waits for those loads
        Rec mx = {0u, 0u, 0.f};
        float mlz = 0.f;
        bool mvalid = false;
        auto meta_load = [&](int64_t ci) {
            if (tid < kBC) {
                const int64_t r = order(ci) * kBC + tid;
                mvalid = r < q.n;
                mx = rec_of(a, q, mvalid ? r : q.n - 1);
                mlz = a.lnz2[mx.row];
            }
        };
        auto meta_store = [&](int64_t ci) {
            if (tid < kBC) {
                const int p = (int)(ci % 3);
                sm.row[p][tid] = mx.row;
                sm.w[p][tid] = mvalid ? mx.w : 0.f;
                sm.valid[p][tid] = mvalid;
                sm.lnz[p][tid] = mlz;
                // the forward sweep also writes the chunk's record list for
                // the chunk launch
                if (!REV)
                    a.slot_meta[(q.base + order(ci)) * kBC + tid] =
                        BwdRec{mx.row, mvalid ? mx.slot : kNoSlot, mvalid ? mx.w : 0.f, mlz};
            }
        };
        auto meta = [&](int64_t ci) {
            meta_load(ci);
            meta_store(ci);
        };
        // this thread's 8-element pieces (key side: record rk, columns jk..;
        // value side: record rv, columns mv..): forward key logits, log
        // decay, v; reverse q, log decay, do
        const int rk = tid / (CK / 8), jk = 8 * (tid % (CK / 8));
        const int rv = tid / (DV / 8), mv = 8 * (tid % (DV / 8));
        const bool kpiece = tid < kBC * CK / 8, vpiece = tid < kBC * DV / 8;
        Row8<TIn> px[2], pl[2], pv[2];
        Row8<float> pd[2];
        auto rows = [&](int64_t ci, auto SI) {
            constexpr int S = decltype(SI)::value;
            const int p = (int)(ci % 3);
            if (kpiece) {
                const int64_t off = (int64_t)sm.row[p][rk] * CK + jk;
                px[S].load((REV ? gq : gk) + off);
                pl[S].load(gl + off);
            }
            if (vpiece) {
                const int64_t off = (int64_t)sm.row[p][rv] * DV + mv;
                if constexpr (REV)
                    pd[S].load(a.dout + off);
                else
                    pv[S].load(gv + off);
            }
        };
        const std::integral_constant<int, 0> I0{};
        const std::integral_constant<int, 1> I1{};
        if (nch > 0) meta(0);
        if (nch > 1) meta(1);
        if (nch > 2) meta_load(2);
        __syncthreads();
        if (nch > 0) rows(0, I0);
        if (nch > 1) rows(1, I1);

        // chunk ci, its rows in register set S = ci % 2
        auto step = [&](int64_t ci, auto SI) {
            constexpr int S = decltype(SI)::value;
            const int64_t c = order(ci);
            const int p = (int)(ci % 3);
            __syncthreads();   // the previous chunk's products are done with x, y
            // padded records: no decay, no key, no output gradient
            if (kpiece) {
                const bool ok = sm.valid[p][rk] != 0;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    sm.x[rk][jk + i] = px[S].get(i);
                    sm.la[rk][jk + i] = ok ? pl[S].get(i) : 0.f;
                }
            }
            if (vpiece) {
                const float wr = sm.w[p][rv];
#pragma unroll
                for (int i = 0; i < 8; i++) sm.y[rv][mv + i] = REV ? wr * pd[S].get(i) : pv[S].get(i);
            }
            if (ci + 2 < nch) meta_store(ci + 2);
            __syncthreads();
            if (ci + 2 < nch) rows(ci + 2, SI);
            if (ci + 3 < nch) meta_load(ci + 3);
            // in-chunk sums of the log decay: forward the suffix sums
            // b_C - b_r, reverse the inclusive prefix sums b_r.  Thread
            // (group, state row j) sums the BG records of its group in
            // registers, adds the totals of the groups before it (reverse) or
            // after it (forward), and forms its records' operand values.
            {
                constexpr int NG = NT / CK, BG = kBC / NG;
                static_assert(NT % CK == 0 && kBC % NG == 0, "record groups of whole rows");
                const int jb = tid % CK, grp = tid / CK, r0 = grp * BG;
                float sl[BG];
                float run = 0.f;
                if constexpr (REV) {
#pragma unroll
                    for (int i = 0; i < BG; i++) {
                        run += sm.la[r0 + i][jb];
                        sl[i] = run;
                    }
                } else {
#pragma unroll
                    for (int i = BG - 1; i >= 0; i--) {
                        sl[i] = run;
                        run += sm.la[r0 + i][jb];
                    }
                }
                sm.btot[grp][jb] = run;
                __syncthreads();
                float other = 0.f;
                if constexpr (REV) {
                    for (int g2 = 0; g2 < grp; g2++) other += sm.btot[g2][jb];
                } else {
                    for (int g2 = grp + 1; g2 < NG; g2++) other += sm.btot[g2][jb];
                }
                if (grp == (REV ? NG - 1 : 0)) sm.ebc[jb] = expf(other + run);
                float xv[BG];
#pragma unroll
                for (int i = 0; i < BG; i++) {
                    const int r = r0 + i;
                    const float sv = other + sl[i];
                    if constexpr (REV)
                        xv[i] = sm.x[r][jb] * expf(sv);
                    else
                        xv[i] = sm.valid[p][r] ? sm.w[p][r] * __builtin_amdgcn_exp2f(
                                                                  (sm.x[r][jb] + sv) * kLog2e - sm.lnz[p][r])
                                               : 0.f;
                }
                if constexpr (kBf) {
                    static_assert(BG % 2 == 0, "record pairs");
                    uint32_t pr[BG / 2][2];
#pragma unroll
                    for (int i = 0; i < BG; i += 2) split_pair<2>(xv[i], xv[i + 1], pr[i / 2]);
                    if constexpr (BG == 8) {
                        // one 16-byte store per term: the 16 rows of a
                        // quarter-wave fall on distinct banks
                        *reinterpret_cast<uint4*>(&sm.xh[jb][r0]) = make_uint4(pr[0][0], pr[1][0], pr[2][0], pr[3][0]);
                        *reinterpret_cast<uint4*>(&sm.xl[jb][r0]) = make_uint4(pr[0][1], pr[1][1], pr[2][1], pr[3][1]);
                    } else {
#pragma unroll
                        for (int i = 0; i < BG; i += 2) {
                            *reinterpret_cast<uint32_t*>(&sm.xh[jb][r0 + i]) = pr[i / 2][0];
                            *reinterpret_cast<uint32_t*>(&sm.xl[jb][r0 + i]) = pr[i / 2][1];
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < BG; i++) sm.x[r0 + i][jb] = xv[i];
                }
            }
            __syncthreads();
            // store the carried state (S_in of chunk c, or D G with G the
            // gradient after chunk c: the only form the chunk launch uses),
            // then X = D X + x^T y
            float* ck = (REV ? a.ckG : a.ckS) + (q.base + c) * (int64_t)(CK * DV);
#pragma unroll
            for (int i = 0; i < TPW; i++) {
                const int t = wv + kSW * i;
                const int jt = t / CT, mt = t % CT;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int j = 16 * jt + 4 * g4 + e;
                    if constexpr (REV) X[i][e] *= sm.ebc[j];
                    ck[(int64_t)j * DV + 16 * mt + l16] = X[i][e];
                    if constexpr (!REV) X[i][e] *= sm.ebc[j];
                }
            }
            if constexpr (kBf) {
                // bf16 inputs: the chunk's 32 records as one bf16 k-step.  The
                // wave's tiles share one column tile, so its B operand (8
                // records of one column: V, exact in bf16, or g in two
                // terms) is read once; the A side comes pre-split.
                static_assert(kSW % CT == 0, "one column tile per wave");
                const int mt = wv % CT;
                float yv[8];
#pragma unroll
                for (int i = 0; i < 8; i++) yv[i] = sm.y[8 * g4 + i][16 * mt + l16];
                uint32_t pb[4][2];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    if constexpr (REV) {
                        split_pair<2>(yv[2 * e2], yv[2 * e2 + 1], pb[e2]);
                    } else {
                        pb[e2][0] = pack_bf16x2(yv[2 * e2], yv[2 * e2 + 1]);
                        pb[e2][1] = 0u;
                    }
                }
                const u16x8 bhi = __builtin_bit_cast(u16x8, make_uint4(pb[0][0], pb[1][0], pb[2][0], pb[3][0]));
                const u16x8 blo = __builtin_bit_cast(u16x8, make_uint4(pb[0][1], pb[1][1], pb[2][1], pb[3][1]));
#pragma unroll
                for (int i = 0; i < TPW; i++) {
                    const int jt = (wv + kSW * i) / CT;
                    const u16x8 ahi = *reinterpret_cast<const u16x8*>(&sm.xh[16 * jt + l16][8 * g4]);
                    const u16x8 alo = *reinterpret_cast<const u16x8*>(&sm.xl[16 * jt + l16][8 * g4]);
                    X[i] = mfma16(ahi, bhi, X[i]);
                    X[i] = mfma16(alo, bhi, X[i]);
                    if constexpr (REV) X[i] = mfma16(ahi, blo, X[i]);
                }
            } else {
                // k-steps outermost (not unrolled): each step's operands are
                // read once for all of the wave's tiles, and few are live at a
                // time
#pragma unroll 1
                for (int ks = 0; ks < kBC / 4; ks++) {
                    const int r = 4 * ks + g4;
#pragma unroll
                    for (int i = 0; i < TPW; i++) {
                        const int t = wv + kSW * i;
                        X[i] = mf(sm.x[r][16 * (t / CT) + l16], sm.y[r][16 * (t % CT) + l16], X[i]);
                    }
                }
            }
        };
        int64_t ci = 0;
        for (; ci + 1 < nch; ci += 2) {
            step(ci, I0);
            step(ci + 1, I1);
        }
        if (ci < nch) step(ci, I0);
        // the reverse sweep's last G is the gradient of the initial state
        if (REV && a.dinit) {
#pragma unroll
            for (int i = 0; i < TPW; i++) {
                const int t = wv + kSW * i;
#pragma unroll
                for (int e = 0; e < 4; e++)
                    a.dinit[q.sbase + (int64_t)(16 * (t / CT) + 4 * g4 + e) * DV + 16 * (t % CT) + l16] =
                        X[i][e];
            }
        }
    };
    if (rev)
        sweep(std::true_type{});
    else
        sweep(std::false_type{});
}

namespace {

template <int CK, int DV, bool BF>
struct ChSmem {
    static constexpr int KS = lds_stride(CK), VS = lds_stride(DV);
    // V: fp32 for fp32 inputs; for bf16 inputs its bf16 bits as loaded
    // (exact), in rows of 2 (DV + 8) bytes (16-byte aligned operand reads)
    using VT = typename std::conditional<BF, uint16_t, float>::type;
    static constexpr int VRS = BF ? DV + 8 : VS;
    static constexpr int NB = BF ? kBC : 1;   // rows of the bf16-only arrays
    static constexpr int NF = BF ? 1 : kBC;   // rows of the fp32-only arrays
    float qt[kBC][KS];           // Qt
    float k0[kBC][KS];           // K0
    float eb[kBC][KS];           // b, then e^b
    alignas(16) VT v[kBC][VRS];
    float g[kBC][VS];            // g = w do
    float A[NF][lds_stride(kBC)];     // A (masked), fp32 inputs
    float GV[NF][lds_stride(kBC)];    // GV (masked), fp32 inputs
    float btot[kCW * kWave / CK][CK];   // per record group: its total of the log decay
    float dwp[kCW][kBC];         // per-wave partials of y . g
    float kdp[kCW][kBC];         // per-wave partials of K0 . dKh
    // bf16 inputs: Qt and Kh = w K0 [record][state row], g [record][column]
    // in two bf16 terms (rows of 2 (n + 8) bytes, 16-byte aligned operand
    // reads)
    alignas(16) uint16_t qh[NB][CK + 8];
    alignas(16) uint16_t ql[NB][CK + 8];
    alignas(16) uint16_t kh[NB][CK + 8];
    alignas(16) uint16_t kl[NB][CK + 8];
    alignas(16) uint16_t gh[NB][DV + 8];
    alignas(16) uint16_t gl[NB][DV + 8];
    // bf16 inputs: A and GV (masked) [record r][record s] in two bf16 terms
    alignas(16) uint16_t ah[NB][kBC + 8];
    alignas(16) uint16_t al[NB][kBC + 8];
    alignas(16) uint16_t gvh[NB][kBC + 8];
    alignas(16) uint16_t gvl[NB][kBC + 8];
    // record lists of the current chunk and the next one
    float w[2][kBC];
    float lnz[2][kBC];
    uint32_t row[2][kBC];
    uint32_t slot[2][kBC];
};

}  // namespace

// Persistent: block b runs the checkpoint slots b, b + G, b + 2G, ... (G =
// the grid, as many blocks as are resident at once; a slot that holds no
// chunk is skipped).  Each chunk's state operands are loaded as row blocks
// first, so that their latency overlaps the record-side work, and as column
// blocks after it; the next slot's record list is loaded during the current
// chunk's row work and its rows during the current chunk's products, so a
// chunk starts with its rows at hand.
template <int CK, int DV, typename TIn>
__global__ __launch_bounds__(kCW * kWave, 1) void bwd_chunk_kernel(const BwdArgs a) {
    constexpr bool kBf = std::is_same<TIn, bf16_t>::value;   // bf16 MFMA for some products
    using SM = ChSmem<CK, DV, kBf>;
    constexpr int CT = DV / 16, RT = CK / 16;
    constexpr int NT = kCW * kWave;
    constexpr int NKC = CK / 4, NKD = DV / 4;
    static_assert(CT <= kCW && RT <= kCW, "one column and one row block per wave");
    static_assert(kBC * CK / 8 <= NT && kBC * DV / 8 <= NT, "one 8-element piece per thread");
    static_assert(DV % 32 == 0, "column quarters of whole 8-column pieces");
    static_assert(CK % 32 == 0, "row quarters of whole 8-row k-steps");
    __shared__ SM sm;
    const TIn* __restrict__ gq = static_cast<const TIn*>(a.q);
    const TIn* __restrict__ gk = static_cast<const TIn*>(a.kl);
    const TIn* __restrict__ gv = static_cast<const TIn*>(a.v);
    const TIn* __restrict__ gl = static_cast<const TIn*>(a.la);
    Row8<TIn> pq, pk, pl, pv;
    Row8<float> pd;
    const int64_t G = gridDim.x;
    int cur = 0;        // record list of the current slot
    bool have = false;  // its records are in LDS and its rows on their way
    for (int64_t x = blockIdx.x; x < a.nslot; x += G) {
    // the LDS struct through an opaque offset (zero) per slot, so that the
    // compiler computes the operand addresses inside the iteration instead of
    // hoisting all of them out of the loop and holding them in registers
    int zo;
    asm volatile("s_mov_b32 %0, 0" : "=s"(zo));
    SM& sl = *reinterpret_cast<SM*>(reinterpret_cast<char*>(&sm) + zo);
    // the thread's indices through the same offset, for the same reason
    const int tid = (int)threadIdx.x + zo, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int l16 = lane % 16, g4 = lane / 16;
    // bf16 MFMA operand over records from a record-major bf16 tile (row
    // stride `stride` elements): lane (l16, g4) gets records 8 g4 + 0..7 of
    // column c0 + l16, by two transpose reads; source lane 4 e + b of each
    // 16-lane group addresses columns c0 + 4 b .. + 3 of record 8 g4 + e (+ 4)
    auto tr16 = [&](const uint16_t* tile, int stride, int c0) {
        const int r = 8 * g4 + l16 / 4, c = c0 + 4 * (l16 % 4);
        return cat_tr(lds_tr(tile + r * stride + c), lds_tr(tile + (r + 4) * stride + c));
    };
    // this thread's 8-element pieces of the chunk's rows: q, key logits and
    // log decay of record rk, columns jk..; v and do of record rv, columns mv..
    const int rk = tid / (CK / 8), jk = 8 * (tid % (CK / 8));
    const int rv = tid / (DV / 8), mv = 8 * (tid % (DV / 8));
    // V[r][m] as fp32
    auto vf = [&](int r, int m) -> float {
        if constexpr (kBf)
            return bf16_bits_to_f32(sl.v[r][m]);
        else
            return sl.v[r][m];
    };
    // record list b (0 or 1) of LDS
    auto put_records = [&](int b, const BwdRec& m) {
        sl.row[b][tid] = m.row;
        sl.slot[b][tid] = m.slot;
        sl.w[b][tid] = m.w;
        sl.lnz[b][tid] = m.lnz;
    };
    auto load_rows = [&](int b) {
        if (tid < kBC * CK / 8) {
            const int64_t off = (int64_t)sl.row[b][rk] * CK + jk;
            pq.load(gq + off);
            pk.load(gk + off);
            pl.load(gl + off);
        }
        if (tid < kBC * DV / 8) {
            const int64_t off = (int64_t)sl.row[b][rv] * DV + mv;
            pv.load(gv + off);
            pd.load(a.dout + off);
        }
    };
    if (!have) {
        if (tid < kBC) put_records(cur, a.slot_meta[x * kBC + tid]);
        __syncthreads();
        if (sl.slot[cur][0] == kNoSlot) {  // uniform: no chunk here
            __syncthreads();
            continue;
        }
        load_rows(cur);
    }
    const int64_t xn = x + G;

    // ---- this wave's state operands.  Column block wv of S_in and G~ (the
    //      products that contract over state rows; loaded further down):
    //      lane (l16, g4) takes row g4 CK/4 + ks, column 16 wv + l16.  Row block
    //      wv (the products that contract over columns; any order of the
    //      columns will do): lane (l16, g4) takes row 16 wv + l16 and the
    //      columns g4 DV/4 + ks, so each lane reads one contiguous quarter row
    //      with 16-byte loads.
    const float* __restrict__ Sin = a.ckS + x * (int64_t)(CK * DV);
    const float* __restrict__ Gc = a.ckG + x * (int64_t)(CK * DV);
    float sc[NKC], gc[NKC], sr[NKD], gr[NKD];
    if (wv < RT) {
        const float4* s4 = reinterpret_cast<const float4*>(Sin + (int64_t)(16 * wv + l16) * DV + g4 * NKD);
        const float4* g4p = reinterpret_cast<const float4*>(Gc + (int64_t)(16 * wv + l16) * DV + g4 * NKD);
#pragma unroll
        for (int i = 0; i < NKD / 4; i++) {
            const float4 u = s4[i], w4 = g4p[i];
            sr[4 * i] = u.x; sr[4 * i + 1] = u.y; sr[4 * i + 2] = u.z; sr[4 * i + 3] = u.w;
            gr[4 * i] = w4.x; gr[4 * i + 1] = w4.y; gr[4 * i + 2] = w4.z; gr[4 * i + 3] = w4.w;
        }
    }

    // ---- the chunk's rows (8-element pieces) into LDS: Qt, K0 and b start
    //      as q, key logits and log decay; padded records have no decay, key
    //      or output gradient
    {
        if (tid < kBC * CK / 8) {
            const bool ok = sl.slot[cur][rk] != kNoSlot;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                sl.qt[rk][jk + i] = pq.get(i);
                sl.k0[rk][jk + i] = pk.get(i);
                sl.eb[rk][jk + i] = ok ? pl.get(i) : 0.f;
            }
        }
        if (tid < kBC * DV / 8) {
            const float wr = sl.w[cur][rv];
            float gg[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                gg[i] = wr * pd.get(i);
                sl.g[rv][mv + i] = gg[i];
            }
            if constexpr (kBf) {
                *reinterpret_cast<uint4*>(&sl.v[rv][mv]) = pv.u;
                uint32_t pr[4][2];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) split_pair<2>(gg[2 * e2], gg[2 * e2 + 1], pr[e2]);
                *reinterpret_cast<uint4*>(&sl.gh[rv][mv]) = make_uint4(pr[0][0], pr[1][0], pr[2][0], pr[3][0]);
                *reinterpret_cast<uint4*>(&sl.gl[rv][mv]) = make_uint4(pr[0][1], pr[1][1], pr[2][1], pr[3][1]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; i++) sl.v[rv][mv + i] = pv.get(i);
            }
        }
    }
    __syncthreads();
    // the next slot's record list (written to LDS after the decay scan)
    BwdRec mnext{};
    if (tid < kBC && xn < a.nslot) mnext = a.slot_meta[xn * kBC + tid];
    // inclusive in-chunk cumulative log decay b: thread (group, state row j)
    // scans the BG records of its group in registers, then adds the totals
    // of the groups before it; the same thread forms Qt, K0 and e^b of its
    // records
    {
        constexpr int NG = NT / CK, BG = kBC / NG;
        static_assert(NT % CK == 0 && kBC % NG == 0, "record groups of whole rows");
        const int jb = tid % CK, grp = tid / CK, r0 = grp * BG;
        float bl[BG];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < BG; i++) {
            run += sl.eb[r0 + i][jb];
            bl[i] = run;
        }
        sl.btot[grp][jb] = run;
        __syncthreads();
        float pre = 0.f;
        for (int g2 = 0; g2 < grp; g2++) pre += sl.btot[g2][jb];
#pragma unroll
        for (int i = 0; i < BG; i++) {
            const int r = r0 + i;
            const float b = pre + bl[i];
            const float e = expf(b);
            const float qv = sl.qt[r][jb] * e;
            const float kv = sl.slot[cur][r] != kNoSlot
                                 ? __builtin_amdgcn_exp2f((sl.k0[r][jb] - b) * kLog2e - sl.lnz[cur][r])
                                 : 0.f;
            sl.qt[r][jb] = qv;
            sl.k0[r][jb] = kv;
            sl.eb[r][jb] = e;
            if constexpr (kBf) {
                uint16_t tq[2], tk[2];
                split_levels<2>(qv, tq);
                split_levels<2>(sl.w[cur][r] * kv, tk);
                sl.qh[r][jb] = tq[0];
                sl.ql[r][jb] = tq[1];
                sl.kh[r][jb] = tk[0];
                sl.kl[r][jb] = tk[1];
            }
        }
    }
    if (tid < kBC && xn < a.nslot) put_records(cur ^ 1, mnext);
    __syncthreads();

    // the column blocks of S_in and G~ (issued here, after the record-side
    // work: faster than with the row blocks, although most of their lines
    // come from HBM a second time)
    if (wv < CT) {
#pragma unroll
        for (int ks = 0; ks < NKC; ks++) {
            const int64_t o = (int64_t)(g4 * NKC + ks) * DV + 16 * wv + l16;
            sc[ks] = Sin[o];
            gc[ks] = Gc[o];
        }
    }
    // ---- A = Qt Kh^T and GV = g V^T masked to s <= r: the 16x16 tiles
    //      (0,0), (1,0), (1,1) of each, one wave per tile; tile (0,1) is zero
    if (wv < 6) {
        const bool isA = wv < 3;
        const int tt = wv % 3;
        const int rt = tt == 0 ? 0 : 1, st = tt == 2 ? 1 : 0;
        f32x4b acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kBf) {
            // bf16 MFMA over 32-wide k-steps: lane (l16, g4) supplies the 8
            // consecutive rows j (or columns m) 32 t + 8 g4 + i of its
            // record's row of the pre-split operands (Qt, Kh, g in two
            // terms, V exact); the output layout is that of the fp32 MFMA
            const int ra = 16 * rt + l16, sb = 16 * st + l16;
            if (isA) {
#pragma unroll
                for (int t = 0; t < CK / 32; t++) {
                    const int j0 = 32 * t + 8 * g4;
                    const u16x8 qhi = *reinterpret_cast<const u16x8*>(&sl.qh[ra][j0]);
                    const u16x8 qlo = *reinterpret_cast<const u16x8*>(&sl.ql[ra][j0]);
                    const u16x8 khi = *reinterpret_cast<const u16x8*>(&sl.kh[sb][j0]);
                    const u16x8 klo = *reinterpret_cast<const u16x8*>(&sl.kl[sb][j0]);
                    acc = mfma16(qhi, khi, acc);
                    acc = mfma16(qhi, klo, acc);
                    acc = mfma16(qlo, khi, acc);
                }
            } else {
#pragma unroll
                for (int t = 0; t < DV / 32; t++) {
                    const int m0 = 32 * t + 8 * g4;
                    const u16x8 ghi = *reinterpret_cast<const u16x8*>(&sl.gh[ra][m0]);
                    const u16x8 glo = *reinterpret_cast<const u16x8*>(&sl.gl[ra][m0]);
                    const u16x8 vb = *reinterpret_cast<const u16x8*>(&sl.v[sb][m0]);
                    acc = mfma16(ghi, vb, acc);
                    acc = mfma16(glo, vb, acc);
                }
            }
        } else if (isA) {
            for (int ks = 0; ks < CK / 4; ks++) {
                const int j = 4 * ks + g4;
                acc = mf(sl.qt[16 * rt + l16][j], sl.w[cur][16 * st + l16] * sl.k0[16 * st + l16][j], acc);
            }
        } else {
            for (int ks = 0; ks < DV / 4; ks++) {
                const int m = 4 * ks + g4;
                acc = mf(sl.g[16 * rt + l16][m], vf(16 * st + l16, m), acc);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = 16 * rt + 4 * g4 + e, s = 16 * st + l16;
            const float val = s <= r ? acc[e] : 0.f;
            if constexpr (kBf) {
                uint16_t tv[2];
                split_levels<2>(val, tv);
                (isA ? sl.ah : sl.gvh)[r][s] = tv[0];
                (isA ? sl.al : sl.gvl)[r][s] = tv[1];
            } else {
                (isA ? sl.A : sl.GV)[r][s] = val;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            if constexpr (kBf) {
                (wv == 6 ? sl.ah : sl.gvh)[4 * g4 + e][16 + l16] = 0;
                (wv == 6 ? sl.al : sl.gvl)[4 * g4 + e][16 + l16] = 0;
            } else {
                (wv == 6 ? sl.A : sl.GV)[4 * g4 + e][16 + l16] = 0.f;
            }
        }
    }
    __syncthreads();

    // ---- d-side outputs of column block wv: y (for y . g) and dV
    float yg[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (wv < CT) {
        const int m = 16 * wv + l16;
        f32x4b y[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4b dv[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        // over state rows: y += Qt S_in, dV += Kh G~.  Lane group g4 holds
        // the state rows g4 CK/4 + ks (a contiguous quarter)
        if constexpr (kBf) {
            // bf16 MFMA: k-step t of lane group g4 contracts the rows
            // g4 CK/4 + 8 t + i (i < 8): the lane's own 8 consecutive S_in and
            // G~ values (split here) and 8 consecutive values of its record's
            // row of Qt and Kh (split by the decay scan)
            auto pack8 = [](const uint32_t (&pr)[4][2], int l) {
                return __builtin_bit_cast(u16x8, make_uint4(pr[0][l], pr[1][l], pr[2][l], pr[3][l]));
            };
#pragma unroll
            for (int t = 0; t < NKC / 8; t++) {
                const int j0 = g4 * NKC + 8 * t;
                uint32_t ps[4][2], pg[4][2];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    split_pair<2>(sc[8 * t + 2 * e2], sc[8 * t + 2 * e2 + 1], ps[e2]);
                    split_pair<2>(gc[8 * t + 2 * e2], gc[8 * t + 2 * e2 + 1], pg[e2]);
                }
                const u16x8 shi = pack8(ps, 0), slo = pack8(ps, 1);
                const u16x8 ghi = pack8(pg, 0), glo = pack8(pg, 1);
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    const int r = 16 * rt + l16;
                    const u16x8 qhi = *reinterpret_cast<const u16x8*>(&sl.qh[r][j0]);
                    const u16x8 qlo = *reinterpret_cast<const u16x8*>(&sl.ql[r][j0]);
                    const u16x8 khi = *reinterpret_cast<const u16x8*>(&sl.kh[r][j0]);
                    const u16x8 klo = *reinterpret_cast<const u16x8*>(&sl.kl[r][j0]);
                    y[rt] = mfma16(qhi, shi, y[rt]);
                    y[rt] = mfma16(qhi, slo, y[rt]);
                    y[rt] = mfma16(qlo, shi, y[rt]);
                    dv[rt] = mfma16(khi, ghi, dv[rt]);
                    dv[rt] = mfma16(khi, glo, dv[rt]);
                    dv[rt] = mfma16(klo, ghi, dv[rt]);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKC; ks++) {
                const int jj = g4 * NKC + ks;
                const float bs = sc[ks];
                const float bg = gc[ks];
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    const int r = 16 * rt + l16;
                    y[rt] = mf(sl.qt[r][jj], bs, y[rt]);
                    dv[rt] = mf(sl.w[cur][r] * sl.k0[r][jj], bg, dv[rt]);
                }
            }
        }
        // over records s: y += A V, dV += A^T g
        if constexpr (kBf) {
            // the chunk's 32 records as one bf16 k-step: A rows from the
            // split tiles, A^T, V and g columns by transpose reads
            const u16x8 vb = tr16(&sl.v[0][0], SM::VRS, 16 * wv);
            const u16x8 gbh = tr16(&sl.gh[0][0], DV + 8, 16 * wv);
            const u16x8 gbl = tr16(&sl.gl[0][0], DV + 8, 16 * wv);
#pragma unroll
            for (int rt = 0; rt < 2; rt++) {
                const u16x8 ahi = lds8(&sl.ah[16 * rt + l16][8 * g4]);
                const u16x8 alo = lds8(&sl.al[16 * rt + l16][8 * g4]);
                const u16x8 athi = tr16(&sl.ah[0][0], kBC + 8, 16 * rt);
                const u16x8 atlo = tr16(&sl.al[0][0], kBC + 8, 16 * rt);
                y[rt] = mfma16(ahi, vb, y[rt]);
                y[rt] = mfma16(alo, vb, y[rt]);
                dv[rt] = mfma16(athi, gbh, dv[rt]);
                dv[rt] = mfma16(athi, gbl, dv[rt]);
                dv[rt] = mfma16(atlo, gbh, dv[rt]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kBC / 4; ks++) {
                const int s = 4 * ks + g4;
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    y[rt] = mf(sl.A[16 * rt + l16][s], vf(s, m), y[rt]);
                    dv[rt] = mf(sl.A[s][16 * rt + l16], sl.g[s][m], dv[rt]);
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 16 * rt + 4 * g4 + e;
                if (sl.slot[cur][r] != kNoSlot) a.g_dv[(int64_t)sl.slot[cur][r] * DV + m] = dv[rt][e];
                yg[rt][e] = y[rt][e] * sl.g[r][m];
            }
    }

    // the next slot's rows, loading while this chunk's c-side products run
    // (issued here, when the column blocks' registers are free)
    have = xn < a.nslot && sl.slot[cur ^ 1][0] != kNoSlot;
    if (have) load_rows(cur ^ 1);

    // ---- c-side outputs of row block wv: dQt, dKh, the chunk decay term,
    //      dlog_alpha and dq
    float dkh[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float kd[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int j = 16 * wv + l16;
    if (wv < RT) {
        f32x4b dq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4b vg[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4b dk[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        float sg = 0.f;   // this lane's part of rowsum(S_in . G~) of row j
        // over the columns m = g4 DV/4 + ks: dQt += g S_in^T, V G~^T
#pragma unroll
        for (int ks = 0; ks < NKD; ks++) {
            const int mm = g4 * NKD + ks;
            const float st = sr[ks];
            const float gt = gr[ks];
            sg += st * gt;
            if constexpr (!kBf) {
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    const int r = 16 * rt + l16;
                    dq[rt] = mf(sl.g[r][mm], st, dq[rt]);
                    vg[rt] = mf(sl.v[r][mm], gt, vg[rt]);
                }
            }
        }
        if constexpr (kBf) {
            // bf16 inputs: both products on bf16 MFMA.  k-step t of lane
            // group g4 contracts the columns g4 DV/4 + 8 t + i (i < 8): the
            // lane's own 8 consecutive S_in and G~ values (split here) and 8
            // consecutive values of its record's row of g (split by the row
            // loader) and of V (exact in bf16).
            auto pack8 = [](const uint32_t (&pr)[4][2], int l) {
                return __builtin_bit_cast(u16x8, make_uint4(pr[0][l], pr[1][l], pr[2][l], pr[3][l]));
            };
#pragma unroll
            for (int t = 0; t < NKD / 8; t++) {
                const int m0 = g4 * NKD + 8 * t;
                uint32_t pg[4][2], ps[4][2];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    split_pair<2>(gr[8 * t + 2 * e2], gr[8 * t + 2 * e2 + 1], pg[e2]);
                    split_pair<2>(sr[8 * t + 2 * e2], sr[8 * t + 2 * e2 + 1], ps[e2]);
                }
                const u16x8 gthi = pack8(pg, 0), gtlo = pack8(pg, 1);
                const u16x8 shi = pack8(ps, 0), slo = pack8(ps, 1);
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    const int r = 16 * rt + l16;
                    const u16x8 va = *reinterpret_cast<const u16x8*>(&sl.v[r][m0]);
                    const u16x8 ghi = *reinterpret_cast<const u16x8*>(&sl.gh[r][m0]);
                    const u16x8 glo = *reinterpret_cast<const u16x8*>(&sl.gl[r][m0]);
                    vg[rt] = mfma16(va, gthi, vg[rt]);
                    vg[rt] = mfma16(va, gtlo, vg[rt]);
                    dq[rt] = mfma16(ghi, shi, dq[rt]);
                    dq[rt] = mfma16(ghi, slo, dq[rt]);
                    dq[rt] = mfma16(glo, shi, dq[rt]);
                }
            }
        }
        // over records s: dQt += GV Kh, dKh += GV^T Qt
        if constexpr (kBf) {
            const u16x8 kbh = tr16(&sl.kh[0][0], CK + 8, 16 * wv);
            const u16x8 kbl = tr16(&sl.kl[0][0], CK + 8, 16 * wv);
            const u16x8 qbh = tr16(&sl.qh[0][0], CK + 8, 16 * wv);
            const u16x8 qbl = tr16(&sl.ql[0][0], CK + 8, 16 * wv);
#pragma unroll
            for (int rt = 0; rt < 2; rt++) {
                const u16x8 ghi = lds8(&sl.gvh[16 * rt + l16][8 * g4]);
                const u16x8 glo = lds8(&sl.gvl[16 * rt + l16][8 * g4]);
                const u16x8 gthi = tr16(&sl.gvh[0][0], kBC + 8, 16 * rt);
                const u16x8 gtlo = tr16(&sl.gvl[0][0], kBC + 8, 16 * rt);
                dq[rt] = mfma16(ghi, kbh, dq[rt]);
                dq[rt] = mfma16(ghi, kbl, dq[rt]);
                dq[rt] = mfma16(glo, kbh, dq[rt]);
                dk[rt] = mfma16(gthi, qbh, dk[rt]);
                dk[rt] = mfma16(gthi, qbl, dk[rt]);
                dk[rt] = mfma16(gtlo, qbh, dk[rt]);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < kBC / 4; ks++) {
                const int s = 4 * ks + g4;
#pragma unroll
                for (int rt = 0; rt < 2; rt++) {
                    dq[rt] = mf(sl.GV[16 * rt + l16][s], sl.w[cur][s] * sl.k0[s][j], dq[rt]);
                    dk[rt] = mf(sl.GV[s][16 * rt + l16], sl.qt[s][j], dk[rt]);
                }
            }
        }
        // the chunk decay term t of row j: rowsum(S_in . G~) over the four
        // lane groups, plus sum_s Kh[s][j] (V G~^T)[s][j]
        float t2 = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int s = 16 * rt + 4 * g4 + e;
                t2 += sl.w[cur][s] * sl.k0[s][j] * vg[rt][e];
            }
        float tj = sg + t2;
        tj += __shfl_xor(tj, 16, kWave);
        tj += __shfl_xor(tj, 32, kWave);
        // db and its reverse cumulative sum over the chunk's records
        // s = 16 rt + 4 g4 + e: within the lane, then the lane groups above,
        // then the second row tile into the first
        float db[2][4], tot[2];
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
            float run = 0.f;
#pragma unroll
            for (int e = 3; e >= 0; e--) {
                const int s = 16 * rt + 4 * g4 + e;
                dkh[rt][e] = vg[rt][e] + dk[rt][e];
                run += sl.qt[s][j] * dq[rt][e] - sl.w[cur][s] * sl.k0[s][j] * dkh[rt][e];
                db[rt][e] = run;
                kd[rt][e] = sl.k0[s][j] * dkh[rt][e];
            }
            tot[rt] = run;
        }
        float above[2], all1 = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
            const float T0 = __shfl(tot[rt], l16, kWave);
            const float T1 = __shfl(tot[rt], l16 + 16, kWave);
            const float T2 = __shfl(tot[rt], l16 + 32, kWave);
            const float T3 = __shfl(tot[rt], l16 + 48, kWave);
            above[rt] = (g4 < 1 ? T1 : 0.f) + (g4 < 2 ? T2 : 0.f) + (g4 < 3 ? T3 : 0.f);
            if (rt == 1) all1 = T0 + T1 + T2 + T3;
        }
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int s = 16 * rt + 4 * g4 + e;
                if (sl.slot[cur][s] != kNoSlot) {
                    const int64_t o = (int64_t)sl.slot[cur][s] * CK + j;
                    a.g_dla[o] = db[rt][e] + above[rt] + (rt == 0 ? all1 : 0.f) + tj;
                    a.g_dq[o] = dq[rt][e] * sl.eb[s][j];
                }
            }
    }
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float x1 = row_reduce<16>(yg[rt][e], [](float p, float o) { return p + o; });
            const float x2 = row_reduce<16>(kd[rt][e], [](float p, float o) { return p + o; });
            if (l16 == 0) {
                sl.dwp[wv][16 * rt + 4 * g4 + e] = x1;
                sl.kdp[wv][16 * rt + 4 * g4 + e] = x2;
            }
        }
    __syncthreads();

    // ---- key-logit gradients (kappa . dkappa = w K0 . dKh over all rows)
    //      and the gate gradients
    if (wv < RT) {
#pragma unroll
        for (int rt = 0; rt < 2; rt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int s = 16 * rt + 4 * g4 + e;
                if (sl.slot[cur][s] != kNoSlot) {
                    float kds = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < kCW; w2++) kds += sl.kdp[w2][s];
                    a.g_dkl[(int64_t)sl.slot[cur][s] * CK + j] =
                        sl.w[cur][s] * sl.k0[s][j] * (dkh[rt][e] - sl.eb[s][j] * kds);
                }
            }
    }
    if (tid < kBC && sl.slot[cur][tid] != kNoSlot) {
        float yg2 = 0.f, kds = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kCW; w2++) {
            yg2 += sl.dwp[w2][tid];
            kds += sl.kdp[w2][tid];
        }
        // y . do = (y . g) / w; a gate of zero has no gradient through e
        const float wr = sl.w[cur][tid];
        a.g_dw[sl.slot[cur][tid]] = (wr > 0.f ? yg2 / wr : 0.f) + kds;
    }
    // every read of this chunk's LDS is done before the next chunk's rows
    // and records overwrite it
    __syncthreads();
    cur ^= 1;
    }
}

// Per (token, head): sum the k + 1 slots of every gradient; the router
// logits' gradient through e = softmax(z): dz = e * (de - e . de) with de
// the gate gradients of the k chosen partitions (zero elsewhere).  One wave
// per (token, head), kCbRows per block: the wave walks the row's 16-byte
// pieces of dq, dkey_logits, dlog_alpha (c each) and dv (d), each the sum of
// its k + 1 slots in slot order, then computes the router part.
constexpr int kCbRows = 4;
template <typename TIn>
__global__ __launch_bounds__(kCbRows * kWave) void bwd_combine_kernel(const BwdArgs a, int c, int d,
                                                                     int64_t rows) {
    const int64_t row = (int64_t)blockIdx.x * kCbRows + threadIdx.x / kWave;
    if (row >= rows) return;   // wave-uniform
    const int lane = threadIdx.x % kWave;
    const int K = a.topk, N = a.N, P = K + 1;
    const int64_t sb = row * P;
    const int c4 = c / 4, items = 3 * c4 + d / 4;
    for (int it = lane; it < items; it += kWave) {
        const int arr = it < 3 * c4 ? it / c4 : 3;   // 0 dq, 1 dkl, 2 dla, 3 dv
        const int e4 = arr < 3 ? it - arr * c4 : it - 3 * c4;
        const int n = arr < 3 ? c : d;
        const float* src = arr == 0 ? a.g_dq : arr == 1 ? a.g_dkl : arr == 2 ? a.g_dla : a.g_dv;
        float* dst = arr == 0 ? a.dq : arr == 1 ? a.dkl : arr == 2 ? a.dla : a.dv;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int p = 0; p < P; p++) {
            const float4 x = *reinterpret_cast<const float4*>(src + (sb + p) * n + 4 * e4);
            acc.x += x.x;
            acc.y += x.y;
            acc.z += x.z;
            acc.w += x.w;
        }
        *reinterpret_cast<float4*>(dst + row * n + 4 * e4) = acc;
    }
    // router softmax over N (N <= 64)
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

namespace {

template <int CK, int DV, typename TIn>
void launch_bwd_cfg(const BwdArgs& a, hipStream_t st) {
    const int64_t nseg = (int64_t)a.num_seqs * a.H * (a.N + 1);
    if (nseg == 0) return;
    bwd_sweep_kernel<CK, DV, TIn><<<(unsigned)(2 * nseg), sweep_waves<CK, DV>() * kWave, 0, st>>>(a);
    if (a.nslot > 0) {
        // as many chunk blocks as the device holds at once (each walks the
        // slots b, b + grid, ...); queried once per device and shape
        constexpr int kDevs = 64;
        static std::atomic<int> resident[kDevs];   // 0: not queried yet
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) dev = -1;
        int blocks = dev >= 0 ? resident[dev].load(std::memory_order_relaxed) : 0;
        if (blocks <= 0) {
            int cus = 0, per_cu = 0;
            if (dev < 0 ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_chunk_kernel<CK, DV, TIn>,
                                                             kCW * kWave, 0) != hipSuccess ||
                cus < 1 || per_cu < 1) {
                cus = 256;
                per_cu = 1;
            }
            blocks = cus * per_cu;
            if (dev >= 0) resident[dev].store(blocks, std::memory_order_relaxed);
        }
        const int64_t grid = std::min<int64_t>(a.nslot, (int64_t)blocks);
        bwd_chunk_kernel<CK, DV, TIn><<<(unsigned)grid, kCW * kWave, 0, st>>>(a);
    }
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
    const unsigned nb = (unsigned)((a.rows + kCbRows - 1) / kCbRows);
    if (dtype == kF32)
        bwd_combine_kernel<float><<<nb, kCbRows * kWave, 0, st>>>(a, c, d, a.rows);
    else
        bwd_combine_kernel<bf16_t><<<nb, kCbRows * kWave, 0, st>>>(a, c, d, a.rows);
    return hipGetLastError();
}

}  // namespace sse
