// piece_state.hip -- key-softmax normalisers and the shared partition's
// piece states, for bf16 inputs on gfx950.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eq. 11 (the key is the softmax of the key logits over the c state
// rows), §2.1 eq. 6 (diagonal decay) and §2.5 (the always-active shared
// partition takes every token with weight 1).
//
// The shared partition's chain is split into pieces of piece_len tokens so
// that its output pass can run the pieces in parallel; piece p starts from
//   S_in(p) = D(p-1) S_in(p-1) + S_loc(p-1),
// where S_loc(p) is the state the piece builds from zero and D(p) its total
// decay.  Unrolling the recurrence over the piece's records r,
//   S_loc = sum_r diag(exp(R_r)) kappa_r^T v_r,  R_r = sum_{u > r in piece} log_alpha_u,
//   D     = exp(sum_{u in piece} log_alpha_u),
// so S_loc is one product K~^T V with K~_r = kappa_r * exp(R_r): no state
// decay between records, and every exponent is <= 0.  The kernel walks a
// piece backwards in steps of 16 records (one k-step of a 32x32x16 bf16
// MFMA) and carries R per row in registers.
//
// Block = 4 waves per (sequence, head, piece).  Per step:
//   1. row layout (lane = 8 consecutive columns of one record, 16-byte
//      loads issued two steps ahead): the record's key-softmax normaliser
//      lnz2 = log2 sum_j 2^(kl_j log2 e) (max-shifted), kept in LDS and
//      written to lnz2_out for the later passes at the end; the rows of key logits, log decay and v and
//      the normalisers go to one of two LDS stages;
//   2. MFMA layout: LDS transpose reads (ds_read_b64_tr_b16) give each lane
//      8 consecutive records of one row j of the state (the A operand) and of
//      one column of v (the B operand); the lane forms R, K~ = 2^((kl + R)
//      log2 e - lnz2), splits K~ into two bf16 terms (v is exact in bf16) and
//      accumulates its state tiles.
// The last piece of a sequence needs no state: its block only computes the
// normalisers.
//
// The same kernel, in its gathered form, gives the piece states of long
// routed segments (§2.6: each partition's records form a sub-sequence of
// their own; splitting one into pieces is the same unrolling over its
// records).  The records come from the grouping's segment records (input
// row and exponent offset cr = lnz2 - log2 e_i, so that K~ carries the
// router weight: K~_r = e_r kappa_r exp(R_r)).  The routed pass combines
// them into each piece's start state, start(p+1) = D(p) start(p) + S_loc(p)
// with start(0) the segment's initial state.
#include "chunk_common.h"

namespace sse {

namespace {

constexpr int kPsWaves = 4;
constexpr int kPsThreads = kPsWaves * kWave;
constexpr int kPsRec = 16;  // records per step
constexpr int kDepth = 2;   // steps whose row loads are in flight
static_assert(kSharedPiece % kPsRec == 0, "pieces must be whole steps");
static_assert(kMaxRoutedPiece % kPsRec == 0, "pieces must be whole steps");

// Row stride (elements) of an LDS stage row of `cols` bf16 values.  The
// transpose reads of a half-wave touch 4 records x 64 bytes; a stride of
// 64 or 192 bytes modulo 256 puts those four 64-byte pieces on disjoint
// banks.
constexpr int ps_stride(int cols) { return cols >= 64 ? cols + 32 : cols; }

template <int CK, int DV>
struct PsStage {
    uint16_t kl[kPsRec][ps_stride(CK)];
    uint16_t la[kPsRec][ps_stride(CK)];
    uint16_t v[kPsRec][ps_stride(DV)];
    float lnz2[kPsRec];
};

// The 8 values (records 8 (lane/32) + 0..7, column col0 + lane % 32) of a
// 32x32x16 MFMA operand from a record-major LDS tile [16][stride].
template <int STRIDE>
__device__ __forceinline__ u16x8 tr_operand(const uint16_t* tile, int col0, int lane) {
    const int g = lane / 16, jj = lane % 16;
    const int rec = 8 * (g / 2) + jj / 4;
    const int col = col0 + 16 * (g % 2) + 4 * (jj % 4);
    return cat_tr(lds_tr(tile + rec * STRIDE + col), lds_tr(tile + (rec + 4) * STRIDE + col));
}

// Aggregate slot of piece p of routed segment g (records [off, off + n) of
// the grouping): floor(off / P) + g + p.  Segments are in record order, so
// the slots of consecutive segments never overlap and all fit in
// records / P + segments + 1 slots.
__device__ __forceinline__ int64_t rpiece_slot(int64_t off, int g, int p, int P) {
    return off / P + g + p;
}

// One block's work: shared piece `piece` of (sequence, head) unit `bx`, or
// (GATHER) full piece `piece` of routed segment `bx`.  LDS comes from the
// kernel: the two operand stages, and lnz_all (the shared piece's
// normalisers: kSharedPiece floats) or g_row / g_cr (the routed records'
// rows and exponent offsets: kMaxRoutedPiece each).
template <int CK, int DV, bool GATHER>
__device__ __forceinline__ void piece_body(const ChunkArgs& a, const int bx, const int piece,
                                           PsStage<CK, DV>* st, float* lnz_all, uint32_t* g_row,
                                           float* g_cr) {
    constexpr int KS = ps_stride(CK), VS = ps_stride(DV);
    constexpr int RT = CK / 32, CT = DV / 32;         // 32-row / 32-column tiles of the state
    constexpr int WPR = kPsWaves / RT;                // waves sharing one row tile
    constexpr int NT = (CT + WPR - 1) / WPR;          // column tiles per wave
    constexpr int LPR = CK / 8, LPRV = DV / 8;        // lanes per record (16-byte pieces)
    static_assert(RT >= 1 && RT <= kPsWaves && kPsWaves % RT == 0, "unsupported c");
    static_assert(kPsRec * LPR <= kPsThreads && kPsRec * LPRV <= kPsThreads, "unsupported shape");
    // (the piece's normalisers are written to global memory once at the
    // end: a store inside the step loop would be counted with the loads in
    // flight (one vector-memory counter), so every step would wait for it)
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int H = a.H;
    int s = 0, h = 0, n;
    int64_t lo, slot;
    bool state;
    if constexpr (GATHER) {
        // routed segment g, full piece `piece` of rpiece_len records (the
        // segment's last piece needs no state)
        const int g = bx, P = a.rpiece_len;
        const int64_t off = a.seg_offsets[g], len = a.seg_offsets[g + 1] - off;
        const int npieces = len > 0 ? (int)((len + P - 1) / P) : 1;
        if (piece >= npieces - 1) return;  // uniform
        lo = off + (int64_t)piece * P;
        n = P;
        state = true;
        slot = rpiece_slot(off, g, piece, P);
        for (int r = tid; r < n; r += kPsThreads) {
            const SegRec rec = a.seg_rec[lo + r];
            g_row[r] = rec.row;
            g_cr[r] = rec.cr;
        }
        __syncthreads();
    } else {
        const int sh = bx;
        s = sh / H;
        h = sh % H;
        const int64_t t0 = a.cu[s], len = a.cu[s + 1] - t0;
        const int npieces = len > 0 ? (int)((len + a.piece_len - 1) / a.piece_len) : 1;
        if (piece >= npieces || len == 0) return;  // uniform
        lo = t0 + (int64_t)piece * a.piece_len;
        n = (int)min<int64_t>(a.piece_len, len - (int64_t)piece * a.piece_len);
        state = piece < npieces - 1;  // full piece whose state is needed
        slot = ((int64_t)s * H + h) * a.max_pieces + piece;
    }
    const int nsteps = (n + kPsRec - 1) / kPsRec;

    const uint16_t* __restrict__ gk = static_cast<const uint16_t*>(GATHER ? a.kl_r : a.kl);
    const uint16_t* __restrict__ gl = static_cast<const uint16_t*>(a.la);
    const uint16_t* __restrict__ gv = static_cast<const uint16_t*>(a.v);

    // ---- row layout: this thread's record and 8-column piece
    const int rr = tid / LPR, kc = 8 * (tid % LPR);
    const int rv = tid / LPRV, vc = 8 * (tid % LPRV);
    // Guards that hold for every thread of a shape are compile-time true:
    // a runtime condition around code in the step loop makes the compiler
    // wait for every load in flight at the loop head, defeating the prefetch.
    const bool krow = (kPsRec * LPR >= kPsThreads) || rr < kPsRec;
    const bool vrow = (kPsRec * LPRV >= kPsThreads) || rv < kPsRec;
    // record index (within the piece) of row r of step i: backwards over a
    // state piece, forwards over the last piece
    auto rec_of = [&](int i, int r) { return state ? n - kPsRec * (i + 1) + r : kPsRec * i + r; };
    // a valid record for the loads (state pieces are whole multiples of 16)
    auto clamp_rec = [&](int rec) { return min(max(rec, 0), n - 1); };
    struct Raw {
        uint4 k, l, v;
    };
    // Every step issues the same loads (rows past the piece are clamped to a
    // valid one), so the compiler can count the loads in flight and wait
    // only for the ones a step consumes.
    auto load = [&](auto stI, int i, Raw& R) {
        constexpr bool STATE = decltype(stI)::value;
        const int rk = min(rr, kPsRec - 1), rvv = min(rv, kPsRec - 1);
        const int64_t row = GATHER ? (int64_t)g_row[clamp_rec(rec_of(i, rk))]
                                   : (lo + clamp_rec(rec_of(i, rk))) * H + h;
        R.k = *reinterpret_cast<const uint4*>(gk + row * CK + kc % CK);
        if constexpr (STATE) {
            R.l = *reinterpret_cast<const uint4*>(gl + row * CK + kc % CK);
            const int64_t rowv = GATHER ? (int64_t)g_row[clamp_rec(rec_of(i, rvv))]
                                        : (lo + clamp_rec(rec_of(i, rvv))) * H + h;
            R.v = *reinterpret_cast<const uint4*>(gv + rowv * DV + vc % DV);
        }
    };

    // ---- MFMA layout: row tile rt, this wave's column tiles
    const int rt = wv % RT, ct0 = RT == kPsWaves ? 0 : wv / RT;
    constexpr bool kAllTiles = CT % WPR == 0;  // every (ct0, u) names a tile
    const int j = 32 * rt + lane % 32;      // state row of this lane's A operand
    const int half = lane / 32;             // records 8 half .. 8 half + 7 of a step
    f32x16 acc[NT];
#pragma unroll
    for (int u = 0; u < NT; u++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[u][e] = 0.f;
    float carry = 0.f;  // sum of log_alpha over the records after the current step (row j)

    // Step i's rows are loaded kDepth steps ahead into ring[i % (kDepth + 1)]:
    // each step loads into the register set the previous step consumed, not
    // its own (with the set just consumed as the load target the compiler
    // waited for every load in flight at the loop head).  The step loop is
    // unrolled by kDepth + 1 so the ring is indexed statically.
    constexpr int kRing = kDepth + 1;
    Raw ring[kRing];
    auto step = [&](auto stI, int i, Raw& R, Raw& Rnext) {
        constexpr bool STATE = decltype(stI)::value;
        PsStage<CK, DV>& S = st[i & 1];
        // 1. normaliser of this thread's record (max-shifted log-sum-exp over
        //    the LPR lanes of the record), rows into the stage
        if (GATHER && krow) {
            // the exponent offset comes with the record.  (The rows are
            // copied member by member: a whole-struct copy out of the load
            // ring kept the ring in scratch memory, and every step then
            // waited for its own prefetch.)
            if constexpr (STATE) {
                *reinterpret_cast<uint4*>(&S.kl[rr][kc]) = make_uint4(R.k.x, R.k.y, R.k.z, R.k.w);
                *reinterpret_cast<uint4*>(&S.la[rr][kc]) = make_uint4(R.l.x, R.l.y, R.l.z, R.l.w);
                if (kc == 0) S.lnz2[rr] = g_cr[rec_of(i, rr)];
            }
        } else if (krow) {
            const uint32_t w4[4] = {R.k.x, R.k.y, R.k.z, R.k.w};
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                x[2 * e] = __uint_as_float(w4[e] << 16);
                x[2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
            }
            float m = x[0];
#pragma unroll
            for (int e = 1; e < 8; e++) m = fmaxf(m, x[e]);
            m = row_reduce<LPR>(m, [](float p, float q) { return fmaxf(p, q); });
            const float m2 = m * kLog2e;
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) sum += __builtin_amdgcn_exp2f(fmaf(x[e], kLog2e, -m2));
            sum = row_reduce<LPR>(sum, [](float p, float q) { return p + q; });
            const float l2 = m2 + __builtin_amdgcn_logf(sum);  // sum >= 1
            const int rec = rec_of(i, rr);
            if (kc == 0 && rec >= 0 && rec < n) lnz_all[rec] = l2;
            if constexpr (STATE) {
                *reinterpret_cast<uint4*>(&S.kl[rr][kc]) = R.k;
                *reinterpret_cast<uint4*>(&S.la[rr][kc]) = R.l;
                if (kc == 0) S.lnz2[rr] = l2;
            }
        }
        if constexpr (STATE) {
            if (vrow) *reinterpret_cast<uint4*>(&S.v[rv][vc]) = R.v;
        }
        load(stI, i + kDepth, Rnext);
        if constexpr (!STATE) return;
        lds_barrier();

        // 2. this lane's 8 records of row j: log decay suffix sums and K~
        const u16x8 kl8 = tr_operand<KS>(&S.kl[0][0], 32 * rt, lane);
        const u16x8 la8 = tr_operand<KS>(&S.la[0][0], 32 * rt, lane);
        float lav[8], suf[8];
        float run = 0.f;
#pragma unroll
        for (int e = 7; e >= 0; e--) {
            lav[e] = __uint_as_float((uint32_t)la8[e] << 16);
            suf[e] = run;  // records after e within this lane's 8
            run += lav[e];
        }
        const float other = __shfl_xor(run, 32, kWave);  // the partner lane's 8 records
        const float base = carry + (half == 0 ? other : 0.f);
        carry += run + other;
        const float4 z0 = *reinterpret_cast<const float4*>(&S.lnz2[8 * half]);
        const float4 z1 = *reinterpret_cast<const float4*>(&S.lnz2[8 * half + 4]);
        const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        uint32_t hi[4], lo2[4];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            float kv[2];
#pragma unroll
            for (int q = 0; q < 2; q++) {
                const int e = 2 * p + q;
                const float kx = __uint_as_float((uint32_t)kl8[e] << 16);
                kv[q] = __builtin_amdgcn_exp2f(fmaf(kx + (base + suf[e]), kLog2e, -zz[e]));
            }
            uint32_t t2[2];
            split_pair<2>(kv[0], kv[1], t2);
            hi[p] = t2[0];
            lo2[p] = t2[1];
        }
        const u16x8 ah = __builtin_bit_cast(u16x8, make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const u16x8 al = __builtin_bit_cast(u16x8, make_uint4(lo2[0], lo2[1], lo2[2], lo2[3]));
        // 3. S_loc[j, cols of tile] += K~^T v over the 16 records
#pragma unroll
        for (int u = 0; u < NT; u++) {
            const int ct = ct0 + WPR * u;
            if (kAllTiles || ct < CT) {
                const u16x8 vb = tr_operand<VS>(&S.v[0][0], 32 * ct, lane);
                acc[u] = mfma32(ah, vb, acc[u]);
                acc[u] = mfma32(al, vb, acc[u]);
            }
        }
    };
    auto run = [&](auto stI) {
#pragma unroll
        for (int p = 0; p < kDepth; p++) load(stI, p, ring[p]);
        int i0 = 0;
        for (; i0 + kRing <= nsteps; i0 += kRing) {
#pragma unroll
            for (int p = 0; p < kRing; p++) step(stI, i0 + p, ring[p], ring[(p + kDepth) % kRing]);
        }
#pragma unroll
        for (int p = 0; p < kRing - 1; p++)
            if (i0 + p < nsteps) step(stI, i0 + p, ring[p], ring[(p + kDepth) % kRing]);
    };
    if (GATHER || state)
        run(std::true_type{});
    else if constexpr (!GATHER)
        run(std::false_type{});
    // ---- the piece's normalisers
    if constexpr (!GATHER) {
        __syncthreads();
        for (int r = tid; r < n; r += kPsThreads) a.lnz2_out[(lo + r) * H + h] = lnz_all[r];
    }
    if (!state) return;

    // ---- the piece's state (fragment-major: tile (rt, ct) of the piece,
    //      lane, its 16 accumulator values) and total decay
    float* const aS = GATHER ? a.ragg_S : a.agg_S;
    float* const aD = GATHER ? a.ragg_D : a.agg_D;
#pragma unroll
    for (int u = 0; u < NT; u++) {
        const int ct = ct0 + WPR * u;
        if (kAllTiles || ct < CT) {
            float4* fs = reinterpret_cast<float4*>(aS + (((slot * RT + rt) * CT + ct) * kWave + lane) * 16);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                fs[q4] = make_float4(acc[u][4 * q4], acc[u][4 * q4 + 1], acc[u][4 * q4 + 2], acc[u][4 * q4 + 3]);
        }
    }
    if (ct0 == 0 && half == 0) aD[slot * CK + j] = __builtin_amdgcn_exp2f(carry * kLog2e);
}

// Shared pieces only: grid (S*H, max_pieces).
template <int CK, int DV>
__global__ __launch_bounds__(kPsThreads) void piece_state_kernel(const ChunkArgs a) {
    __shared__ __attribute__((aligned(16))) PsStage<CK, DV> st[2];
    __shared__ float lnz_all[kSharedPiece];
    piece_body<CK, DV, false>(a, blockIdx.x, blockIdx.y, st, lnz_all, nullptr, nullptr);
}

// Shared pieces (blocks [0, S*H*max_pieces)) and the full pieces of routed
// segments (the rest, G*(rmax_pieces - 1) blocks) in one launch, so the two
// kinds of blocks fill the chip together.
template <int CK, int DV>
__global__ __launch_bounds__(kPsThreads) void piece_state_both_kernel(const ChunkArgs a) {
    __shared__ __attribute__((aligned(16))) PsStage<CK, DV> st[2];
    __shared__ uint32_t g_row[kMaxRoutedPiece];
    __shared__ float g_cr[kMaxRoutedPiece];   // the shared blocks' normalisers
    static_assert(kMaxRoutedPiece >= kSharedPiece, "normalisers share g_cr");
    const int SH = a.num_seqs * a.H;
    const int nsh = SH * a.max_pieces;
    const int b = blockIdx.x;
    if (b < nsh) {
        piece_body<CK, DV, false>(a, b % SH, b / SH, st, g_cr, nullptr, nullptr);
    } else {
        const int G = SH * a.N, r = b - nsh;
        piece_body<CK, DV, true>(a, r % G, r / G, st, nullptr, g_row, g_cr);
    }
}

template <int CK, int DV>
void launch_ps(const ChunkArgs& a, hipStream_t st) {
    if (a.rpiece_len > 0 && a.rmax_pieces > 1) {
        const int64_t SH = (int64_t)a.num_seqs * a.H;
        const int64_t nb = SH * a.max_pieces + SH * a.N * (a.rmax_pieces - 1);
        piece_state_both_kernel<CK, DV><<<(unsigned)nb, kPsThreads, 0, st>>>(a);
        return;
    }
    const dim3 grid((unsigned)(a.num_seqs * a.H), (unsigned)a.max_pieces);
    piece_state_kernel<CK, DV><<<grid, kPsThreads, 0, st>>>(a);
}

}  // namespace

hipError_t launch_piece_state(const ChunkArgs& a, int c, int d, hipStream_t st) {
    if ((int64_t)a.num_seqs * a.H == 0) return hipSuccess;
    if (a.piece_len > kSharedPiece || a.piece_len % kPsRec != 0) return hipErrorInvalidValue;
#define SSE_PS_CASE(CC, DD)          \
    if (c == CC && d == DD) {        \
        launch_ps<CC, DD>(a, st);    \
        return hipGetLastError();    \
    }
    SSE_PS_CASE(32, 32) SSE_PS_CASE(32, 64) SSE_PS_CASE(32, 128)
    SSE_PS_CASE(64, 32) SSE_PS_CASE(64, 64) SSE_PS_CASE(64, 128)
    SSE_PS_CASE(128, 32) SSE_PS_CASE(128, 64) SSE_PS_CASE(128, 128)
#undef SSE_PS_CASE
    return hipErrorInvalidValue;
}

}  // namespace sse
