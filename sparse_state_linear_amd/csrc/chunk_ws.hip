// chunk_ws.hip -- warp-specialised chunked gated linear attention for bf16
// inputs on gfx950 (the routed and shared passes).
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记",
// §2.3 eqs. 12-14 (gated write and read of a partition state), §2.1 eq. 6
// (diagonal decay), §2.5 (shared partition), §2.6 (each partition runs over
// its own records, identity transition elsewhere; outputs summed back to the
// token).  The chunked form is the one in chunk_gla.hip:
//   Qt = q exp(b),  Kh = w kappa exp(-b),  A = (Qt Kh^T) masked to s <= r,
//   O = w_r (A V + Qt S_in),  S_out = diag(exp(b_C)) (S_in + Kh^T V),
// with b the in-chunk cumulative log decay, chunks of 32 records.
//
// Block = 8 waves.  Waves 0-3 consume: wave w keeps columns [32w, 32w+32) of
// the fp32 state in MFMA accumulator registers and runs every MFMA of the
// chunk.  Waves 4-7 produce: they load the records' rows, form the decayed
// operands, split them into bf16 terms and store them in one of two LDS
// stages.  Iteration n:
//   producers: issue the row loads of chunk n+3 and the metadata loads of
//              chunk n+6, prepare chunk n+1 into stage (n+1)%2, store the
//              metadata of chunk n+5 into the ring;
//   consumers: finish chunk n-1 (O += A V with A from the previous
//              iteration, then the output stores), compute the causal
//              A tiles of chunk n, O = Qt S_in, and S = D (S + Kh^T V);
//   one barrier.
// The A tiles of chunk n are written by three waves and read by all four, so
// their product with V waits one iteration (the barrier orders it); the V
// operand of chunk n stays in registers meanwhile.
//
// LDS layouts (all operand reads are 16-byte):
//   Qt, Kh record-major [r][j]: inside every 16 columns the 4-column blocks
//     are stored in the order 0,2,1,3, so the 8 columns a lane needs as the
//     MFMA partner of the state registers (rows 4h..4h+3 and 8+4h..8+4h+3 of
//     each 16) are contiguous.
//   Kh and V record-major as well (no transposed copies): the operands of
//     S += Kh^T V and O += A V, whose contraction runs over records, come from
//     8-byte LDS transpose reads (row stride and swizzle: rm_stride, rm_swz).
#include "chunk_common.h"

namespace sse {

namespace {

constexpr int kWsC = 32;          // records per chunk
constexpr int kCons = 4;          // consumer waves
constexpr int kProd = 4;          // producer waves
constexpr int kWsThreads = (kCons + kProd) * kWave;
constexpr int kRing = 8;          // metadata ring slots (7 are live at a time)
constexpr int kL = 2;             // bf16 terms of Qt, Kh, A and S
constexpr uint32_t kPadOff = 0x80000000u;  // row offset of padded records: past every
                                           // input (inputs are < 2^31 bytes)
constexpr uint32_t kNoRow = 0xffffffffu;   // masked schedule: token outside the
                                           // partition's write and read sets

static_assert(kProd == kNW, "the preparation layout assumes four producer waves");

// Record-major tiles read by 8-byte transpose reads (Kh, V): row stride in
// elements, and the column swizzle of record r.  With 64 or more columns the
// stride is 64 or 192 bytes modulo 256 and columns are XORed with 48 when
// bit 2 xor bit 3 of r is set: the transpose reads (4 records x 64 bytes per
// half-wave), the producers' 8-byte stores (2 records 4 apart x 64 bytes per
// 16 lanes) and Kh's 16-byte A-tile reads (16 records x 32 bytes per
// half-wave) then all hit distinct banks (found by exhaustive search over
// strides and XOR-linear swizzles under the measured bank rules).  32-column
// tiles have no such layout and keep a padded stride.  The swizzled
// addresses of the two transpose reads of an operand differ per lane, which
// costs registers: the routed pass uses the swizzle, the shared pass (which
// would spill with it) keeps plain rows, conflict-free for its transpose
// reads and 2-way for the A-tile reads and the stores (measured on gfx950:
// routed 446 -> 429 us with the swizzle; shared 316 us with it, 261 without).
constexpr int rm_stride(int cols) { return cols >= 64 ? cols + 32 : cols + 8; }
template <int COLS, bool SWZ>
__device__ __forceinline__ int rm_swz(int r) {
    return (SWZ && COLS >= 64) ? 48 * (((r >> 2) ^ (r >> 3)) & 1) : 0;
}

template <int CK, int DV>
struct WsStage {
    static constexpr int QS = CK + 8;
    static constexpr int KS = rm_stride(CK), VS = rm_stride(DV);
    uint16_t q[kL][kWsC][QS];     // Qt terms [r][perm(j)]
    uint16_t kr[kL][kWsC][KS];    // Kh terms [s][perm(j) ^ rm_swz(s)] (see rm_swz)
    uint16_t v[kWsC][VS];         // V (exact in bf16) [s][col ^ rm_swz(s)]
};

template <int CK, int DV>
struct WsSmem {
    WsStage<CK, DV> st[2];
    uint16_t a[2][kL][kWsC][kWsC + 8];  // A terms [r][s]
    float ebc[3][CK];                   // exp(b_C) per state row, ring by chunk % 3
    uint32_t mrow[kRing][kWsC];         // byte offset of the record's q / key / log_alpha
                                        // row, past every input for a padded record
    uint32_t mrv[kRing][kWsC];          // the same for its v row
    uint32_t mout[kRing][kWsC];         // output row: slot row (t*H + h)*topk + rank
                                        // (routed) or t*H + h (shared)
    float mcr[kRing][kWsC];             // lnz2 - log2 w (+inf if padded)
    float mw[kRing][kWsC];              // read gate; -0.0 marks a padded record
    float xs[kCons][16][32];            // per consumer wave: half an output tile,
                                        // transposed to whole-row 16-byte stores
};

// Storage column of the 4-column block starting at j (j % 4 == 0).
__device__ __forceinline__ int perm_col(int j) {
    const int b = (j >> 2) & 3;
    return (j & ~15) | ((((b & 1) << 1) | (b >> 1)) << 2);
}
struct Meta {
    uint32_t row, orow;  // input row t*H + h; output row (slot row or o row)
    float cr, w;
};

}  // namespace

template <int CK, int DV, int MODE>
__global__ __launch_bounds__(kWsThreads, 1) void chunk_ws_kernel(const ChunkArgs a) {
    using SM = WsSmem<CK, DV>;
    using GK = Geo<kWsC, CK>;
    using GV = Geo<kWsC, DV>;
    static_assert(MODE == kModeShared || MODE == kModeRouted || MODE == kModeMasked,
                  "shared, routed and masked passes only");
    constexpr bool kPart = MODE != kModeShared;  // one block per (sequence, head, partition)
    constexpr bool kSwz = kPart;                 // record-major tile swizzle (rm_swz)
    constexpr int NS = DV / 32;       // consumer waves that own state columns
    constexpr int RT_N = CK / 32;     // 32-row tiles of the state
    constexpr int RPG = GK::RPG, RPGV = GV::RPG;
    __shared__ __attribute__((aligned(16))) SM sm;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const bool producer = wv >= kCons;
    // Wave priority when a producer and a consumer wave of a SIMD are both
    // ready: producers first in the routed pass, consumers first in the
    // shared pass (whose consumers also load slots and store o).  Measured
    // on gfx950 against equal priority: routed 426-429 us against 434-437 on
    // one box, no difference on another; shared 263 against 265 us, and
    // 286 us with the producers first.
    if (kPart ? producer : !producer) __builtin_amdgcn_s_setprio(2);
    const int pw = wv - kCons;                                   // producer index
    const int hh = lane / 32, l32 = lane % 32;
    const int H = a.H, N = a.N;
    const bool col_wave = !producer && (NS == kCons || wv < NS);

    // ---------------- which records this block runs ----------------
    int s, h, part, piece = 0, npieces = 1;
    int64_t lo, n, rslot = 0;
    if constexpr (kPart) {
        // Blocks are dispatched to the 8 XCDs round-robin (block b on XCD
        // b % 8).  Map the N partitions of one (sequence, head) to the same
        // XCD, dispatched together: they walk the same tokens at about the
        // same pace, so the k reads of a token's rows and the k additions to
        // its output row meet in that XCD's L2.  The masked schedule walks
        // every token of the sequence for every partition.
        int g = blockIdx.x;
        const int U = a.num_seqs * H;
        if ((U & 7) == 0) {
            const int x = g & 7, j = g >> 3;
            g = ((j / N) * 8 + x) * N + j % N;
        }
        part = g % N;
        s = g / N / H;
        h = g / N % H;
        if constexpr (MODE == kModeRouted) {
            lo = a.seg_offsets[g];
            n = a.seg_offsets[g + 1] - lo;
            if (a.rpiece_len > 0) {
                // a long segment runs as pieces of rpiece_len records; the
                // local state of its piece p is in slot
                // floor(first record / P) + g + p
                const int P = a.rpiece_len;
                npieces = n > 0 ? (int)((n + P - 1) / P) : 1;
                piece = blockIdx.y;
                if (piece >= npieces) return;  // uniform
                rslot = lo / P + g;
                lo += (int64_t)piece * P;
                n = min<int64_t>(P, n - (int64_t)piece * P);
            }
        } else {
            lo = a.cu[s];
            n = a.cu[s + 1] - lo;
        }
    } else {
        const int sh = blockIdx.x;
        s = sh / H;
        h = sh % H;
        part = N;
        piece = blockIdx.y;
        const int64_t t0 = a.cu[s], len = a.cu[s + 1] - t0;
        npieces = len > 0 ? (int)((len + a.piece_len - 1) / a.piece_len) : 1;
        if (piece >= npieces) return;  // uniform
        lo = t0 + (int64_t)piece * a.piece_len;
        n = min<int64_t>(a.piece_len, len - (int64_t)piece * a.piece_len);
        if (n < 0) n = 0;
    }
    const int64_t nchunks = (n + kWsC - 1) / kWsC;
    const bool last_piece = piece == npieces - 1;
    const int64_t sbase = (((int64_t)s * H + h) * (N + 1) + part) * CK * DV;
    const int64_t abase = ((int64_t)s * H + h) * a.max_pieces;

    const bf16_t* __restrict__ gq = static_cast<const bf16_t*>(a.q);
    const bf16_t* __restrict__ gk = static_cast<const bf16_t*>(a.kl);
    const bf16_t* __restrict__ gv = static_cast<const bf16_t*>(a.v);
    const bf16_t* __restrict__ gl = static_cast<const bf16_t*>(a.la);

    // ---------------- consumer state ----------------
    // rows 32 rt + 8 (i/4) + 4 hh + i%4, column 32 wv + l32
    const int col = 32 * wv + l32;
    const uint32_t col4 = 4u * (uint32_t)col;
    f32x16 S[RT_N];
#pragma unroll
    for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
        for (int i = 0; i < 16; i++) S[rt][i] = 0.f;
    if (col_wave) {
        if (a.init) {
#pragma unroll
            for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                    S[rt][i] = a.init[sbase + (int64_t)row * DV + col];
                }
        }
        // S_in(p) = D_{p-1} S_in(p-1) + S_loc(p-1), from the piece-state pass,
        // whose piece states are stored fragment-major (the 16 values of
        // this lane's 32x32 tile (rt, wv) contiguous: 16-byte loads); a
        // routed segment's pieces have their own slots
        const float* const pS = kPart ? a.ragg_S : a.agg_S;
        const float* const pD = kPart ? a.ragg_D : a.agg_D;
        for (int p = 0; p < piece; p++) {
            const int64_t ab = (kPart ? rslot : abase) + p;
#pragma unroll
            for (int rt = 0; rt < RT_N; rt++) {
                const float4* fs = reinterpret_cast<const float4*>(
                    pS + (((ab * RT_N + rt) * NS + wv) * kWave + lane) * 16);
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) {
                    const float4 d4 = *reinterpret_cast<const float4*>(&pD[ab * CK + 32 * rt + 8 * q4 + 4 * hh]);
                    const float4 s4 = fs[q4];
                    S[rt][4 * q4 + 0] = d4.x * S[rt][4 * q4 + 0] + s4.x;
                    S[rt][4 * q4 + 1] = d4.y * S[rt][4 * q4 + 1] + s4.y;
                    S[rt][4 * q4 + 2] = d4.z * S[rt][4 * q4 + 2] + s4.z;
                    S[rt][4 * q4 + 3] = d4.w * S[rt][4 * q4 + 3] + s4.w;
                }
            }
        }
    }

    // ---------------- producer: metadata ----------------
    // Producer wave 0 loads the metadata of one chunk (lane % 32 = record,
    // clamped into the segment so every load is valid) and stores it into the
    // ring one iteration later.  Padded records keep a real row and carry a
    // read gate of -0.0 and an exponent offset of +inf (so Kh = 0).
    auto meta_load = [&](int64_t chunk, Meta& m) {
        const int64_t idx = chunk * kWsC + (lane % kWsC);
        const int64_t ci = idx < n ? idx : n - 1;
        if constexpr (MODE == kModeRouted) {
            const uint4 r = *reinterpret_cast<const uint4*>(a.seg_rec + (lo + ci));
            m.row = r.x;
            m.orow = r.y;
            m.cr = __uint_as_float(r.z);
            m.w = __uint_as_float(r.w);
        } else if constexpr (MODE == kModeMasked) {
            // token lo + ci is written when the partition is in its write
            // set (weight e: the key is e kappa) and read when it is in its
            // read set (read weight, slot row = the read rank); a token in
            // neither is padding.  All loads are issued before any select.
            const uint32_t row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
            int32_t wi[kMaxTopK], ri[kMaxTopK];
            float ww[kMaxTopK], rw[kMaxTopK];
#pragma unroll
            for (int j = 0; j < kMaxTopK; j++) {
                if (j < a.sel_k) {
                    wi[j] = a.sel_idx[row * (uint32_t)a.sel_k + j];
                    ww[j] = a.sel_w[row * (uint32_t)a.sel_k + j];
                }
                if (j < a.rd_k) {
                    ri[j] = a.rd_idx[row * (uint32_t)a.rd_k + j];
                    rw[j] = a.rd_w[row * (uint32_t)a.rd_k + j];
                }
            }
            const float l2 = a.lnz2_r[row];
            bool wrt = false;
            float we = 1.f, wr = -0.f;
            int jr = -1;
#pragma unroll
            for (int j = 0; j < kMaxTopK; j++) {
                if (j < a.sel_k && wi[j] == part) {
                    wrt = true;
                    we = ww[j];
                }
                if (j < a.rd_k && ri[j] == part) {
                    jr = j;
                    wr = rw[j];
                }
            }
            m.row = (wrt || jr >= 0) ? row : kNoRow;
            m.orow = row * (uint32_t)a.rd_k + (uint32_t)(jr >= 0 ? jr : 0);
            // a weight that underflowed to zero keeps a finite offset, so
            // the record still decays the state
            m.cr = wrt ? l2 - log2f(fmaxf(we, 1.17549435e-38f)) : INFINITY;
            m.w = wr;
        } else {
            m.row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
            m.orow = m.row;
            m.cr = a.lnz2[m.row];
            m.w = 1.f;
        }
    };
    auto meta_store = [&](int64_t chunk, const Meta& m) {
        if (lane < kWsC) {
            const int slot = (int)(chunk % kRing);
            const bool valid = chunk * kWsC + lane < n && (MODE != kModeMasked || m.row != kNoRow);
            // padded records read zeros (buffer loads past the end): no log
            // decay, no key, no value
            sm.mrow[slot][lane] = valid ? m.row * (uint32_t)(CK * 2) : kPadOff;
            sm.mrv[slot][lane] = valid ? m.row * (uint32_t)(DV * 2) : kPadOff;
            sm.mout[slot][lane] = m.orow;
            sm.mcr[slot][lane] = valid ? m.cr : INFINITY;
            sm.mw[slot][lane] = valid ? m.w : -0.f;
        }
    };
    auto is_real = [](float w) { return (__float_as_uint(w) >> 31) == 0u; };

    // ---------------- producer: row loads ----------------
    // lane = (group cg of 4 columns, group gk of RPG consecutive records)
    const int cg = lane % GK::NCG, gk_ = lane / GK::NCG;
    const int j0 = pw * GK::CW + cg * kPC, r0 = gk_ * RPG;
    const int cgv = lane % GV::NCG, gv_ = lane / GV::NCG;
    const int c0v = pw * GV::CW + cgv * kPC, r0v = gv_ * RPGV;
    struct Raw {
        Vec4<bf16_t> q[RPG], k[RPG], l[RPG], v[RPGV];
    };
    // row indices (from the metadata ring) of the next chunk to load, and the
    // read gates / exponent offsets of the next chunk to prepare: read from
    // LDS one step before they are needed
    uint32_t rowq[RPG], rowv[RPGV];
    float gcr[RPG];
    auto read_rows = [&](int64_t chunk) {
        const int slot = (int)(chunk % kRing);
#pragma unroll
        for (int i = 0; i < RPG; i++) rowq[i] = sm.mrow[slot][r0 + i];
#pragma unroll
        for (int i = 0; i < RPGV; i++) rowv[i] = sm.mrv[slot][r0v + i];
    };
    auto read_gates = [&](int64_t chunk) {
        const int slot = (int)(chunk % kRing);
#pragma unroll
        for (int i = 0; i < RPG; i++) gcr[i] = sm.mcr[slot][r0 + i];
    };
    // part 0: log_alpha, 1: key logits, 2: q, 3: v.  Buffer loads at byte
    // offsets (< 2^31, checked on the host), so the rows of padded records
    // (offsets past the end) read as zeros.
    const uint32_t bk = a.rows * (uint32_t)(CK * 2), bv = a.rows * (uint32_t)(DV * 2);
    const __amdgpu_buffer_rsrc_t rsq = make_rsrc(a.q, bk), rsk = make_rsrc(a.kl, bk);
    const __amdgpu_buffer_rsrc_t rsl = make_rsrc(a.la, bk), rsv = make_rsrc(a.v, bv);
    auto raw_load_part = [&](Raw& R, int part) {
        if (part == 3) {
#pragma unroll
            for (int i = 0; i < RPGV; i++) R.v[i].load(rsv, rowv[i] + (uint32_t)(c0v * 2));
            return;
        }
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            const uint32_t off = rowq[i] + (uint32_t)(j0 * 2);
            if (part == 0) R.l[i].load(rsl, off);
            if (part == 1) R.k[i].load(rsk, off);
            if (part == 2) R.q[i].load(rsq, off);
        }
    };
    auto raw_load = [&](Raw& R) {
#pragma unroll
        for (int part = 0; part < 4; part++) raw_load_part(R, part);
    };

    // Inclusive scans of x[e] (e < 4, independent columns) over the record
    // groups of this lane's column group (lanes cg, cg + NCG, ...), plus the
    // totals over all groups.  With 8 column groups (c = 128) the groups are
    // 8 lanes apart, two per 16-lane row: a DPP row shift adds inside rows,
    // then the row-pair and half-wave swaps (v_permlane16/32_swap with one
    // register as both operands: each lane receives its partner row's value)
    // add across rows, with no LDS traffic.  The swaps are inline assembly,
    // four per block with wait states on both sides, since the compiler's
    // model of the swap builtins merges their results and cannot see their
    // hazards.
    auto group_scan4 = [&](const float (&x)[kPC], float (&incl)[kPC], float (&total)[kPC]) {
        if constexpr (GK::NCG == 8) {
            const bool hi8 = (lane & 8) != 0, odd = ((lane >> 4) & 1) != 0, upper = lane >= 32;
            float a1[kPC], rt[kPC], pair[kPC];
            unsigned s16[kPC], s32[kPC];
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                // within the row: the odd group adds the even one; the row
                // total is the odd group's inclusive value
                a1[e] = x[e] + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                             0, __builtin_bit_cast(int, x[e]), 0x118, 0xf, 0xf, false));
                const float sh = __builtin_bit_cast(
                    float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a1[e]), 0x108, 0xf, 0xf, false));
                rt[e] = hi8 ? a1[e] : sh;
                s16[e] = __builtin_bit_cast(unsigned, rt[e]);
            }
            asm volatile("s_nop 4\n\tv_permlane16_swap_b32 %0, %0\n\tv_permlane16_swap_b32 %1, %1\n\t"
                         "v_permlane16_swap_b32 %2, %2\n\tv_permlane16_swap_b32 %3, %3\n\ts_nop 4"
                         : "+v"(s16[0]), "+v"(s16[1]), "+v"(s16[2]), "+v"(s16[3]));
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                pair[e] = rt[e] + __builtin_bit_cast(float, s16[e]);   // rows 0-1 or 2-3
                s32[e] = __builtin_bit_cast(unsigned, pair[e]);
            }
            asm volatile("s_nop 4\n\tv_permlane32_swap_b32 %0, %0\n\tv_permlane32_swap_b32 %1, %1\n\t"
                         "v_permlane32_swap_b32 %2, %2\n\tv_permlane32_swap_b32 %3, %3\n\ts_nop 4"
                         : "+v"(s32[0]), "+v"(s32[1]), "+v"(s32[2]), "+v"(s32[3]));
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                const float other_half = __builtin_bit_cast(float, s32[e]);
                total[e] = pair[e] + other_half;
                incl[e] = a1[e] + (odd ? __builtin_bit_cast(float, s16[e]) : 0.f) + (upper ? other_half : 0.f);
            }
        } else {
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                float inc = x[e];
#pragma unroll
                for (int off = GK::NCG; off < kWave; off <<= 1) {
                    const float y = __shfl_up(inc, off, kWave);
                    if (lane >= off) inc += y;
                }
                incl[e] = inc;
                total[e] = __shfl(inc, kWave - GK::NCG + cg, kWave);
            }
        }
    };

    // ---------------- producer: preparation of one chunk ----------------
    // hook(k), k = 0..3, is called at four points spread over the
    // preparation, so the next chunk's row loads issue between its phases
    // instead of in one burst after the barrier
    auto prep = [&](int64_t chunk, const Raw& R, auto&& hook) {
        auto& st = sm.st[chunk & 1];
        hook(0);
        float run[kPC] = {0.f, 0.f, 0.f, 0.f};
        float bb[RPG][kPC];
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            // masked schedule: a record that is only read does not decay the
            // state (its exponent offset is +inf: it writes nothing either)
            const bool dec = MODE != kModeMasked || gcr[i] != INFINITY;
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                const float x = dec ? R.l[i].get(e) : 0.f;
                run[e] = fmaf(x, kLog2e, run[e]);  // zero for a padded record
                bb[i][e] = run[e];
            }
        }
        hook(1);
        float excl[kPC], ebc_own[kPC], incl[kPC], tot[kPC];
        group_scan4(run, incl, tot);
#pragma unroll
        for (int e = 0; e < kPC; e++) {
            excl[e] = incl[e] - run[e];
            ebc_own[e] = __builtin_amdgcn_exp2f(tot[e]);
        }
        hook(2);
        uint2 pk[RPG][kL];
        const int jp = perm_col(j0);
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            const float cr = gcr[i];
            float xq[kPC], xk[kPC];
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                const float b = bb[i][e] + excl[e];
                xq[e] = R.q[i].get(e) * __builtin_amdgcn_exp2f(b);
                xk[e] = __builtin_amdgcn_exp2f(fmaf(R.k[i].get(e), kLog2e, -cr) - b);
            }
            split4<kL>(xk, pk[i]);
            uint2 pq[kL];
            split4<kL>(xq, pq);
#pragma unroll
            for (int l = 0; l < kL; l++) {
                *reinterpret_cast<uint2*>(&st.q[l][r0 + i][jp]) = pq[l];
                *reinterpret_cast<uint2*>(&st.kr[l][r0 + i][jp ^ rm_swz<CK, kSwz>(r0 + i)]) = pk[i][l];
            }
        }
        hook(3);
        // V rows as loaded (record-major, 4 columns per store)
#pragma unroll
        for (int i = 0; i < RPGV; i++)
            *reinterpret_cast<uint2*>(&st.v[r0v + i][c0v ^ rm_swz<DV, kSwz>(r0v + i)]) = R.v[i].u;
        if (gk_ == 0)
#pragma unroll
            for (int e = 0; e < kPC; e++) sm.ebc[chunk % 3][j0 + e] = ebc_own[e];
    };

    // ---------------- consumer: one software-pipelined iteration ----------------
    // The MFMA work of iteration nn is a fixed list of steps:
    //   F        finish chunk nn-1: Op += A V (A from the previous iteration,
    //            V operand kept in registers); its outputs follow later
    //   A0 ..    this wave's causal 16x16 A tile of chunk nn, one 32-wide k-step
    //            each (waves 0, 1, 2 compute (s-tile, r-tile) = (0,0), (0,1),
    //            (1,1); wave 3 repeats (1,1) and stores the same bits, so no
    //            wave branches; the (1,0) tile is zero and written once)
    //   R0 ..    Oc = Qt S_in, one 16-row k-step each: the B operand is the
    //            state registers (rows 16 kk + {4 hh + e, 8 + 4 hh + e}, e < 4,
    //            = registers 8 (kk%2) + 0..7 of tile kk/2), split into bf16
    //            terms on the fly; the permuted Qt storage puts the matching 8
    //            columns side by side
    //   U0 ..    S += Kh^T V, one (row tile, 16-record k-step) each
    // The decay diag(exp(b_C)) of a chunk is applied lazily: between
    // iterations S holds S_in + Kh^T V of the last chunk, and the readout
    // steps of the next chunk scale each group of 8 state registers just
    // before splitting them.
    // The LDS operands of step s+2 are read while step s runs (three register
    // slots) and scheduling fences keep that order, so LDS latency hides
    // behind the MFMA pipeline.
    const int g16 = lane / 16, l16 = lane % 16;
    const int sT = wv >= 2 ? 1 : 0, rT = wv == 0 ? 0 : 1;
    constexpr int nA = CK / 32, nR = CK / 16, nU = RT_N * 2;
    constexpr int sF = 0, sA = 1, sR = sA + nA, sU = sR + nR, sEnd = sU + nU;
    constexpr int sOut = sA + (nA > 1 ? 1 : 0);   // outputs of chunk nn-1 after this step
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // 32x32x16 MFMA operand over records from a record-major tile: lane l
    // gets records rec0 + 8 (l / 32) + 0..7 of column col0 + l % 32.  Source
    // lane (g, 4e + b) of each 16-lane group addresses the 4-column block
    // col0 + 16 (g % 2) + 4 b of record rec0 + 8 (g / 2) + e (+ 4).
    const int trg = lane / 16, trj = lane % 16;
    const int tr_rec = 8 * (trg / 2) + trj / 4, tr_col = 16 * (trg % 2) + 4 * (trj % 4);
    auto tr_kh = [&](const uint16_t* tile, int rec0, int col0) {   // Kh^T (A operand)
        constexpr int KS = WsStage<CK, DV>::KS;
        const int r = rec0 + tr_rec, c = perm_col(col0 + tr_col);
        return cat_tr(lds_tr(tile + r * KS + (c ^ rm_swz<CK, kSwz>(r))),
                      lds_tr(tile + (r + 4) * KS + (c ^ rm_swz<CK, kSwz>(r + 4))));
    };
    auto tr_v = [&](const uint16_t* tile, int rec0, int col0) {    // V (B operand)
        constexpr int VS = WsStage<CK, DV>::VS;
        const int r = rec0 + tr_rec, c = col0 + tr_col;
        return cat_tr(lds_tr(tile + r * VS + (c ^ rm_swz<DV, kSwz>(r))),
                      lds_tr(tile + (r + 4) * VS + (c ^ rm_swz<DV, kSwz>(r + 4))));
    };

    // operands of step s of iteration nn
    auto fetch = [&](auto sI, int64_t nn, u16x8(&o)[4]) {
        constexpr int s = decltype(sI)::value;
        const auto& st = sm.st[nn & 1];
        if (!(s >= sA && s < sR) && !col_wave) return;  // waves without state columns
        if constexpr (s == sF) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int l = 0; l < kL; l++)
                    o[2 * ks + l] = lds8(&sm.a[(nn - 1) & 1][l][l32][16 * ks + 8 * hh]);
        } else if constexpr (s < sR) {
            constexpr int kk = s - sA;
#pragma unroll
            for (int l = 0; l < kL; l++) {
                o[l] = lds8(&st.kr[l][16 * sT + l16][(32 * kk + 8 * g16) ^ rm_swz<CK, kSwz>(16 * sT + l16)]);
                o[2 + l] = lds8(&st.q[l][16 * rT + l16][32 * kk + 8 * g16]);
            }
        } else if constexpr (s < sU) {
            constexpr int kk = s - sR;
#pragma unroll
            for (int l = 0; l < kL; l++) o[l] = lds8(&st.q[l][l32][16 * kk + 8 * hh]);
            // exp(b_C) of chunk nn-1 for the 8 state rows of this k-step
            const float* d = sm.ebc[(nn + 2) % 3];
            o[2] = *reinterpret_cast<const u16x8*>(&d[16 * kk + 4 * hh]);
            o[3] = *reinterpret_cast<const u16x8*>(&d[16 * kk + 8 + 4 * hh]);
        } else {
            constexpr int u = s - sU, rt = u / 2, ks = u % 2;
#pragma unroll
            for (int l = 0; l < kL; l++) o[l] = tr_kh(&st.kr[l][0][0], 16 * ks, 32 * rt);
        }
    };

    // Outputs of a finished chunk.  The wave's 32 x 32 tile (lane = column,
    // 16 rows in registers) is scaled by the read gates and transposed
    // through LDS, 16 rows at a time, so that each lane holds 4 consecutive
    // columns of one record: tv[p][h2] is record 16 p + 8 h2 + lane / 8,
    // columns 32 wv + 4 (lane % 8) .. +3, and one 16-byte store per value
    // writes whole 128-byte row segments.
    const int trow = lane / 8, tcol = 32 * wv + 4 * (lane % 8);
    // half p (records 16 p .. 16 p + 15) of the transpose
    auto transpose_half = [&](int p, const f32x16& Op, const float4 (&mw4)[4], float4 (&th)[2]) {
        float* xs = &sm.xs[wv][0][0];
#pragma unroll
        for (int i = 8 * p; i < 8 * p + 8; i++) {
            const float4 g = mw4[i / 4];
            const float wr = (i % 4 == 0) ? g.x : (i % 4 == 1) ? g.y : (i % 4 == 2) ? g.z : g.w;
            const int r = 8 * (i / 4) + 4 * hh + (i % 4) - 16 * p;
            xs[r * 32 + l32] = wr * Op[i];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++)
            th[h2] = *reinterpret_cast<const float4*>(&xs[(8 * h2 + trow) * 32 + 4 * (lane % 8)]);
    };
    auto transpose = [&](const f32x16& Op, const float4 (&mw4)[4], float4 (&tv)[2][2]) {
        float* xs = &sm.xs[wv][0][0];
#pragma unroll
        for (int p = 0; p < 2; p++) {
#pragma unroll
            for (int i = 8 * p; i < 8 * p + 8; i++) {
                const float4 g = mw4[i / 4];
                const float wr = (i % 4 == 0) ? g.x : (i % 4 == 1) ? g.y : (i % 4 == 2) ? g.z : g.w;
                const int r = 8 * (i / 4) + 4 * hh + (i % 4) - 16 * p;
                xs[r * 32 + l32] = wr * Op[i];
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                tv[p][h2] = *reinterpret_cast<const float4*>(&xs[(8 * h2 + trow) * 32 + 4 * (lane % 8)]);
        }
    };
    // output row and gate of the records this lane stores
    auto out_rows = [&](int64_t chunk, uint32_t (&orow)[2][2], bool (&oval)[2][2]) {
        const int slot = (int)(chunk % kRing);
#pragma unroll
        for (int p = 0; p < 2; p++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                const int r = 16 * p + 8 * h2 + trow;
                orow[p][h2] = sm.mout[slot][r];
                oval[p][h2] = is_real(sm.mw[slot][r]);
            }
    };
    // 16-byte store of one value to its row (routed: the record's slot row;
    // shared: o), or to the dummy row for a padded record
    auto store_out = [&](float* dst, uint32_t orow, bool valid, const float4& v) {
        const uint32_t off = orow * (uint32_t)(DV * 4) + (uint32_t)(tcol * 4);
        char* base = reinterpret_cast<char*>(valid ? dst : a.trash);
        *reinterpret_cast<float4*>(base + (valid ? off : (uint32_t)(tcol * 4))) = v;
    };
    // Routed slots in block floating point: slot row r holds DV int16 values
    // (a.part, [r][DV]) and one fp32 step per 32-column group (a.part_scale,
    // [r][DV/32]): value = int16 * step.  A group is one consumer wave's
    // columns of one record, 8 lanes x 4 values; with 2^e the smallest power
    // of two above the group's largest magnitude, the values are scaled by
    // 2^-e into (-1, 1) and converted to normalised int16, step 2^e/32767, so
    // every value is stored within one step, below 2^-14 of that magnitude.
    struct SlotQ {
        uint2 q;      // 4 int16 values
        float step;
    };
    auto slot_encode = [&](const float4& v) {
        // largest magnitude over the 8 lanes of the group (quad swaps, then
        // the half-row mirror), compared as bit patterns (non-negative floats
        // order like their bits)
        uint32_t m = __float_as_uint(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        auto dpp = [](uint32_t x, auto ctrl) {
            return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xf, 0xf, false);
        };
        m = max(m, dpp(m, std::integral_constant<int, 0xb1>{}));
        m = max(m, dpp(m, std::integral_constant<int, 0x4e>{}));
        m = max(m, dpp(m, std::integral_constant<int, 0x141>{}));
        const int e = __builtin_amdgcn_frexp_expf(__uint_as_float(m));  // max < 2^e (e = 0 for 0)
        SlotQ r;
        r.q.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(
                                                 __builtin_amdgcn_ldexpf(v.x, -e), __builtin_amdgcn_ldexpf(v.y, -e)));
        r.q.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(
                                                 __builtin_amdgcn_ldexpf(v.z, -e), __builtin_amdgcn_ldexpf(v.w, -e)));
        r.step = __builtin_amdgcn_ldexpf(1.f / 32767.f, e);
        return r;
    };
    // slot row of record row `orow` and rank j (shared pass): orow*topk + j
    auto slot_ld = [&](uint32_t orow, int j) {
        const uint32_t srow = orow * (uint32_t)a.topk + (uint32_t)j;
        SlotQ r;
        r.q = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(a.part) +
                                              srow * (uint32_t)(DV * 2) + (uint32_t)(tcol * 2));
        r.step = a.part_scale[srow * (uint32_t)(DV / 32) + (uint32_t)wv];
        return r;
    };
    auto slot_add = [](float4& v, const SlotQ& r) {
        v.x = fmaf((float)(int)(int16_t)(r.q.x & 0xffffu), r.step, v.x);
        v.y = fmaf((float)((int)r.q.x >> 16), r.step, v.y);
        v.z = fmaf((float)(int)(int16_t)(r.q.y & 0xffffu), r.step, v.z);
        v.w = fmaf((float)((int)r.q.y >> 16), r.step, v.w);
    };
    // routed pass: the record's slot row, or the spare row past the last
    // one when the record is padding; the 8 lanes of a group all store its
    // step (same value, same address)
    auto slot_store = [&](uint32_t orow, bool valid, const float4& v) {
        const SlotQ r = slot_encode(v);
        const uint32_t srow = valid ? orow : a.slot_rows;
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(a.part) + srow * (uint32_t)(DV * 2) +
                                  (uint32_t)(tcol * 2)) = r.q;
        a.part_scale[srow * (uint32_t)(DV / 32) + (uint32_t)wv] = r.step;
    };
    constexpr int kPre = 2;  // slots per record prefetched before the shared outputs
    // Iteration nn (PREV: finish chunk nn-1; CUR: run chunk nn).  Op holds
    // the readout of chunk nn-1 and Vp its V operand; Oc and Vc receive those
    // of chunk nn.
    auto iteration = [&](auto prevI, auto curI, int64_t nn, f32x16& Op, u16x8(&Vp)[2], f32x16& Oc,
                         u16x8(&Vc)[2]) {
        constexpr bool HASPREV = decltype(prevI)::value;   // S holds chunk nn-1 undecayed
        constexpr bool PREV = HASPREV;
        constexpr bool CUR = decltype(curI)::value;
        const auto& st = sm.st[nn & 1];
        u16x8 ob[3][4];
        float4 mw4[4];
        uint32_t orow[2][2];
        bool oval[2][2];
        float4 tv[2][2];
        SlotQ pre[2][2][kPre];
        f32x4 Aacc = {0.f, 0.f, 0.f, 0.f};
        auto fetch_extra = [&](auto sI) {
            constexpr int s = decltype(sI)::value;
            if (!col_wave) return;
            // the shared pass needs the output rows early, for its slot loads
            if constexpr (s == sF && PREV && MODE == kModeShared) out_rows(nn - 1, orow, oval);
            if constexpr (CUR && s == sR) {
#pragma unroll
                for (int ks = 0; ks < 2; ks++) Vc[ks] = tr_v(&st.v[0][0], 16 * ks, 32 * wv);
            }
        };
        auto compute = [&](auto sI, const u16x8(&o)[4]) {
            constexpr int s = decltype(sI)::value;
            if (!(s >= sA && s < sR) && !col_wave) return;  // waves without state columns
            if constexpr (s == sF) {
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    const u16x8 aa[kL] = {o[2 * ks], o[2 * ks + 1]};
                    const u16x8 vb[1] = {Vp[ks]};
                    mma32_terms<kL, 1>(aa, vb, Op);
                }
            } else if constexpr (s < sR) {
                const u16x8 ka[kL] = {o[0], o[1]}, qb[kL] = {o[2], o[3]};
                mma16_terms<kL, kL>(ka, qb, Aacc);
            } else if constexpr (s < sU) {
                constexpr int kk = s - sR;
                if constexpr (kk == 0)
#pragma unroll
                    for (int i = 0; i < 16; i++) Oc[i] = 0.f;
                if constexpr (HASPREV) {
                    // S_in of this chunk = diag(exp(b_C) of chunk nn-1) S'
                    const float4 d0 = __builtin_bit_cast(float4, o[2]);
                    const float4 d1 = __builtin_bit_cast(float4, o[3]);
                    const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                    for (int e = 0; e < 8; e++) S[kk / 2][8 * (kk % 2) + e] *= dd[e];
                }
                u16x8 sb[kL];
                uint32_t pr[4][kL];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++)
                    split_pair<kL>(S[kk / 2][8 * (kk % 2) + 2 * e2], S[kk / 2][8 * (kk % 2) + 2 * e2 + 1],
                                   pr[e2]);
#pragma unroll
                for (int l = 0; l < kL; l++)
                    sb[l] = __builtin_bit_cast(u16x8, make_uint4(pr[0][l], pr[1][l], pr[2][l], pr[3][l]));
                const u16x8 qa[kL] = {o[0], o[1]};
                mma32_terms<kL, kL>(qa, sb, Oc);
            } else {
                constexpr int u = s - sU, rt = u / 2, ks = u % 2;
                const u16x8 ka[kL] = {o[0], o[1]};
                const u16x8 vb[1] = {Vc[ks]};
                mma32_terms<kL, 1>(ka, vb, S[rt]);
            }
        };
        // work that waits for an earlier step's MFMA results
        // shared pass: o = shared read + the record's routed slots.  In an
        // iteration that also runs a chunk, slots 0 .. kPre-1 (loaded at step
        // sF) are added at step sU and slots kPre .. 2 kPre - 1 are loaded
        // there into the same registers, so up to 2 kPre slots arrive without
        // a wait; further slots are loaded where they are added.
        auto shared_store = [&](auto midI) {
            constexpr bool MID = decltype(midI)::value;  // slots 0 .. kPre-1 already in tv
            constexpr int j0 = MID ? kPre : 0;
#pragma unroll
            for (int p = 0; p < 2; p++)
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    float4 v = tv[p][h2];
#pragma unroll
                    for (int j = 0; j < kPre; j++)
                        if (j0 + j < a.topk) slot_add(v, pre[p][h2][j]);
                    for (int j = j0 + kPre; j < a.topk; j++) slot_add(v, slot_ld(orow[p][h2], j));
                    store_out(a.o, orow[p][h2], oval[p][h2], v);
                }
        };
        auto after = [&](auto sI) {
            constexpr int s = decltype(sI)::value;
            if constexpr (PREV && MODE == kModeShared && s == sF) {
                // the first kPre slots of the finished records, consumed at
                // the end of the iteration
                if (col_wave)
#pragma unroll
                    for (int p = 0; p < 2; p++)
#pragma unroll
                        for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                            for (int j = 0; j < kPre; j++)
                                pre[p][h2][j] = slot_ld(orow[p][h2], j < a.topk ? j : 0);
            }
            if constexpr (PREV && s == (CUR ? sOut : sF)) {
                if (col_wave) {
                    const int slot = (int)((nn - 1) % kRing);
#pragma unroll
                    for (int q4 = 0; q4 < 4; q4++)
                        mw4[q4] = *reinterpret_cast<const float4*>(&sm.mw[slot][8 * q4 + 4 * hh]);
                    if constexpr (kPart) {
                        out_rows(nn - 1, orow, oval);
#pragma unroll
                        for (int p = 0; p < 2; p++) {
                            float4 th[2];
                            transpose_half(p, Op, mw4, th);
#pragma unroll
                            for (int h2 = 0; h2 < 2; h2++) slot_store(orow[p][h2], oval[p][h2], th[h2]);
                        }
                    } else {
                        transpose(Op, mw4, tv);
                        if constexpr (!CUR) shared_store(std::false_type{});
                    }
                }
            }
            if constexpr (PREV && CUR && MODE == kModeShared && s == sU) {
                if (col_wave) {
#pragma unroll
                    for (int p = 0; p < 2; p++)
#pragma unroll
                        for (int h2 = 0; h2 < 2; h2++) {
#pragma unroll
                            for (int j = 0; j < kPre; j++)
                                if (j < a.topk) slot_add(tv[p][h2], pre[p][h2][j]);
                            if (a.topk > kPre)
#pragma unroll
                                for (int j = 0; j < kPre; j++)
                                    pre[p][h2][j] = slot_ld(orow[p][h2], kPre + j < a.topk ? kPre + j : 0);
                        }
                }
            }
            if constexpr (PREV && CUR && MODE == kModeShared && s == sEnd - 1)
                if (col_wave) shared_store(std::true_type{});
            if constexpr (CUR && s == sR) {
                // causal mask, bf16 terms, store of this wave's A tile
                const int r = 16 * rT + l16, s0 = 16 * sT + 4 * g16;
                if (sT == rT) {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (s0 + i > r) Aacc[i] = 0.f;
                }
                uint32_t p01[kL], p23[kL];
                split_pair<kL>(Aacc[0], Aacc[1], p01);
                split_pair<kL>(Aacc[2], Aacc[3], p23);
#pragma unroll
                for (int l = 0; l < kL; l++)
                    *reinterpret_cast<uint2*>(&sm.a[nn & 1][l][r][s0]) = make_uint2(p01[l], p23[l]);
            }
        };
        // Steps first .. last run in order (all of them enabled); the
        // operands of step s+2 are read after step s is issued.
        constexpr int first = PREV ? sF : sA;
        constexpr int last = CUR ? sEnd - 1 : sF;
        static_for<first, (first + 2 <= last + 1 ? first + 2 : last + 1)>([&](auto sI) {
            constexpr int s = decltype(sI)::value;
            fetch(sI, nn, ob[s % 3]);
            fetch_extra(sI);
        });
        fence();
        static_for<first, last + 1>([&](auto sI) {
            constexpr int s = decltype(sI)::value;
            compute(sI, ob[s % 3]);
            after(sI);
            if constexpr (s + 2 <= last) {
                constexpr std::integral_constant<int, s + 2> nI{};
                fetch(nI, nn, ob[(s + 2) % 3]);
                fetch_extra(nI);
            }
            fence();
        });
    };

    // ---------------- pipeline ----------------
    // Producers and consumers run separate loops (so their registers are not
    // live at the same time) with the same barriers: two in the prologue and
    // one per iteration nn = 0 .. nchunks.
    if (nchunks > 0) {
        if (producer) {
            // Every producer wave issues the same loads in every step (chunks
            // past the end re-load clamped, valid rows), so the compiler can
            // count the loads in flight and wait only for the ones it uses.
            Raw R0, R1, R2;
            Meta M0, M1, M2;
            for (int c = 0; c < 5; c++) {
                meta_load(c, M0);
                if (pw == 0) meta_store(c, M0);
            }
            lds_barrier();
            meta_load(5, M2);
            read_rows(0);
            raw_load(R0);
            read_rows(1);
            raw_load(R1);
            read_rows(2);
            raw_load(R2);
            read_rows(3);
            read_gates(0);
            prep(0, R0, [](int) {});
            read_gates(1);
            lds_barrier();
            // Step nn: issue the metadata loads of chunk nn+6 (first: the
            // counter of outstanding loads is in order, so waiting for them
            // next step must not also wait for this step's row loads);
            // prepare chunk nn+1 (gates read last step) while issuing the row
            // loads of chunk nn+3 between its phases (rows read last step;
            // chunk c's rows live in R[c % 3], so every load has two steps to
            // arrive); read the rows of chunk nn+4 and the gates of chunk
            // nn+2; store the metadata of chunk nn+5.
            auto step = [&](int64_t nn, Raw& Rl, const Raw& Rp, Meta& Ml, const Meta& Ms) {
                meta_load(nn + 6, Ml);
                auto hook = [&](int part) {
                    __builtin_amdgcn_sched_barrier(0);
                    raw_load_part(Rl, part);
                    __builtin_amdgcn_sched_barrier(0);
                };
                if (nn + 1 < nchunks)
                    prep(nn + 1, Rp, hook);
                else
                    raw_load(Rl);
                read_rows(nn + 4);
                read_gates(nn + 2);
                if (pw == 0) meta_store(nn + 5, Ms);
                lds_barrier();
            };
            int64_t nn = 0;
            for (; nn + 2 <= nchunks; nn += 3) {
                step(nn, R0, R1, M0, M2);
                step(nn + 1, R1, R2, M1, M0);
                step(nn + 2, R2, R0, M2, M1);
            }
            if (nn <= nchunks) step(nn, R0, R1, M0, M2);
            if (nn + 1 <= nchunks) step(nn + 1, R1, R2, M1, M0);
        } else {
            if (wv == 3) {
                // the zero (r-tile 0, s-tile 1) block of A in both buffers
                for (int i = lane; i < 2 * kL * 16; i += kWave) {
                    const int b = i / (kL * 16), l = (i / 16) % kL, r = i % 16;
                    *reinterpret_cast<uint4*>(&sm.a[b][l][r][16]) = make_uint4(0, 0, 0, 0);
                    *reinterpret_cast<uint4*>(&sm.a[b][l][r][24]) = make_uint4(0, 0, 0, 0);
                }
            }
            // the producers' two prologue barriers
            lds_barrier();
            lds_barrier();
            // iteration 0 runs chunk 0; iterations 1 .. nchunks-1 finish the
            // previous chunk and run the next (unrolled by two so the readout
            // and V registers alternate without copies); the last iteration
            // finishes chunk nchunks-1.
            using T_ = std::true_type;
            using F_ = std::false_type;
            f32x16 O0, O1;
            u16x8 V0[2], V1[2];
            iteration(F_{}, T_{}, 0, O1, V1, O0, V0);
            lds_barrier();
            int64_t nn = 1;
            for (; nn + 1 < nchunks; nn += 2) {
                iteration(T_{}, T_{}, nn, O0, V0, O1, V1);
                lds_barrier();
                iteration(T_{}, T_{}, nn + 1, O1, V1, O0, V0);
                lds_barrier();
            }
            if (nn < nchunks) {
                iteration(T_{}, T_{}, nn, O0, V0, O1, V1);
                lds_barrier();
                iteration(T_{}, F_{}, nn + 1, O1, V1, O0, V0);
            } else {
                iteration(T_{}, F_{}, nn, O0, V0, O1, V1);
            }
            lds_barrier();
        }
    }

    // ---------------- results ----------------
    // the state still lacks the decay of the last chunk
    if (col_wave && nchunks > 0) {
        const float* d = sm.ebc[(nchunks - 1) % 3];
#pragma unroll
        for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
            for (int i = 0; i < 16; i++) S[rt][i] *= d[32 * rt + 8 * (i / 4) + 4 * hh + (i % 4)];
    }
    if (col_wave && last_piece) {
#pragma unroll
        for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                a.final_states[sbase + (int64_t)row * DV + col] = S[rt][i];
            }
    }
}

// ============================ launcher ============================
namespace {

template <int CK, int DV, int MODE>
void launch_ws_cfg(const ChunkArgs& a, hipStream_t st) {
    dim3 grid;
    if (MODE == kModeRouted && a.rpiece_len > 0)
        grid = dim3((unsigned)(a.num_seqs * a.H * a.N), (unsigned)a.rmax_pieces);
    else if (MODE != kModeShared)
        grid = dim3((unsigned)(a.num_seqs * a.H * a.N));
    else
        grid = dim3((unsigned)(a.num_seqs * a.H), (unsigned)a.max_pieces);
    if (grid.x == 0 || grid.y == 0) return;
    chunk_ws_kernel<CK, DV, MODE><<<grid, kWsThreads, 0, st>>>(a);
}

template <int MODE>
bool launch_ws_shape(const ChunkArgs& a, int c, int d, hipStream_t st) {
#define SSE_WS_CASE(CC, DD)                      \
    if (c == CC && d == DD) {                    \
        launch_ws_cfg<CC, DD, MODE>(a, st);      \
        return true;                             \
    }
    SSE_WS_CASE(32, 32) SSE_WS_CASE(32, 64) SSE_WS_CASE(32, 128)
    SSE_WS_CASE(64, 32) SSE_WS_CASE(64, 64) SSE_WS_CASE(64, 128)
    SSE_WS_CASE(128, 32) SSE_WS_CASE(128, 64) SSE_WS_CASE(128, 128)
#undef SSE_WS_CASE
    return false;
}

}  // namespace

hipError_t launch_chunk_ws(int mode, const ChunkArgs& a, int c, int d, hipStream_t st) {
    if ((int64_t)a.num_seqs * a.H == 0) return hipSuccess;
    bool ok = false;
    if (mode == kModeShared)
        ok = launch_ws_shape<kModeShared>(a, c, d, st);
    else if (mode == kModeRouted)
        ok = launch_ws_shape<kModeRouted>(a, c, d, st);
    else if (mode == kModeMasked)
        ok = launch_ws_shape<kModeMasked>(a, c, d, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace sse
