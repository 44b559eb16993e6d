// chunk_gla.hip -- chunked gated linear attention over partition segments
// (routed and shared) for gfx950: MFMA bf16 with fp32 state.
//
// Method: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记".
// A routed partition's state only moves on the records that select it (§2.6:
// identity transition elsewhere; §2.4: the partition keeps its own clock), so
// each (sequence, head, partition) segment of records is an ordinary gated
// linear attention (§2.1 eq. 6, diagonal decay) over its own subsequence, with
// the router probability w gating both the write and the read (§2.3, eqs.
// 12-14).  The shared partition (§2.5) is the segment of all tokens with w = 1.
// Every token's k+1 partition reads are summed into o (§2.6, gated sum back to
// the token): the shared pass stores o, the routed pass adds into it.
//
// Chunked form, for a chunk of C records r = 0..C-1 with b_r = sum_{u<=r}
// log_alpha_u (per state row j, within the chunk), b_C = b at the last record:
//   Qt[r,j]  = q[r,j] exp(b[r,j])
//   Kh[s,j]  = w_s kappa[s,j] exp(-b[s,j])
//   A[r,s]   = (Qt Kh^T)[r,s] for s <= r, else 0      (the own write is read)
//   O        = w_r (A V + Qt S_in)
//   S_out    = diag(exp(b_C)) (S_in + Kh^T V)
// which is the token recurrence unrolled over the chunk.  kappa comes from the
// per-token normaliser stored by the router pass (w kappa exp(-b) is one exp2
// of kl log2e - cr - b with cr = lnz2 - log2 w), so no row reduction is needed.
//
// Precision: MFMA takes bf16 operands; each operand that is not exactly a bf16
// value is carried as LV bf16 terms (x = t0 + t1 + ...) and the products of
// term pairs with level sum < LV are accumulated in fp32.  LV = 2 for bf16
// inputs (q and v exact, ~16-bit products), LV = 3 for fp32 inputs (~24-bit).
//
// Long chains: a shared segment is cut into pieces of piece_len records.  A
// pre-pass (mode Local) computes each piece's local state (from zero) and its
// decay product; a piece then starts from
//   S_in(p) = D_{p-1} (... (D_0 S_init + S_loc(0)) ...) + S_loc(p-1)
// so all pieces run in parallel.
//
// Block = 4 waves, one piece (shared) or segment (routed), all of d, chunks of
// C = 32 records.  Wave w owns state and
// output columns [32w, 32w+32) (c x 32 fp32 in MFMA accumulator layout) and
// prepares key/query columns [w c/4, (w+1) c/4) for all records of a chunk:
// lane = (group of 4 columns, group of consecutive records), so the decay
// cumsum is in-lane plus a short cross-lane scan and every LDS store is a
// vector store.  Two blocks share a CU (LDS ~72 KB, <= 256 registers per
// lane), so one block's MFMA phase overlaps the other's element-wise work and
// memory waits.  The loads of chunk n+1 are issued a whole iteration ahead and
// before chunk n's output stores, and the barriers wait only for LDS traffic,
// so global loads and output atomics stay in flight across them.
#include "chunk_common.h"

namespace sse {

namespace {

template <int C, int CK, int DV, int LV, int LVV>
struct Smem {
    static constexpr int QS = CK + 8;   // record-major row stride (elements)
    static constexpr int TS = C + 8;    // record-minor row stride (elements)
    uint16_t q[LV][C][QS];              // Qt terms [r][j]
    uint16_t kr[LV][C][QS];             // Kh terms [s][j]
    uint16_t kt[LV][CK][TS];            // Kh terms [j][s]
    uint16_t vt[LVV][DV][TS];           // V terms [col][s]
    uint16_t a[LV][C][TS];              // A terms [r][s]
    float ebc[CK];                      // exp(b_C) per state row
    uint32_t mrow[3][C];                // record row t*H + h (a real row even if padded)
    uint32_t mout[3][C];                // output row: routed slot row or t*H + h
    float mcr[3][C];                    // exponent offset lnz2 - log2 w (+inf if padded)
    float mw[3][C];                     // read gate; -0.0 marks a padded record
};

}  // namespace

// Blocks per CU the register allocation targets: two when the LDS of two
// blocks fits in the 160 KB of a CU (each SIMD then runs two waves that hide
// each other's LDS and memory latency), else one.
template <int C, int CK, int DV, int LV, int LVV>
constexpr int kMinBlocks = sizeof(Smem<C, CK, DV, LV, LVV>) <= 80 * 1024 ? 2 : 1;

template <int C, int CK, int DV, int LV, int LVV, typename TIn, int MODE>
__global__ __launch_bounds__(kThreads, (kMinBlocks<C, CK, DV, LV, LVV>)) void chunk_kernel(
    const ChunkArgs a) {
    using SM = Smem<C, CK, DV, LV, LVV>;
    using GK = Geo<C, CK>;
    using GV = Geo<C, DV>;
    constexpr bool kLocal = MODE == kModeLocal;
    constexpr int kOT = C / 32;          // 32-record output tiles
    constexpr int NS = DV / 32;          // column waves
    constexpr int RT_N = CK / 32;        // 32-row tiles of the state
    __shared__ __attribute__((aligned(16))) SM sm;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int hh = lane / 32, l32 = lane % 32;
    const int H = a.H, N = a.N;
    const bool col_wave = NS == kNW || wv < NS;  // this wave owns state columns

    // ---------------- which records this block runs ----------------
    int s, h, part, piece = 0, npieces = 1;
    int64_t lo, n;
    if constexpr (MODE == kModeRouted) {
        const int g = blockIdx.x;
        part = g % N;
        s = g / N / H;
        h = g / N % H;
        lo = a.seg_offsets[g];
        n = a.seg_offsets[g + 1] - lo;
    } else {
        const int sh = blockIdx.x;
        s = sh / H;
        h = sh % H;
        part = N;
        piece = blockIdx.y;
        const int64_t t0 = a.cu[s], len = a.cu[s + 1] - t0;
        npieces = len > 0 ? (int)((len + a.piece_len - 1) / a.piece_len) : 1;
        if (piece >= npieces - (kLocal ? 1 : 0)) return;  // uniform
        lo = t0 + (int64_t)piece * a.piece_len;
        n = min<int64_t>(a.piece_len, len - (int64_t)piece * a.piece_len);
        if (n < 0) n = 0;
    }
    const int64_t nchunks = (n + C - 1) / C;
    const bool last_piece = piece == npieces - 1;
    const int64_t sbase = (((int64_t)s * H + h) * (N + 1) + part) * CK * DV;
    const int64_t abase = ((int64_t)s * H + h) * a.max_pieces;

    const TIn* __restrict__ gq = static_cast<const TIn*>(a.q);
    const TIn* __restrict__ gk = static_cast<const TIn*>(a.kl);
    const TIn* __restrict__ gv = static_cast<const TIn*>(a.v);
    const TIn* __restrict__ gl = static_cast<const TIn*>(a.la);

    // ---------------- initial state of this wave's column slice ----------------
    // rows 32 rt + 8 (i/4) + 4 hh + i%4, column 32 wv + l32
    f32x16 S[RT_N];
#pragma unroll
    for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
        for (int i = 0; i < 16; i++) S[rt][i] = 0.f;
    if (col_wave && !kLocal) {
        const int col = 32 * wv + l32;
        if (a.init) {
#pragma unroll
            for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                    S[rt][i] = a.init[sbase + (int64_t)row * DV + col];
                }
        }
        // S_in(p) = D_{p-1} S_in(p-1) + S_loc(p-1), from the local-state pass
        for (int p = 0; p < piece; p++) {
            const int64_t ab = abase + p;
#pragma unroll
            for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                    S[rt][i] = a.agg_D[ab * CK + row] * S[rt][i] +
                               a.agg_S[(ab * CK + row) * DV + col];
                }
        }
    }

    // ---------------- metadata of one chunk ----------------
    // Every thread loads (record index tid % C, clamped into the piece) so the
    // loads carry no branch; threads < C store it after the next barrier.
    // Padded records keep a real row (so every address stays valid) and are
    // marked by a read gate of -0.0.
    auto meta_load = [&](int64_t chunk, uint32_t& row, uint32_t& orow, float& cr, float& w) {
        const int64_t idx = chunk * C + (tid % C);
        const int64_t ci = idx < n ? idx : (n > 0 ? n - 1 : 0);
        if constexpr (MODE == kModeRouted) {
            const uint4 r = *reinterpret_cast<const uint4*>(a.seg_rec + (lo + ci));
            row = r.x;
            orow = r.y;
            cr = __uint_as_float(r.z);
            w = __uint_as_float(r.w);
        } else {
            row = (uint32_t)(lo + ci) * (uint32_t)H + (uint32_t)h;
            orow = row;
            cr = a.lnz2[row];
            w = 1.f;
        }
    };
    auto meta_store = [&](int64_t chunk, int buf, uint32_t row, uint32_t orow, float cr, float w) {
        const bool valid = chunk * C + tid < n;
        sm.mrow[buf][tid] = row;
        sm.mout[buf][tid] = orow;
        sm.mcr[buf][tid] = valid ? cr : INFINITY;
        sm.mw[buf][tid] = valid ? w : -0.f;
    };
    auto is_real = [](float w) { return (__float_as_uint(w) >> 31) == 0u; };

    // ---------------- raw loads of one chunk into registers ----------------
    constexpr int RPG = GK::RPG, RPGV = GV::RPG;
    const int cg = lane % GK::NCG, gk_ = lane / GK::NCG;
    const int j0 = wv * GK::CW + cg * kPC, r0 = gk_ * RPG;
    const int cgv = lane % GV::NCG, gv_ = lane / GV::NCG;
    const int c0v = wv * GV::CW + cgv * kPC, r0v = gv_ * RPGV;
    Vec4<TIn> rq[RPG], rk[RPG], rl[RPG], rv[RPGV];
    auto raw_load_qkl = [&](int buf) {
        // byte offsets fit in 32 bits (checked on the host): scalar base +
        // 32-bit vector offset addressing
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            const uint32_t off = sm.mrow[buf][r0 + i] * (uint32_t)(CK * sizeof(TIn)) +
                                 (uint32_t)(j0 * sizeof(TIn));
            if constexpr (!kLocal) rq[i].load(gq, off);
            rk[i].load(gk, off);
            rl[i].load(gl, off);
        }
    };
    auto raw_load_v = [&](int buf) {
#pragma unroll
        for (int i = 0; i < RPGV; i++)
            rv[i].load(gv, sm.mrow[buf][r0v + i] * (uint32_t)(DV * sizeof(TIn)) +
                               (uint32_t)(c0v * sizeof(TIn)));
    };

    // ---------------- element-wise preparation into registers ----------------
    uint2 pq[RPG][LV], pk[RPG][LV];
    float ebc_own[kPC];
    float btot[kPC] = {0.f, 0.f, 0.f, 0.f};
    auto prep = [&](int buf) {
        float run[kPC] = {0.f, 0.f, 0.f, 0.f};
        float bb[RPG][kPC];
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            const bool valid = is_real(sm.mw[buf][r0 + i]);
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                const float x = valid ? rl[i].get(e) : 0.f;
                run[e] = fmaf(x, kLog2e, run[e]);
                bb[i][e] = run[e];
            }
        }
        float excl[kPC];
#pragma unroll
        for (int e = 0; e < kPC; e++) {
            float inc = run[e];
#pragma unroll
            for (int off = GK::NCG; off < kWave; off <<= 1) {
                const float y = __shfl_up(inc, off, kWave);
                if (lane >= off) inc += y;
            }
            excl[e] = inc - run[e];
            const float tot = __shfl(inc, kWave - GK::NCG + cg, kWave);
            ebc_own[e] = __builtin_amdgcn_exp2f(tot);
            if constexpr (kLocal) btot[e] += tot;
        }
#pragma unroll
        for (int i = 0; i < RPG; i++) {
            const float cr = sm.mcr[buf][r0 + i];
            float xq[kPC], xk[kPC];
#pragma unroll
            for (int e = 0; e < kPC; e++) {
                const float b = bb[i][e] + excl[e];
                if constexpr (!kLocal) xq[e] = rq[i].get(e) * __builtin_amdgcn_exp2f(b);
                xk[e] = __builtin_amdgcn_exp2f(fmaf(rk[i].get(e), kLog2e, -cr) - b);
            }
            if constexpr (!kLocal) split4<LV>(xq, pq[i]);
            split4<LV>(xk, pk[i]);
        }
    };
    auto prep_store = [&]() {
#pragma unroll
        for (int i = 0; i < RPG; i++)
#pragma unroll
            for (int l = 0; l < LV; l++) {
                if constexpr (!kLocal) {
                    *reinterpret_cast<uint2*>(&sm.q[l][r0 + i][j0]) = pq[i][l];
                    *reinterpret_cast<uint2*>(&sm.kr[l][r0 + i][j0]) = pk[i][l];
                }
            }
#pragma unroll
        for (int e = 0; e < kPC; e++)
#pragma unroll
            for (int l = 0; l < LV; l++) {
                uint16_t run[RPG];
#pragma unroll
                for (int i = 0; i < RPG; i++) run[i] = elem(pk[i][l], e);
                store_run<RPG>(&sm.kt[l][j0 + e][r0], run);
            }
        // V^T terms
#pragma unroll
        for (int e = 0; e < kPC; e++) {
            if constexpr (LVV == 1) {
                uint16_t run[RPGV];
#pragma unroll
                for (int i = 0; i < RPGV; i++) run[i] = rv[i].bits(e);
                store_run<RPGV>(&sm.vt[0][c0v + e][r0v], run);
            } else {
                uint16_t run[LVV][RPGV];
#pragma unroll
                for (int i = 0; i < RPGV; i++) {
                    float x = rv[i].get(e);
#pragma unroll
                    for (int l = 0; l < LVV; l++) {
                        run[l][i] = f32_to_bf16_bits(x);
                        if (l + 1 < LVV) x -= bf16_bits_to_f32(run[l][i]);
                    }
                }
#pragma unroll
                for (int l = 0; l < LVV; l++) store_run<RPGV>(&sm.vt[l][c0v + e][r0v], run[l]);
            }
        }
        if (gk_ == 0)
#pragma unroll
            for (int e = 0; e < kPC; e++) sm.ebc[j0 + e] = ebc_own[e];
    };

    // ---------------- causal A tiles (16x16x32 MFMA) ----------------
    const int g16 = lane / 16, l16 = lane % 16;
    auto a_tiles = [&]() {
        constexpr int kTiles = (C / 16) * (C / 16 + 1) / 2 + C / 32;
        constexpr int kTPW = (kTiles + kNW - 1) / kNW;
#pragma unroll
        for (int u = 0; u < kTPW; u++) {
            const int ti = wv + kNW * u;
            if (ti >= kTiles) break;  // uniform per wave
            int st, rt;
            a_tile<C>(ti, st, rt);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (st <= rt) {
#pragma unroll
                for (int kk = 0; kk < CK / 32; kk++) {
                    u16x8 ka[LV], qb[LV];
#pragma unroll
                    for (int l = 0; l < LV; l++) {
                        ka[l] = lds8(&sm.kr[l][16 * st + l16][32 * kk + 8 * g16]);
                        qb[l] = lds8(&sm.q[l][16 * rt + l16][32 * kk + 8 * g16]);
                    }
                    mma16_terms<LV, LV>(ka, qb, acc);
                }
                // lane holds r = 16 rt + l16 and s = 16 st + 4 g16 + i; keep s <= r
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (16 * st + 4 * g16 + i > 16 * rt + l16) acc[i] = 0.f;
            }
            const int r = 16 * rt + l16, s0 = 16 * st + 4 * g16;
            uint32_t p01[LV], p23[LV];
            split_pair<LV>(acc[0], acc[1], p01);
            split_pair<LV>(acc[2], acc[3], p23);
#pragma unroll
            for (int l = 0; l < LV; l++)
                *reinterpret_cast<uint2*>(&sm.a[l][r][s0]) = make_uint2(p01[l], p23[l]);
        }
    };

    // ---------------- MFMA phase of one chunk ----------------
    f32x16 O[kOT];
    const int col = 32 * wv + l32;
    const uint32_t col4 = 4u * (uint32_t)col;
    auto mma_out = [&]() {
        if constexpr (!kLocal) {
#pragma unroll
            for (int t = 0; t < kOT; t++)
#pragma unroll
                for (int i = 0; i < 16; i++) O[t][i] = 0.f;
            // O += Qt S_in: the B operand is this wave's state registers; k-step
            // kk uses rows 16kk + {4hh+e, 8+4hh+e} (e < 4) = registers
            // 8 (kk%2) + 0..7 of tile kk/2.
#pragma unroll
            for (int kk = 0; kk < CK / 16; kk++) {
                u16x8 sb[LV];
                {
                    uint32_t pr[4][LV];
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2++)
                        split_pair<LV>(S[kk / 2][8 * (kk % 2) + 2 * e2],
                                       S[kk / 2][8 * (kk % 2) + 2 * e2 + 1], pr[e2]);
#pragma unroll
                    for (int l = 0; l < LV; l++)
                        sb[l] = __builtin_bit_cast(
                            u16x8, make_uint4(pr[0][l], pr[1][l], pr[2][l], pr[3][l]));
                }
                const int jq = 16 * kk + 4 * hh;
#pragma unroll
                for (int t2 = 0; t2 < kOT; t2++) {
                    const int r = 32 * t2 + l32;
                    u16x8 qa[LV];
#pragma unroll
                    for (int l = 0; l < LV; l++) qa[l] = lds4x2(&sm.q[l][r][jq], &sm.q[l][r][jq + 8]);
                    mma32_terms<LV, LV>(qa, sb, O[t2]);
                }
            }
            // O += A V (row tile t2 needs s < 32 (t2 + 1))
#pragma unroll
            for (int t2 = 0; t2 < kOT; t2++)
#pragma unroll
                for (int ks = 0; ks < 2 * (t2 + 1); ks++) {
                    const int r = 32 * t2 + l32, s0 = 16 * ks + 8 * hh;
                    u16x8 aa[LV], vb[LVV];
#pragma unroll
                    for (int l = 0; l < LV; l++) aa[l] = lds8(&sm.a[l][r][s0]);
#pragma unroll
                    for (int l = 0; l < LVV; l++) vb[l] = lds8(&sm.vt[l][col][s0]);
                    mma32_terms<LV, LVV>(aa, vb, O[t2]);
                }
        }
    };
    // S_out = diag(exp(b_C)) (S_in + Kh^T V)
    auto mma_state = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT_N; rt++) {
#pragma unroll
            for (int ks = 0; ks < C / 16; ks++) {
                const int j = 32 * rt + l32, s0 = 16 * ks + 8 * hh;
                u16x8 ka[LV], vb[LVV];
#pragma unroll
                for (int l = 0; l < LV; l++) ka[l] = lds8(&sm.kt[l][j][s0]);
#pragma unroll
                for (int l = 0; l < LVV; l++) vb[l] = lds8(&sm.vt[l][col][s0]);
                mma32_terms<LV, LVV>(ka, vb, S[rt]);
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const float4 e4 =
                    *reinterpret_cast<const float4*>(&sm.ebc[32 * rt + 8 * q4 + 4 * hh]);
                S[rt][4 * q4 + 0] *= e4.x;
                S[rt][4 * q4 + 1] *= e4.y;
                S[rt][4 * q4 + 2] *= e4.z;
                S[rt][4 * q4 + 3] *= e4.w;
            }
        }
    };
    // Routed: the record's slot row = w_r O[r].  Shared: o[token] = w_r O[r]
    // + the token's routed slots.  A padded record's store goes to a dummy row.
    auto outputs = [&](int buf) {
        if constexpr (!kLocal) {
#pragma unroll
            for (int t2 = 0; t2 < kOT; t2++)
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++) {
                    const int rb = 32 * t2 + 8 * q4 + 4 * hh;
                    const uint4 rw = *reinterpret_cast<const uint4*>(&sm.mout[buf][rb]);
                    const float4 wr = *reinterpret_cast<const float4*>(&sm.mw[buf][rb]);
                    const uint32_t rows[4] = {rw.x, rw.y, rw.z, rw.w};
                    const float ws[4] = {wr.x, wr.y, wr.z, wr.w};
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        float val = ws[e] * O[t2][4 * q4 + e];
                        const uint32_t off = rows[e] * (uint32_t)(DV * 4) + col4;
                        const bool valid = is_real(ws[e]);
                        if constexpr (MODE == kModeShared) {
                            for (int j = 0; j < a.topk; j++)
                                val += a.part[((int64_t)rows[e] * a.topk + j) * DV + col];
                            char* base = reinterpret_cast<char*>(valid ? a.o : a.trash);
                            *reinterpret_cast<float*>(base + (valid ? off : col4)) = val;
                        } else {
                            char* base = reinterpret_cast<char*>(valid ? a.part : a.trash);
                            *reinterpret_cast<float*>(base + (valid ? off : col4)) = val;
                        }
                    }
                }
        }
    };


    // ---------------- pipeline ----------------
    // Per chunk n (two blocks share a CU and fill each other's stalls):
    //   prepare chunk n from registers; start the q/k/log_alpha loads of
    //   chunk n+1 (a whole iteration ahead, and ahead of this chunk's output
    //   stores, so waiting for them never waits for stores) and the metadata
    //   loads of n+2; barrier; store chunk n operands and start the v loads
    //   of n+1; barrier; causal A tiles; barrier; MFMA phase with the outputs
    //   of chunk n.
    if (nchunks > 0) {
        uint32_t mrw = 0, mor = 0;
        float mc = 0.f, mwv = 0.f;
        meta_load(0, mrw, mor, mc, mwv);
        if (tid < C) meta_store(0, 0, mrw, mor, mc, mwv);
        meta_load(1, mrw, mor, mc, mwv);
        if (tid < C) meta_store(1, 1, mrw, mor, mc, mwv);
        lds_barrier();
        raw_load_qkl(0);
        raw_load_v(0);
        for (int64_t c = 0; c < nchunks; c++) {
            const int cur = (int)(c % 3), nxt = (int)((c + 1) % 3), nn = (int)((c + 2) % 3);
            const bool more = c + 1 < nchunks;  // uniform
            prep(cur);
            if (more) raw_load_qkl(nxt);  // q, k, log_alpha registers are free now
            meta_load(c + 2, mrw, mor, mc, mwv);
            lds_barrier();  // previous chunk's MFMA phase is done with the tiles
            prep_store();
            if (more) raw_load_v(nxt);    // v registers are free after the V^T store
            if (tid < C) meta_store(c + 2, nn, mrw, mor, mc, mwv);
            lds_barrier();
            if constexpr (!kLocal) {
                a_tiles();
                lds_barrier();
            }
            if (col_wave) {
                mma_out();
                outputs(cur);
                mma_state();
            }
        }
    }

    // ---------------- results ----------------
    if constexpr (kLocal) {
        // local state and decay product of this piece
        if (col_wave) {
#pragma unroll
            for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                    a.agg_S[((abase + piece) * CK + row) * DV + col] = S[rt][i];
                }
        }
        if (gk_ == 0)
#pragma unroll
            for (int e = 0; e < kPC; e++)
                a.agg_D[(abase + piece) * CK + j0 + e] = __builtin_amdgcn_exp2f(btot[e]);
    } else if (col_wave && last_piece) {
#pragma unroll
        for (int rt = 0; rt < RT_N; rt++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int row = 32 * rt + 8 * (i / 4) + 4 * hh + (i % 4);
                a.final_states[sbase + (int64_t)row * DV + col] = S[rt][i];
            }
    }
}

// ============================ launchers ============================
namespace {

template <int C, int CK, int DV, int LV, int LVV, typename TIn, int MODE>
void launch_cfg(const ChunkArgs& a, hipStream_t st) {
    dim3 grid;
    if (MODE == kModeRouted)
        grid = dim3((unsigned)(a.num_seqs * a.H * a.N));
    else
        grid = dim3((unsigned)(a.num_seqs * a.H),
                    (unsigned)(MODE == kModeLocal ? a.max_pieces - 1 : a.max_pieces));
    if (grid.x == 0 || grid.y == 0) return;
    chunk_kernel<C, CK, DV, LV, LVV, TIn, MODE><<<grid, kThreads, 0, st>>>(a);
}

template <int C, int LV, int LVV, typename TIn, int MODE>
bool launch_shape(const ChunkArgs& a, int c, int d, hipStream_t st) {
#define SSE_CASE(CC, DD)                                   \
    if (c == CC && d == DD) {                              \
        launch_cfg<C, CC, DD, LV, LVV, TIn, MODE>(a, st);  \
        return true;                                       \
    }
    SSE_CASE(32, 32) SSE_CASE(32, 64) SSE_CASE(32, 128)
    SSE_CASE(64, 32) SSE_CASE(64, 64) SSE_CASE(64, 128)
    SSE_CASE(128, 32) SSE_CASE(128, 64) SSE_CASE(128, 128)
#undef SSE_CASE
    return false;
}

template <int MODE>
hipError_t launch_mode(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    if ((int64_t)a.num_seqs * a.H == 0) return hipSuccess;
    // bf16 inputs: the warp-specialised kernel of chunk_ws.hip.  fp32 inputs:
    // this kernel, 32-record chunks, 3 bf16 terms.
    if (dtype != kF32) return launch_chunk_ws(MODE, a, c, d, st);
    const bool ok = launch_shape<32, 3, 3, float, MODE>(a, c, d, st);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int chunk_piece_len(int dtype) { return dtype == kF32 ? 1024 : SSE_SHARED_PIECE; }

int chunk_max_pieces(int max_seqlen, int dtype) {
    const int p = chunk_piece_len(dtype);
    return max_seqlen <= 0 ? 1 : (max_seqlen + p - 1) / p;
}

hipError_t launch_chunk_local(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    // fp32: nothing to do without a second piece; bf16: the pass also
    // computes every token's key-softmax normaliser, so it always runs
    if (dtype == kF32 && a.max_pieces <= 1) return hipSuccess;
    if (dtype != kF32) return launch_piece_state(a, c, d, st);
    return launch_mode<kModeLocal>(a, dtype, c, d, st);
}
hipError_t launch_chunk_shared(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    return launch_mode<kModeShared>(a, dtype, c, d, st);
}
hipError_t launch_chunk_routed(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st) {
    return launch_mode<kModeRouted>(a, dtype, c, d, st);
}

}  // namespace sse
