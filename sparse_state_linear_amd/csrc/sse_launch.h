// sse_launch.h -- internal launcher declarations shared by the C-ABI layer
// and the kernel translation units of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sse_device.h"

namespace sse {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kMaxN = 64;
constexpr int kMaxTopK = 8;
constexpr int kMaxH = 256;

// Tokens per grouping block (one wave ranks a block's records).
constexpr int kTokBlock = 64;
inline int group_nblk(int max_seqlen) {
    return max_seqlen <= 0 ? 1 : (max_seqlen + kTokBlock - 1) / kTokBlock;
}

hipError_t launch_router_rows(const void* z, int dtype, int64_t rows, int N, int K, int32_t* idx,
                              float* w, hipStream_t st);

// One routed record of a partition segment (16 bytes): input row t*H + h,
// slot row (t*H + h)*topk + rank, exponent offset lnz2 - log2 w (so that
// 2^(kl log2 e - cr) = w kappa), read gate w.
struct SegRec {
    uint32_t row, orow;
    float cr, w;
};

// Routing of the forward: top-k + weights into idx / w ([T, H, K]), block
// counts, head-major (partition | rank << 16, w) records in rinfo
// ([H, T, K]), and with lnz2 non-null the key-softmax log2 normalisers.
hipError_t launch_route_count(const void* z, const void* kl, int dtype, const int32_t* cu,
                              int num_seqs, int max_seqlen, int64_t T, int H, int c, int N, int K,
                              int32_t* idx, float* w, int32_t* counts, uint2* rinfo, float* lnz2,
                              hipStream_t st);

// Standalone grouping from a given top-k choice (separate output arrays).
hipError_t launch_group(const int32_t* idx, const float* w, const int32_t* cu, int num_seqs,
                        int max_seqlen, int H, int N, int K, int32_t* counts,
                        int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot, float* seg_w,
                        hipStream_t st);

// Grouping of the forward from route_count's counts and records into packed
// segment records.
hipError_t launch_group_fwd(const uint2* rinfo, const int32_t* cu, int num_seqs, int max_seqlen,
                            int64_t T, int H, int N, int K, int32_t* counts, int32_t* seg_offsets,
                            const float* lnz2, SegRec* seg, hipStream_t st);

// Key-softmax log2 normaliser of every (token, head) row of c key logits:
// lnz2 = log2 sum_j 2^(kl_j log2 e), so that kappa_j = 2^(kl_j log2 e - lnz2).
hipError_t launch_key_norm(const void* kl, int dtype, int64_t rows, int c, float* lnz2,
                           hipStream_t st);

// Debug outputs of the forward's grouping: copies of the segment offsets
// [nseg + 1] and, per record, its token t and top-k rank (any pointer may be
// null).
hipError_t launch_seg_debug(const SegRec* seg, const int32_t* seg_off, int64_t nrec, int64_t nseg,
                            int H, int K, int32_t* out_off, int32_t* out_tok, int32_t* out_slot,
                            hipStream_t st);

// Arguments of the chunked GLA passes (see chunk_gla.hip).
struct ChunkArgs {
    const void* q;
    const void* kl;
    const void* v;
    const void* la;
    const int32_t* cu;
    const int32_t* seg_offsets;  // routed segments
    const SegRec* seg_rec;       // routed records, segment by segment
    const float* lnz2;           // [T, H] key-softmax log2 normaliser of the keys
                                 // this pass writes with (shared pass: the shared
                                 // partition's keys)
    float* lnz2_out;             // where the bf16 piece-state pass stores lnz2
    const float* lnz2_r;         // masked pass: normaliser of the routed keys
    const int32_t* sel_idx;      // masked pass: write set [T, H, sel_k] and its
    const float* sel_w;          //   router probabilities
    const int32_t* rd_idx;       // masked pass: read set [T, H, rd_k] and its
    const float* rd_w;           //   read weights (the write set by default)
    int sel_k, rd_k;
    const float* init;           // [S, H, N+1, c, d] or null
    float* o;
    float* final_states;
    float* agg_S;                // local piece states, [S*H, max_pieces] of c x d: row-major
                                 // for fp32 inputs; for bf16 inputs fragment-major
                                 // [c/32][d/32][64 lanes][16] (32x32 MFMA accumulator tiles)
    float* agg_D;                // [S*H, max_pieces, c] piece decay products
    float* trash;                // one dummy output row for padded records
    float* part;                 // [T, H, topk, d] e-gated routed reads (the
                                 // routed pass writes them, the shared pass adds
                                 // them into o): fp32 for fp32 inputs, int16
                                 // values for bf16 inputs
    float* part_scale;           // bf16 inputs: [T, H, topk, d/32] fp32 steps
    uint32_t slot_rows;          // T H topk; bf16 slots have one spare row past it
    uint32_t rows;               // T H: rows of every token input
    int num_seqs, H, N, topk;
    int piece_len;               // records per shared piece
    int max_pieces;
    // routed segments split into pieces (bf16 inputs, few segments): 0 =
    // every segment in one block; else records per piece, the most pieces a
    // segment can have, and the local states of the pieces (fragment-major
    // like agg_S, one c x d slot per piece but the last) with the piece
    // decays [slots, c]
    int rpiece_len;
    int rmax_pieces;
    float* ragg_S;
    float* ragg_D;
    const void* kl_r;            // the routed keys' logits (the piece states of
                                 // routed pieces run in the shared pass's
                                 // piece launch, whose kl may be the shared
                                 // partition's own keys)
};

// Passes of the chunked kernels: the shared partition's chain, the routed
// partitions' segments (records gathered by the grouping), or the masked
// schedule (every token of a sequence is a record of every partition; those
// outside the partition's write and read sets are padding).
enum { kModeShared = 1, kModeRouted = 2, kModeMasked = 3 };

// Records per shared piece of the bf16 kernels (the longest piece length).
constexpr int kSharedPiece = 1024;
// Longest piece of a split routed segment, and the most pieces per segment
// the piece length aims for (the routed pass combines all earlier pieces'
// states in its prologue; only sequences past 32K tokens exceed it).
constexpr int kMaxRoutedPiece = 2048;
constexpr int kMaxRoutedPieces = 16;
inline int chunk_piece_len() { return kSharedPiece; }

// bf16 inputs: key-softmax normalisers of every token and the shared
// partition's piece states (piece_state.hip), plus, with rpiece_len > 0, the
// local states and decays of every piece but the last of the split routed
// segments (then it runs after the grouping); fp32 inputs: nothing (the fp64
// kernel walks each shared chain in one block and computes its own
// normalisers).
hipError_t launch_chunk_local(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st);

hipError_t launch_piece_state(const ChunkArgs& a, int c, int d, hipStream_t st);
hipError_t launch_chunk_shared(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st);
hipError_t launch_chunk_routed(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st);
// masked schedule: one block per (sequence, head, partition) over every
// token of the sequence, membership from sel_idx / rd_idx
hipError_t launch_chunk_masked(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st);
// fp32 inputs: the fp64 chunk kernel (chunk_f64.hip), mode kModeRouted or
// kModeShared.
hipError_t launch_chunk_f64(int mode, const ChunkArgs& a, int c, int d, hipStream_t st);

// Row-sparse key variant: per (token, head) row of c key logits, kl_out =
// kl on the k largest entries (equal values: lower rows first) and -inf
// elsewhere; la_out = la on those rows and 0 elsewhere (identity != 0) or la
// everywhere.  Inputs and outputs in the storage type of dtype.
hipError_t launch_rowsparse_mask(const void* kl, const void* la, int dtype, int64_t rows, int c,
                                 int k, int identity, void* kl_out, void* la_out, hipStream_t st);

// Arguments of the backward pass (backward.hip).
// One record of a backward chunk: input row t*H + h, gradient slot row
// (kNoSlot for padding; on a slot's first record: the slot holds no
// chunk), gate, key normaliser (log2).
constexpr uint32_t kNoSlot = 0xffffffffu;
struct BwdRec {
    uint32_t row, slot;
    float w, lnz;
};

struct BwdArgs {
    const void *q, *kl, *v, *la, *z;
    const int32_t* cu;
    const int32_t* seg_offsets;   // routed segments of the forward's grouping
    const SegRec* seg_rec;
    const int32_t* sel_idx;       // [T, H, topk] the forward's top-k choices
    const float* lnz2;            // [T, H] key-softmax log2 normalisers
    const float* init;            // [S, H, N+1, c, d] or null
    const float* dfinal;          // gradient of the final states, or null
    const float* dout;            // [T, H, d] gradient of o
    float* ckS;                   // [nslot, c, d] state at the start of each chunk
    float* ckG;                   // [nslot, c, d] D G: the state gradient after each
                                  // chunk times the chunk's decay diag(e^{b_C})
    BwdRec* slot_meta;            // [nslot, 32] the records of each slot's chunk
    int64_t nslot, sh_slots;      // slots in all; slots of the shared chains
    float *g_dq, *g_dkl, *g_dla;  // per-record slots [T*H*(topk+1), c]
    float* g_dv;                  // [T*H*(topk+1), d]
    float* g_dw;                  // [T*H*(topk+1)]
    float *dq, *dkl, *dla, *dv, *dz, *dinit;   // outputs (dinit may be null)
    int64_t rows;                 // T*H
    int num_seqs, H, N, topk;
};

// Records per chunk of the backward, and the checkpoint slot of the first
// chunk of segment `idx` whose records start at `first` (segments numbered
// in record order): floor(first / C) + idx.  Consecutive segments' slots
// never overlap, and records / C + segments + 1 slots hold them all.
constexpr int kBwdChunk = 32;
__host__ __device__ inline int64_t bwd_slot_base(int64_t first, int64_t idx) {
    return first / kBwdChunk + idx;
}
inline int64_t bwd_slots(int64_t records, int64_t segments) {
    return records / kBwdChunk + segments + 1;
}

hipError_t launch_backward(const BwdArgs& a, int dtype, int c, int d, hipStream_t st);

// General decode step: own shared q/k and read set (each may be null).
hipError_t launch_decode_ex(const void* q, const void* kl, const void* v, const void* la,
                            const void* z, const void* q_sh, const void* kl_sh, const void* zr,
                            int dtype, int B, int H, int c, int d, int N, int K, int KR,
                            float* states, float* o, int32_t* topk_idx, int32_t* read_idx,
                            hipStream_t st);

hipError_t launch_decode(const void* q, const void* kl, const void* v, const void* la,
                         const void* z, int dtype, int B, int H, int c, int d, int N, int K,
                         float* states, float* o, int32_t* topk_idx, hipStream_t st);

}  // namespace sse
