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

int group_nblk(int max_seqlen);

hipError_t launch_router_rows(const void* z, int dtype, int64_t rows, int N, int K, int32_t* idx,
                              float* w, hipStream_t st);

hipError_t launch_route_count(const void* z, int dtype, const int32_t* cu, int num_seqs,
                              int max_seqlen, int H, int N, int K, int32_t* idx, float* w,
                              int32_t* counts, float* o_zero, int d, hipStream_t st);

hipError_t launch_group(const int32_t* idx, const float* w, const int32_t* cu, int num_seqs,
                        int max_seqlen, int H, int N, int K, bool counts_ready, int32_t* counts,
                        int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot, float* seg_w,
                        hipStream_t st);

struct ChunkArgs {
    const void* q;
    const void* kl;
    const void* v;
    const void* la;
    const int32_t* cu;
    const int32_t* seg_offsets;
    const int32_t* seg_tok;
    const float* seg_w;
    const float* init;
    float* o;
    float* final_states;
    int num_seqs, H, N;
};

hipError_t launch_chunk_gla(const ChunkArgs& a, int dtype, int c, int d, hipStream_t st);

hipError_t launch_decode(const void* q, const void* kl, const void* v, const void* la,
                         const void* z, int dtype, int B, int H, int c, int d, int N, int K,
                         float* states, float* o, int32_t* topk_idx, hipStream_t st);

}  // namespace sse
