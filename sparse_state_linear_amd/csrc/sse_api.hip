// sse_api.hip -- the extern "C" entry points declared in include/sse.h:
// host-side argument checks, workspace carving and launch sequencing.
// Every check runs before the first HIP call, so invalid arguments are
// reported without touching a device.
#include <limits.h>

#include "sse.h"
#include "sse_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool supported_dim(int x) { return x == 32 || x == 64 || x == 128; }

int check_common(int dtype, int H, int c, int d, int N, int topk) {
    if (dtype != SSE_F32 && dtype != SSE_BF16) return SSE_ERR_INVALID_ARG;
    if (H < 1 || c < 1 || d < 1 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (!supported_dim(c) || !supported_dim(d)) return SSE_ERR_UNSUPPORTED;
    if (N > sse::kMaxN || topk > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    return SSE_OK;
}

struct FwdLayout {
    size_t idx, w, counts, seg_off, seg_tok, seg_w, total;
};

// Returns false when the sizes overflow the int32 indexing of the kernels.
bool forward_layout(int64_t T, int S, int max_seqlen, int H, int N, int K, FwdLayout& L) {
    if (T < 0 || S < 0 || max_seqlen < 0 || H < 1 || N < 1 || K < 1) return false;
    const int64_t recs = T * H * K;
    const int64_t nblk = sse::group_nblk(max_seqlen);
    const int64_t cnt = (int64_t)S * H * N * nblk;
    const int64_t units = (int64_t)S * H * (N + 1);
    if (recs >= INT_MAX || cnt >= INT_MAX || units >= INT_MAX || T >= INT_MAX) return false;
    if ((int64_t)S * H >= INT_MAX || (int64_t)S * H * N + 1 >= INT_MAX) return false;
    size_t off = 0;
    L.idx = off;     off += align_up(sizeof(int32_t) * (size_t)recs);
    L.w = off;       off += align_up(sizeof(float) * (size_t)recs);
    L.counts = off;  off += align_up(sizeof(int32_t) * (size_t)cnt);
    L.seg_off = off; off += align_up(sizeof(int32_t) * (size_t)((int64_t)S * H * N + 1));
    L.seg_tok = off; off += align_up(sizeof(int32_t) * (size_t)recs);
    L.seg_w = off;   off += align_up(sizeof(float) * (size_t)recs);
    L.total = off;
    return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSE_OK : SSE_ERR_HIP; }

}  // namespace

extern "C" {

const char* sse_status_string(int status) {
    switch (status) {
        case SSE_OK: return "SSE_OK";
        case SSE_ERR_INVALID_ARG: return "SSE_ERR_INVALID_ARG: null pointer or inconsistent size";
        case SSE_ERR_UNSUPPORTED: return "SSE_ERR_UNSUPPORTED: size outside the supported set";
        case SSE_ERR_WORKSPACE: return "SSE_ERR_WORKSPACE: workspace too small";
        case SSE_ERR_HIP: return "SSE_ERR_HIP: a HIP launch failed";
        default: return "SSE_ERR_UNKNOWN";
    }
}

int sse_version(void) { return 100; }

size_t sse_forward_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                   int c, int d, int N, int topk) {
    if (check_common(SSE_BF16, H, c, d, N, topk) != SSE_OK) return 0;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, N, topk, L)) return 0;
    return L.total;
}

int sse_forward(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                const void* router_logits, int dtype, const int32_t* cu_seqlens, int num_seqs,
                int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                const float* initial_states, float* o, float* final_states, int32_t* topk_idx,
                float* topk_w, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !o))
        return SSE_ERR_INVALID_ARG;
    if (num_seqs > 0 && !final_states) return SSE_ERR_INVALID_ARG;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, N, topk, L))
        return SSE_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return SSE_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(ws + L.w);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* seg_off = reinterpret_cast<int32_t*>(ws + L.seg_off);
    int32_t* seg_tok = reinterpret_cast<int32_t*>(ws + L.seg_tok);
    float* seg_w = reinterpret_cast<float*>(ws + L.seg_w);

    hipError_t e = sse::launch_route_count(router_logits, dtype, cu_seqlens, num_seqs, max_seqlen,
                                           H, N, topk, idx, w, counts, o, d, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    e = sse::launch_group(idx, w, cu_seqlens, num_seqs, max_seqlen, H, N, topk, true, counts,
                          seg_off, seg_tok, nullptr, seg_w, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    sse::ChunkArgs a;
    a.q = q;
    a.kl = key_logits;
    a.v = v;
    a.la = log_alpha;
    a.cu = cu_seqlens;
    a.seg_offsets = seg_off;
    a.seg_tok = seg_tok;
    a.seg_w = seg_w;
    a.init = initial_states;
    a.o = o;
    a.final_states = final_states;
    a.num_seqs = num_seqs;
    a.H = H;
    a.N = N;
    return hip_status(sse::launch_chunk_gla(a, dtype, c, d, s));
}

int sse_decode_step(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                    const void* router_logits, int dtype, int B, int H, int c, int d, int N,
                    int topk, float* states, float* o, int32_t* topk_idx, void* stream) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    if (B < 0) return SSE_ERR_INVALID_ARG;
    if ((int64_t)B * H >= INT_MAX) return SSE_ERR_UNSUPPORTED;
    if (B > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !states || !o))
        return SSE_ERR_INVALID_ARG;
    return hip_status(sse::launch_decode(q, key_logits, v, log_alpha, router_logits, dtype, B, H,
                                         c, d, N, topk, states, o, topk_idx,
                                         static_cast<hipStream_t>(stream)));
}

int sse_router_topk(const void* router_logits, int dtype, int64_t rows, int N, int topk,
                    int32_t* topk_idx, float* topk_w, void* stream) {
    if (dtype != SSE_F32 && dtype != SSE_BF16) return SSE_ERR_INVALID_ARG;
    if (rows < 0 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (N > sse::kMaxN || topk > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    if (rows * topk >= INT_MAX) return SSE_ERR_UNSUPPORTED;
    if (rows > 0 && (!router_logits || !topk_idx || !topk_w)) return SSE_ERR_INVALID_ARG;
    return hip_status(sse::launch_router_rows(router_logits, dtype, rows, N, topk, topk_idx,
                                              topk_w, static_cast<hipStream_t>(stream)));
}

size_t sse_group_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H, int N,
                                 int topk) {
    if (N < 1 || topk < 1 || topk > N || N > sse::kMaxN || topk > sse::kMaxTopK) return 0;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, N, topk, L)) return 0;
    return L.seg_off - L.counts;
}

int sse_group_by_partition(const int32_t* topk_idx, const float* topk_w,
                           const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                           int64_t total_tokens, int H, int N, int topk, int32_t* seg_offsets,
                           int32_t* seg_tok, int32_t* seg_slot, float* seg_w, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (H < 1 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (N > sse::kMaxN || topk > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens || !seg_offsets) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!topk_idx || !seg_tok)) return SSE_ERR_INVALID_ARG;
    if (seg_w && !topk_w) return SSE_ERR_INVALID_ARG;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, N, topk, L))
        return SSE_ERR_UNSUPPORTED;
    const size_t need = L.seg_off - L.counts;
    if (workspace_bytes < need || (need > 0 && !workspace)) return SSE_ERR_WORKSPACE;
    return hip_status(sse::launch_group(topk_idx, topk_w, cu_seqlens, num_seqs, max_seqlen, H, N,
                                        topk, false, static_cast<int32_t*>(workspace),
                                        seg_offsets, seg_tok, seg_slot, seg_w,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
