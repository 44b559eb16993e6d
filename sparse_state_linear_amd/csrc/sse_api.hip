// sse_api.hip -- the extern "C" entry points declared in include/sse.h:
// host-side argument checks, workspace carving and launch sequencing.
// Every check runs before the first HIP call, so invalid arguments are
// reported without touching a device.
#include <limits.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "sse.h"
#include "sse_launch.h"

// Workspace of sse_forward_noalloc (see scratch_ptr below).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool supported_dim(int x) { return x == 32 || x == 64 || x == 128; }

int check_common(int dtype, int H, int c, int d, int N, int topk) {
    if (dtype != SSE_F32 && dtype != SSE_BF16) return SSE_ERR_INVALID_ARG;
    if (H < 1 || c < 1 || d < 1 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (!supported_dim(c) || !supported_dim(d)) return SSE_ERR_UNSUPPORTED;
    if (N > sse::kMaxN || topk > sse::kMaxTopK || H > sse::kMaxH) return SSE_ERR_UNSUPPORTED;
    return SSE_OK;
}

struct FwdLayout {
    size_t idx, w, ridx, rw, counts, seg_off, rinfo, seg_rec, lnz2, lnz2_sh, agg_S, agg_D, ragg_S,
        ragg_D, trash, part, total;
    int rpiece_len, rmax_pieces;
};

// Piece length of the shared partition's chain (bf16 inputs; the fp32-input
// kernel walks each chain in one block): 1024 tokens, halved (down to 256)
// while the shared pass would run fewer than 512 (sequence, head, piece)
// blocks and a sequence would still have at most 16 pieces, so that a few
// short sequences spread over the chip; the shared pass and the piece-state
// pass launch one block per piece.  The cap bounds the shared pass's
// prologue, which reads the aggregates of every earlier piece (quadratic in
// the piece count).
int shared_piece_len(int64_t S, int H, int max_seqlen) {
    int p = sse::chunk_piece_len();
    auto pieces = [&](int pl) { return max_seqlen <= 0 ? 1 : (max_seqlen + pl - 1) / pl; };
    while (p > 256 && S * H * pieces(p) < 512 && pieces(p / 2) <= 16) p /= 2;
    return p;
}

int max_pieces(int max_seqlen, int piece_len) {
    return max_seqlen <= 0 ? 1 : (max_seqlen + piece_len - 1) / piece_len;
}

// Records per piece of a routed segment (bf16 inputs, varlen schedule), or
// 0 to run every segment in one block.  With fewer (sequence, head,
// partition) segments than the chip has compute units, one block per
// segment leaves CUs idle while a few blocks walk long segments, so the
// segments are cut into pieces when they hold 512 records or more on
// average (shorter ones cost less than the piece states would): the
// smallest power of two from 64 records up that gives at most one piece per
// compute unit and at most 16 pieces per segment, capped at 2048 records.
// No segment is longer than max_seqlen records (a token enters a partition
// at most once).
constexpr int kComputeUnits = 256;
int routed_piece_len(int64_t T, int S, int max_seqlen, int H, int N, int K) {
    const int64_t segs = (int64_t)S * H * N;
    const int64_t recs = T * H * K;
    if (segs >= kComputeUnits || recs < 512 * segs) return 0;
    int p = 64;
    while (p < sse::kMaxRoutedPiece &&
           (recs / p > kComputeUnits || (max_seqlen + p - 1) / p > sse::kMaxRoutedPieces))
        p *= 2;
    return max_seqlen > p ? p : 0;
}

// Workspace carving.  c, d = 0 sizes the grouping part only; Kr > 0
// reserves the read-set choices (Kr per token) and sizes the routed-read
// slots by Kr instead of K.  Returns false when the sizes overflow the
// 32-bit indexing of the kernels.
bool forward_layout(int64_t T, int S, int max_seqlen, int H, int c, int d, int N, int K,
                    FwdLayout& L, int Kr = 0) {
    if (T < 0 || S < 0 || max_seqlen < 0 || H < 1 || N < 1 || K < 1 || Kr < 0) return false;
    const int64_t recs = T * H * K;
    const int64_t rrecs = T * H * Kr;
    const int64_t slots = Kr > 0 ? rrecs : recs;
    const int64_t nblk = sse::group_nblk(max_seqlen);
    const int64_t cnt = (int64_t)S * H * N * nblk;
    const int64_t units = (int64_t)S * H * (N + 1);
    if (recs >= INT_MAX || rrecs >= INT_MAX || cnt >= INT_MAX || units >= INT_MAX ||
        T >= INT_MAX)
        return false;
    if ((int64_t)S * H >= INT_MAX || (int64_t)S * H * N + 1 >= INT_MAX) return false;
    if ((int64_t)S * nblk * H >= INT_MAX) return false;
    const int64_t maxp = max_pieces(max_seqlen, shared_piece_len(S, H, max_seqlen));
    if (maxp >= 65536) return false;
    size_t off = 0;
    L.idx = off;     off += align_up(sizeof(int32_t) * (size_t)recs);
    L.w = off;       off += align_up(sizeof(float) * (size_t)recs);
    L.ridx = off;    off += align_up(sizeof(int32_t) * (size_t)rrecs);
    L.rw = off;      off += align_up(sizeof(float) * (size_t)rrecs);
    L.counts = off;  off += align_up(sizeof(int32_t) * (size_t)cnt);
    L.seg_off = off; off += align_up(sizeof(int32_t) * (size_t)((int64_t)S * H * N + 1));
    L.rinfo = off;   off += align_up(sizeof(uint2) * (size_t)recs);
    L.seg_rec = off; off += align_up(sizeof(sse::SegRec) * (size_t)recs);
    L.lnz2 = off;    off += align_up(sizeof(float) * (size_t)(T * H));
    L.lnz2_sh = off; off += align_up(sizeof(float) * (size_t)(T * H));
    L.agg_S = off;   off += align_up(sizeof(float) * (size_t)((int64_t)S * H * maxp * c * d));
    L.agg_D = off;   off += align_up(sizeof(float) * (size_t)((int64_t)S * H * maxp * c));
    // start states of routed pieces: records / P + segments + 1 slots
    L.rpiece_len = Kr > 0 ? 0 : routed_piece_len(T, S, max_seqlen, H, N, K);
    L.rmax_pieces = L.rpiece_len > 0 ? max_pieces(max_seqlen, L.rpiece_len) : 1;
    const int64_t rslots = L.rpiece_len > 0 ? recs / L.rpiece_len + (int64_t)S * H * N + 1 : 0;
    if (L.rmax_pieces >= 65536) return false;
    L.ragg_S = off;  off += align_up(sizeof(float) * (size_t)(rslots * c * d));
    L.ragg_D = off;  off += align_up(sizeof(float) * (size_t)(rslots * c));
    L.trash = off;   off += align_up(sizeof(float) * (size_t)(d > 0 ? 2 * d : 1));
    // fp32 slots: `slots` rows of d floats; bf16 slots: slots + 1 rows of d
    // int16 values, then slots + 1 rows of d/32 fp32 steps
    L.part = off;    off += align_up(sizeof(float) * (size_t)(slots + 1) * (size_t)d);
    L.total = off;
    return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSE_OK : SSE_ERR_HIP; }

// Workspace of the row-sparse forward: the masked key logits and log decay
// (fp32-sized rows, either input type), the key normalisers, the shared
// pieces' aggregates, a dummy output row and one slot row (no routed reads).
struct RsLayout {
    size_t kl, la, lnz2, agg_S, agg_D, trash, part, total;
};

bool rowsparse_layout(int64_t T, int S, int max_seqlen, int H, int c, int d, RsLayout& L) {
    if (T < 0 || S < 0 || max_seqlen < 0 || H < 1) return false;
    if (T >= INT_MAX || (int64_t)S * H >= INT_MAX) return false;
    const int64_t maxp = max_pieces(max_seqlen, shared_piece_len(S, H, max_seqlen));
    if (maxp >= 65536) return false;
    size_t off = 0;
    L.kl = off;    off += align_up(sizeof(float) * (size_t)(T * H * c));
    L.la = off;    off += align_up(sizeof(float) * (size_t)(T * H * c));
    L.lnz2 = off;  off += align_up(sizeof(float) * (size_t)(T * H));
    L.agg_S = off; off += align_up(sizeof(float) * (size_t)((int64_t)S * H * maxp * c * d));
    L.agg_D = off; off += align_up(sizeof(float) * (size_t)((int64_t)S * H * maxp * c));
    L.trash = off; off += align_up(sizeof(float) * (size_t)(2 * d));
    L.part = off;  off += align_up(sizeof(float) * (size_t)d);
    L.total = off;
    return true;
}

int check_rowsparse(int dtype, int H, int c, int d, int row_topk) {
    if (dtype != SSE_F32 && dtype != SSE_BF16) return SSE_ERR_INVALID_ARG;
    if (H < 1 || c < 1 || d < 1 || row_topk < 1 || row_topk > c) return SSE_ERR_INVALID_ARG;
    if (!supported_dim(c) || !supported_dim(d)) return SSE_ERR_UNSUPPORTED;
    if (H > sse::kMaxH) return SSE_ERR_UNSUPPORTED;
    return SSE_OK;
}

// ---- stage tracing: a ring of per-call HIP events (profiling aid) ----------
constexpr int kTraceCalls = 256;
constexpr int kTraceMarks = SSE_TRACE_STAGES + 1;
struct Trace {
    bool on = false;
    bool created = false;
    hipEvent_t ev[kTraceCalls][kTraceMarks];
    int64_t calls = 0;   // forward calls recorded since the last read
} g_trace;

inline void trace_mark(int mark, hipStream_t s) {
    if (g_trace.on) (void)hipEventRecord(g_trace.ev[g_trace.calls % kTraceCalls][mark], s);
}

// ---- debug mode: host checks of cu_seqlens, synchronous errors --------------
// Off unless the environment variable SSE_DEBUG_CHECKS is set to anything
// but "0" when the library is first used, or sse_debug_checks(1) is called.
std::atomic<int> g_debug{-1};   // -1: environment not read yet

bool debug_on() {
    int v = g_debug.load();
    if (v < 0) {
        const char* e = getenv("SSE_DEBUG_CHECKS");
        int want = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
        g_debug.compare_exchange_strong(v, want);
        v = g_debug.load();
    }
    return v == 1;
}

// The preconditions on cu_seqlens that the kernels rely on: it starts at 0,
// never decreases, ends at total_tokens, and no sequence is longer than
// max_seqlen.  Copies the array to the host, which synchronises the stream.
int debug_check_cu(const int32_t* cu, int num_seqs, int64_t total_tokens, int max_seqlen,
                   hipStream_t s) {
    std::vector<int32_t> h((size_t)num_seqs + 1);
    if (hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return SSE_ERR_HIP;
    if (h[0] != 0 || (int64_t)h[num_seqs] != total_tokens) return SSE_ERR_INVALID_ARG;
    for (int i = 0; i < num_seqs; i++) {
        const int64_t len = (int64_t)h[i + 1] - (int64_t)h[i];
        if (len < 0 || len > max_seqlen) return SSE_ERR_INVALID_ARG;
    }
    return SSE_OK;
}

// A call's status in debug mode: the stream is synchronised, so a kernel
// that failed is reported by the call that launched it.
int debug_finish(int status, void* stream) {
    if (status != SSE_OK || !debug_on()) return status;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SSE_ERR_HIP;
    return hipGetLastError() == hipSuccess ? SSE_OK : SSE_ERR_HIP;
}

// ---- no-allocation forward: the workspace in a static device array ----------
// Callers that cannot allocate device memory (code under graph capture,
// serving loops, harnesses that forbid hipMalloc) use sse_forward_noalloc,
// whose workspace is this array.  Each device that loads the library holds
// its own copy until the process ends; host code reaches a device's copy
// only through the address hipGetSymbolAddress returns for it (the array's
// name is a host-side stand-in, not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up once per
// device), or null on a HIP error.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Options of the general forward (the defaults give sse_forward).
struct FwdOpts {
    const void* q_sh = nullptr;   // shared partition's own query rows (or q)
    const void* kl_sh = nullptr;  // shared partition's own key logits (or key_logits)
    const void* zr = nullptr;     // read-set router logits (or the write set's)
    int kr = 0;                   // read-set size when zr is given
    int schedule = SSE_SCHEDULE_VARLEN;
    int32_t* ridx_out = nullptr;  // read-set choices [T, H, kr] (optional)
    bool use_scratch = false;     // workspace = the static array
};

FwdOpts scratch_opts() {
    FwdOpts opt;
    opt.use_scratch = true;
    return opt;
}

int forward_impl(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                 const void* router_logits, int dtype, const int32_t* cu_seqlens, int num_seqs,
                 int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                 const float* initial_states, float* o, float* final_states, int32_t* topk_idx,
                 float* topk_w, int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot,
                 void* workspace, size_t workspace_bytes, void* stream, const FwdOpts& opt) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    const bool masked = opt.schedule == SSE_SCHEDULE_MASKED;
    if (opt.schedule != SSE_SCHEDULE_VARLEN && !masked) return SSE_ERR_INVALID_ARG;
    const bool rsets = opt.zr != nullptr;
    if (rsets && (opt.kr < 1 || opt.kr > N)) return SSE_ERR_INVALID_ARG;
    if (rsets && opt.kr > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    if (!rsets && opt.ridx_out) return SSE_ERR_INVALID_ARG;
    // the varlen grouping carries one set per token: read sets that differ
    // run on the masked schedule
    if (rsets && !masked) return SSE_ERR_UNSUPPORTED;
    if (masked && (seg_offsets || seg_tok || seg_slot)) return SSE_ERR_INVALID_ARG;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !o))
        return SSE_ERR_INVALID_ARG;
    if (num_seqs > 0 && !final_states) return SSE_ERR_INVALID_ARG;
    const int kslot = rsets ? opt.kr : topk;   // routed reads per token
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk, L,
                        rsets ? opt.kr : 0))
        return SSE_ERR_UNSUPPORTED;
    // byte offsets of token rows (fp32 worst case) and of the routed slots
    // [T, H, kslot, d] fp32 must fit in 32 bits
    if (total_tokens * H * (c > d ? c : d) >= (int64_t(1) << 30)) return SSE_ERR_UNSUPPORTED;
    if (total_tokens * H * kslot * d >= (int64_t(1) << 30)) return SSE_ERR_UNSUPPORTED;
    void* ws_ptr = workspace;
    size_t ws_bytes = workspace_bytes;
    if (opt.use_scratch) {
        // every argument is checked; now the static array (no allocation)
        if (L.total > kScratchBytes) return SSE_ERR_WORKSPACE;
        ws_ptr = scratch_ptr();
        if (!ws_ptr) return SSE_ERR_HIP;
        ws_bytes = kScratchBytes;
    }
    if (!ws_ptr || ws_bytes < L.total) return SSE_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        st = debug_check_cu(cu_seqlens, num_seqs, total_tokens, max_seqlen, s);
        if (st != SSE_OK) return st;
    }
    char* ws = static_cast<char*>(ws_ptr);
    int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(ws + L.idx);
    float* w = topk_w ? topk_w : reinterpret_cast<float*>(ws + L.w);
    int32_t* ridx = opt.ridx_out ? opt.ridx_out : reinterpret_cast<int32_t*>(ws + L.ridx);
    float* rw = reinterpret_cast<float*>(ws + L.rw);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* seg_off = reinterpret_cast<int32_t*>(ws + L.seg_off);
    uint2* rinfo = reinterpret_cast<uint2*>(ws + L.rinfo);
    sse::SegRec* seg_rec = reinterpret_cast<sse::SegRec*>(ws + L.seg_rec);
    float* lnz2 = reinterpret_cast<float*>(ws + L.lnz2);
    // the shared partition's normalisers: the routed ones unless it has its
    // own keys
    const bool own_keys = opt.kl_sh != nullptr;
    float* lnz2_sh = own_keys ? reinterpret_cast<float*>(ws + L.lnz2_sh) : lnz2;

    // routed passes (routed / masked)
    sse::ChunkArgs a = {};
    a.q = q;
    a.kl = key_logits;
    a.v = v;
    a.la = log_alpha;
    a.cu = cu_seqlens;
    a.seg_offsets = seg_off;
    a.seg_rec = seg_rec;
    a.lnz2 = lnz2;
    a.lnz2_out = lnz2;
    a.lnz2_r = lnz2;
    a.sel_idx = idx;
    a.sel_w = w;
    a.sel_k = topk;
    a.rd_idx = rsets ? ridx : idx;
    a.rd_w = rsets ? rw : w;
    a.rd_k = kslot;
    a.init = initial_states;
    a.o = o;
    a.final_states = final_states;
    a.agg_S = reinterpret_cast<float*>(ws + L.agg_S);
    a.agg_D = reinterpret_cast<float*>(ws + L.agg_D);
    a.trash = reinterpret_cast<float*>(ws + L.trash);
    a.part = reinterpret_cast<float*>(ws + L.part);
    // bf16 inputs: int16 slot values, then their steps, inside the fp32-sized
    // slot area (2 d + d/8 <= 4 d bytes per slot row)
    a.slot_rows = (uint32_t)(total_tokens * H * kslot);
    a.rows = (uint32_t)(total_tokens * H);
    a.part_scale = reinterpret_cast<float*>(ws + L.part + sizeof(int16_t) * ((size_t)a.slot_rows + 1) *
                                                             (size_t)d);
    a.num_seqs = num_seqs;
    a.H = H;
    a.N = N;
    a.topk = kslot;
    a.piece_len = shared_piece_len(num_seqs, H, max_seqlen);
    a.max_pieces = max_pieces(max_seqlen, a.piece_len);
    const bool rsplit = dtype == SSE_BF16 && !masked && L.rpiece_len > 0;
    a.kl_r = key_logits;
    a.rpiece_len = rsplit ? L.rpiece_len : 0;
    a.rmax_pieces = rsplit ? L.rmax_pieces : 1;
    a.ragg_S = reinterpret_cast<float*>(ws + L.ragg_S);
    a.ragg_D = reinterpret_cast<float*>(ws + L.ragg_D);
    // the shared partition's passes: its own query and keys when given
    sse::ChunkArgs ash = a;
    if (opt.q_sh) ash.q = opt.q_sh;
    if (own_keys) ash.kl = opt.kl_sh;
    ash.lnz2 = lnz2_sh;
    ash.lnz2_out = lnz2_sh;

    hipError_t e;
    trace_mark(0, s);
    if (!masked) {
        // 1. router + per-block counts (+ the routed keys' normalisers when
        //    the piece-state pass will not compute them before the grouping
        //    needs them: fp32 inputs, a shared partition with its own keys,
        //    or split routed segments, whose piece states need the grouping)
        e = sse::launch_route_count(router_logits, key_logits, dtype, cu_seqlens, num_seqs,
                                    max_seqlen, total_tokens, H, c, N, topk, idx, w, counts, rinfo,
                                    (dtype == SSE_F32 || own_keys || rsplit) ? lnz2 : nullptr, s);
    } else {
        // 1. routers of the write set and the read set (no grouping), the
        //    routed keys' normalisers when the shared pass has its own keys
        e = sse::launch_router_rows(router_logits, dtype, total_tokens * H, N, topk, idx, w, s);
        if (e == hipSuccess && rsets)
            e = sse::launch_router_rows(opt.zr, dtype, total_tokens * H, N, opt.kr, ridx, rw, s);
        if (e == hipSuccess && own_keys && dtype != SSE_F32)
            e = sse::launch_key_norm(key_logits, dtype, total_tokens * H, c, lnz2, s);
    }
    if (e != hipSuccess) return SSE_ERR_HIP;
    // 2. piece states of the shared partition and its keys' normalisers
    //    (bf16 inputs; the fp32-input kernels compute their own), and, when
    //    routed segments are split, the states of their pieces in the same
    //    launch, after the grouping
    // 3. grouping into (sequence, head, partition) segments
    auto group = [&]() {
        e = sse::launch_group_fwd(rinfo, cu_seqlens, num_seqs, max_seqlen, total_tokens, H, N,
                                  topk, counts, seg_off, lnz2, seg_rec, s);
        if (e == hipSuccess)
            e = sse::launch_seg_debug(seg_rec, seg_off, total_tokens * H * topk,
                                      (int64_t)num_seqs * H * N, H, topk, seg_offsets, seg_tok,
                                      seg_slot, s);
        return e == hipSuccess;
    };
    trace_mark(1, s);
    if (rsplit && !group()) return SSE_ERR_HIP;
    e = sse::launch_chunk_local(ash, dtype, c, d, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    trace_mark(2, s);
    if (!masked && !rsplit && !group()) return SSE_ERR_HIP;
    trace_mark(3, s);
    // 4. routed partitions: e-gated reads into the workspace slots
    e = masked ? sse::launch_chunk_masked(a, dtype, c, d, s)
               : sse::launch_chunk_routed(a, dtype, c, d, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    trace_mark(4, s);
    // 5. shared partition: o = shared read + the token's routed slots
    e = sse::launch_chunk_shared(ash, dtype, c, d, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    trace_mark(5, s);
    if (g_trace.on) g_trace.calls++;
    return SSE_OK;
}

// ---- backward -----------------------------------------------------------------
struct BwdLayout {
    FwdLayout f;              // routing and grouping part (no slots of its own)
    size_t ckS, ckG, tab, g_dq, g_dkl, g_dla, g_dv, g_dw, total;
    int64_t nslot, sh_slots;
};

bool backward_layout(int64_t T, int S, int max_seqlen, int H, int c, int d, int N, int K,
                     BwdLayout& L) {
    if (!forward_layout(T, S, max_seqlen, H, 0, 0, N, K, L.f)) return false;
    const int64_t SH = (int64_t)S * H;
    // chunk slots: shared chains first, then the routed segments
    L.sh_slots = sse::bwd_slots(T * H, SH);
    L.nslot = L.sh_slots + sse::bwd_slots(T * H * K, SH * N);
    if (L.nslot >= INT_MAX || 2 * SH * (N + 1) >= INT_MAX) return false;
    const int64_t slots = T * H * (K + 1);
    if (slots >= INT_MAX) return false;
    size_t off = L.f.part;   // the forward layout's slot area is not used
    L.ckS = off;   off += align_up(sizeof(float) * (size_t)L.nslot * (size_t)c * (size_t)d);
    L.ckG = off;   off += align_up(sizeof(float) * (size_t)L.nslot * (size_t)c * (size_t)d);
    L.tab = off;   off += align_up(sizeof(sse::BwdRec) * sse::kBwdChunk * (size_t)L.nslot);
    L.g_dq = off;  off += align_up(sizeof(float) * (size_t)slots * (size_t)c);
    L.g_dkl = off; off += align_up(sizeof(float) * (size_t)slots * (size_t)c);
    L.g_dla = off; off += align_up(sizeof(float) * (size_t)slots * (size_t)c);
    L.g_dv = off;  off += align_up(sizeof(float) * (size_t)slots * (size_t)d);
    L.g_dw = off;  off += align_up(sizeof(float) * (size_t)slots);
    L.total = off;
    return true;
}

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
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk, L)) return 0;
    return L.total;
}

int sse_forward(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                const void* router_logits, int dtype, const int32_t* cu_seqlens, int num_seqs,
                int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                const float* initial_states, float* o, float* final_states, int32_t* topk_idx,
                float* topk_w, int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot,
                void* workspace, size_t workspace_bytes, void* stream) {
    const int st = forward_impl(q, key_logits, v, log_alpha, router_logits, dtype, cu_seqlens,
                                num_seqs, max_seqlen, total_tokens, H, c, d, N, topk,
                                initial_states, o, final_states, topk_idx, topk_w, seg_offsets,
                                seg_tok, seg_slot, workspace, workspace_bytes, stream, FwdOpts());
    return debug_finish(st, stream);
}

size_t sse_forward_ex_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                      int c, int d, int N, int topk, int read_topk) {
    if (check_common(SSE_BF16, H, c, d, N, topk) != SSE_OK) return 0;
    if (read_topk < 0 || read_topk > N || read_topk > sse::kMaxTopK) return 0;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk, L, read_topk))
        return 0;
    return L.total;
}

int sse_forward_ex(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                   const void* router_logits, int dtype, const int32_t* cu_seqlens, int num_seqs,
                   int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                   const void* q_shared, const void* key_logits_shared,
                   const void* read_router_logits, int read_topk, int schedule,
                   const float* initial_states, float* o, float* final_states,
                   int32_t* topk_idx, float* topk_w, int32_t* read_topk_idx,
                   int32_t* seg_offsets, int32_t* seg_tok, int32_t* seg_slot, void* workspace,
                   size_t workspace_bytes, void* stream) {
    FwdOpts opt;
    opt.q_sh = q_shared;
    opt.kl_sh = key_logits_shared;
    opt.zr = read_router_logits;
    opt.kr = read_topk;
    opt.schedule = schedule;
    opt.ridx_out = read_topk_idx;
    const int st = forward_impl(q, key_logits, v, log_alpha, router_logits, dtype, cu_seqlens,
                                num_seqs, max_seqlen, total_tokens, H, c, d, N, topk,
                                initial_states, o, final_states, topk_idx, topk_w, seg_offsets,
                                seg_tok, seg_slot, workspace, workspace_bytes, stream, opt);
    return debug_finish(st, stream);
}

size_t sse_forward_noalloc_max_bytes(void) { return kScratchBytes; }

int sse_forward_noalloc(const void* q, const void* key_logits, const void* v,
                        const void* log_alpha, const void* router_logits, int dtype,
                        const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                        int64_t total_tokens, int H, int c, int d, int N, int topk,
                        const float* initial_states, float* o, float* final_states,
                        int32_t* topk_idx, float* topk_w, void* stream) {
    const int st = forward_impl(q, key_logits, v, log_alpha, router_logits, dtype, cu_seqlens,
                                num_seqs, max_seqlen, total_tokens, H, c, d, N, topk,
                                initial_states, o, final_states, topk_idx, topk_w, nullptr,
                                nullptr, nullptr, nullptr, 0, stream, scratch_opts());
    return debug_finish(st, stream);
}

size_t sse_rowsparse_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                     int c, int d) {
    if (check_rowsparse(SSE_BF16, H, c, d, 1) != SSE_OK) return 0;
    RsLayout L;
    if (!rowsparse_layout(total_tokens, num_seqs, max_seqlen, H, c, d, L)) return 0;
    return L.total;
}

int sse_rowsparse_forward(const void* q, const void* key_logits, const void* v,
                          const void* log_alpha, int dtype, const int32_t* cu_seqlens, int num_seqs,
                          int max_seqlen, int64_t total_tokens, int H, int c, int d, int row_topk,
                          int identity_unselected, const float* initial_states, float* o,
                          float* final_states, void* workspace, size_t workspace_bytes,
                          void* stream) {
    int st = check_rowsparse(dtype, H, c, d, row_topk);
    if (st != SSE_OK) return st;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !key_logits || !v || !log_alpha || !o)) return SSE_ERR_INVALID_ARG;
    if (num_seqs > 0 && !final_states) return SSE_ERR_INVALID_ARG;
    RsLayout L;
    if (!rowsparse_layout(total_tokens, num_seqs, max_seqlen, H, c, d, L)) return SSE_ERR_UNSUPPORTED;
    if (total_tokens * H * (c > d ? c : d) >= (int64_t(1) << 30)) return SSE_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return SSE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        st = debug_check_cu(cu_seqlens, num_seqs, total_tokens, max_seqlen, s);
        if (st != SSE_OK) return st;
    }
    char* ws = static_cast<char*>(workspace);
    sse::ChunkArgs a = {};
    a.q = q;
    a.kl = ws + L.kl;
    a.v = v;
    a.la = ws + L.la;
    a.cu = cu_seqlens;
    a.lnz2 = reinterpret_cast<float*>(ws + L.lnz2);
    a.lnz2_out = reinterpret_cast<float*>(ws + L.lnz2);
    a.init = initial_states;
    a.o = o;
    a.final_states = final_states;
    a.agg_S = reinterpret_cast<float*>(ws + L.agg_S);
    a.agg_D = reinterpret_cast<float*>(ws + L.agg_D);
    a.trash = reinterpret_cast<float*>(ws + L.trash);
    a.part = reinterpret_cast<float*>(ws + L.part);
    a.part_scale = reinterpret_cast<float*>(ws + L.part + sizeof(int16_t) * (size_t)d);
    a.slot_rows = 0;
    a.rows = (uint32_t)(total_tokens * H);
    a.num_seqs = num_seqs;
    a.H = H;
    a.N = 0;       // the single state is the shared partition's slot
    a.topk = 0;    // no routed reads to add
    a.piece_len = shared_piece_len(num_seqs, H, max_seqlen);
    a.max_pieces = max_pieces(max_seqlen, a.piece_len);
    hipError_t e = sse::launch_rowsparse_mask(key_logits, log_alpha, dtype, total_tokens * H, c,
                                              row_topk, identity_unselected, ws + L.kl,
                                              ws + L.la, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    if (num_seqs == 0) return debug_finish(SSE_OK, stream);
    e = sse::launch_chunk_local(a, dtype, c, d, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    return debug_finish(hip_status(sse::launch_chunk_shared(a, dtype, c, d, s)), stream);
}

size_t sse_backward_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H,
                                    int c, int d, int N, int topk) {
    if (check_common(SSE_BF16, H, c, d, N, topk) != SSE_OK) return 0;
    BwdLayout L;
    if (!backward_layout(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk, L)) return 0;
    return L.total;
}

int sse_backward(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                 const void* router_logits, int dtype, const int32_t* cu_seqlens, int num_seqs,
                 int max_seqlen, int64_t total_tokens, int H, int c, int d, int N, int topk,
                 const float* initial_states, const float* d_o, const float* d_final_states,
                 float* dq, float* dkey_logits, float* dv, float* dlog_alpha,
                 float* drouter_logits, float* dinitial_states, void* workspace,
                 size_t workspace_bytes, void* stream) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !d_o ||
                             !dq || !dkey_logits || !dv || !dlog_alpha || !drouter_logits))
        return SSE_ERR_INVALID_ARG;
    BwdLayout L;
    if (!backward_layout(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk, L))
        return SSE_ERR_UNSUPPORTED;
    if (total_tokens * H * (topk + 1) * (c > d ? c : d) >= (int64_t(1) << 31))
        return SSE_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return SSE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_on()) {
        st = debug_check_cu(cu_seqlens, num_seqs, total_tokens, max_seqlen, s);
        if (st != SSE_OK) return st;
    }
    char* ws = static_cast<char*>(workspace);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + L.f.idx);
    float* w = reinterpret_cast<float*>(ws + L.f.w);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.f.counts);
    int32_t* seg_off = reinterpret_cast<int32_t*>(ws + L.f.seg_off);
    uint2* rinfo = reinterpret_cast<uint2*>(ws + L.f.rinfo);
    sse::SegRec* seg_rec = reinterpret_cast<sse::SegRec*>(ws + L.f.seg_rec);
    float* lnz2 = reinterpret_cast<float*>(ws + L.f.lnz2);
    // the forward's routing and grouping (the segments the reverse pass walks)
    hipError_t e = sse::launch_route_count(router_logits, key_logits, dtype, cu_seqlens, num_seqs,
                                           max_seqlen, total_tokens, H, c, N, topk, idx, w,
                                           counts, rinfo, lnz2, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    e = sse::launch_group_fwd(rinfo, cu_seqlens, num_seqs, max_seqlen, total_tokens, H, N, topk,
                              counts, seg_off, lnz2, seg_rec, s);
    if (e != hipSuccess) return SSE_ERR_HIP;
    sse::BwdArgs a = {};
    a.q = q;
    a.kl = key_logits;
    a.v = v;
    a.la = log_alpha;
    a.z = router_logits;
    a.cu = cu_seqlens;
    a.seg_offsets = seg_off;
    a.seg_rec = seg_rec;
    a.sel_idx = idx;
    a.lnz2 = lnz2;
    a.init = initial_states;
    a.dfinal = d_final_states;
    a.dout = d_o;
    a.ckS = reinterpret_cast<float*>(ws + L.ckS);
    a.ckG = reinterpret_cast<float*>(ws + L.ckG);
    a.slot_meta = reinterpret_cast<sse::BwdRec*>(ws + L.tab);
    a.nslot = L.nslot;
    a.sh_slots = L.sh_slots;
    a.g_dq = reinterpret_cast<float*>(ws + L.g_dq);
    a.g_dkl = reinterpret_cast<float*>(ws + L.g_dkl);
    a.g_dla = reinterpret_cast<float*>(ws + L.g_dla);
    a.g_dv = reinterpret_cast<float*>(ws + L.g_dv);
    a.g_dw = reinterpret_cast<float*>(ws + L.g_dw);
    a.dq = dq;
    a.dkl = dkey_logits;
    a.dla = dlog_alpha;
    a.dv = dv;
    a.dz = drouter_logits;
    a.dinit = dinitial_states;
    a.rows = total_tokens * H;
    a.num_seqs = num_seqs;
    a.H = H;
    a.N = N;
    a.topk = topk;
    return debug_finish(hip_status(sse::launch_backward(a, dtype, c, d, s)), stream);
}

int sse_trace_enable(int enable) {
    if (enable && !g_trace.created) {
        for (int i = 0; i < kTraceCalls; i++)
            for (int j = 0; j < kTraceMarks; j++)
                if (hipEventCreate(&g_trace.ev[i][j]) != hipSuccess) {
                    // release the events made so far; tracing stays off
                    for (int x = 0; x <= i; x++)
                        for (int y = 0; y < (x < i ? kTraceMarks : j); y++)
                            (void)hipEventDestroy(g_trace.ev[x][y]);
                    g_trace.on = false;
                    return SSE_ERR_HIP;
                }
        g_trace.created = true;
    }
    g_trace.on = enable != 0;
    g_trace.calls = 0;
    return SSE_OK;
}

int sse_trace_read(float* ms_per_stage, int n_stages, int64_t* calls) {
    if (!ms_per_stage || n_stages < 1 || n_stages > SSE_TRACE_STAGES || !calls)
        return SSE_ERR_INVALID_ARG;
    for (int j = 0; j < n_stages; j++) ms_per_stage[j] = 0.f;
    const int64_t n = g_trace.calls < kTraceCalls ? g_trace.calls : kTraceCalls;
    *calls = n;
    if (!g_trace.created || n == 0) return SSE_OK;
    for (int64_t i = 0; i < n; i++) {
        hipEvent_t* ev = g_trace.ev[(g_trace.calls - n + i) % kTraceCalls];
        if (hipEventSynchronize(ev[kTraceMarks - 1]) != hipSuccess) return SSE_ERR_HIP;
        for (int j = 0; j < n_stages; j++) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, ev[j], ev[j + 1]) != hipSuccess) return SSE_ERR_HIP;
            ms_per_stage[j] += ms;
        }
    }
    g_trace.calls = 0;
    return SSE_OK;
}

int sse_debug_checks(int mode) {
    if (mode == 0 || mode == 1) {
        debug_on();   // read the environment first, so it cannot override this call later
        g_debug.store(mode);
    }
    return debug_on() ? 1 : 0;
}

int sse_decode_step(const void* q, const void* key_logits, const void* v, const void* log_alpha,
                    const void* router_logits, int dtype, int B, int H, int c, int d, int N,
                    int topk, float* states, float* o, int32_t* topk_idx, void* stream) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    if (B < 0) return SSE_ERR_INVALID_ARG;
    // one 256-thread block per (b, h, 32 columns): the grid's work-items must
    // stay below 2^32
    if ((int64_t)B * H * (d / 32) * 256 >= ((int64_t)1 << 32)) return SSE_ERR_UNSUPPORTED;
    if (B > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !states || !o))
        return SSE_ERR_INVALID_ARG;
    const hipError_t e =
        sse::launch_decode(q, key_logits, v, log_alpha, router_logits, dtype, B, H, c, d, N, topk,
                           states, o, topk_idx, static_cast<hipStream_t>(stream));
    return debug_finish(hip_status(e), stream);
}

int sse_decode_step_ex(const void* q, const void* key_logits, const void* v,
                       const void* log_alpha, const void* router_logits, int dtype, int B, int H,
                       int c, int d, int N, int topk, const void* q_shared,
                       const void* key_logits_shared, const void* read_router_logits,
                       int read_topk, float* states, float* o, int32_t* topk_idx,
                       int32_t* read_topk_idx, void* stream) {
    int st = check_common(dtype, H, c, d, N, topk);
    if (st != SSE_OK) return st;
    if (B < 0) return SSE_ERR_INVALID_ARG;
    if (read_router_logits) {
        if (read_topk < 1 || read_topk > N) return SSE_ERR_INVALID_ARG;
        if (read_topk > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    } else if (read_topk_idx) {
        return SSE_ERR_INVALID_ARG;
    }
    if ((int64_t)B * H * (d / 32) * 256 >= ((int64_t)1 << 32)) return SSE_ERR_UNSUPPORTED;
    if (B > 0 && (!q || !key_logits || !v || !log_alpha || !router_logits || !states || !o))
        return SSE_ERR_INVALID_ARG;
    const hipError_t e = sse::launch_decode_ex(
        q, key_logits, v, log_alpha, router_logits, q_shared, key_logits_shared,
        read_router_logits, dtype, B, H, c, d, N, topk, read_router_logits ? read_topk : 0, states,
        o, topk_idx, read_topk_idx, static_cast<hipStream_t>(stream));
    return debug_finish(hip_status(e), stream);
}

int sse_router_topk(const void* router_logits, int dtype, int64_t rows, int N, int topk,
                    int32_t* topk_idx, float* topk_w, void* stream) {
    if (dtype != SSE_F32 && dtype != SSE_BF16) return SSE_ERR_INVALID_ARG;
    if (rows < 0 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (N > sse::kMaxN || topk > sse::kMaxTopK) return SSE_ERR_UNSUPPORTED;
    if (rows * topk >= INT_MAX) return SSE_ERR_UNSUPPORTED;
    if (rows > 0 && (!router_logits || !topk_idx || !topk_w)) return SSE_ERR_INVALID_ARG;
    const hipError_t e = sse::launch_router_rows(router_logits, dtype, rows, N, topk, topk_idx,
                                                 topk_w, static_cast<hipStream_t>(stream));
    return debug_finish(hip_status(e), stream);
}

size_t sse_group_workspace_bytes(int64_t total_tokens, int num_seqs, int max_seqlen, int H, int N,
                                 int topk) {
    if (N < 1 || topk < 1 || topk > N || N > sse::kMaxN || topk > sse::kMaxTopK) return 0;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, 0, 0, N, topk, L)) return 0;
    return L.seg_off - L.counts;
}

int sse_group_by_partition(const int32_t* topk_idx, const float* topk_w,
                           const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                           int64_t total_tokens, int H, int N, int topk, int32_t* seg_offsets,
                           int32_t* seg_tok, int32_t* seg_slot, float* seg_w, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (H < 1 || N < 1 || topk < 1 || topk > N) return SSE_ERR_INVALID_ARG;
    if (N > sse::kMaxN || topk > sse::kMaxTopK || H > sse::kMaxH) return SSE_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 0 || max_seqlen < 0) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && num_seqs == 0) return SSE_ERR_INVALID_ARG;
    if (!cu_seqlens || !seg_offsets) return SSE_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!topk_idx || !seg_tok)) return SSE_ERR_INVALID_ARG;
    if (seg_w && !topk_w) return SSE_ERR_INVALID_ARG;
    FwdLayout L;
    if (!forward_layout(total_tokens, num_seqs, max_seqlen, H, 0, 0, N, topk, L))
        return SSE_ERR_UNSUPPORTED;
    const size_t need = L.seg_off - L.counts;
    if (workspace_bytes < need || (need > 0 && !workspace)) return SSE_ERR_WORKSPACE;
    if (debug_on()) {
        const int st = debug_check_cu(cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                      static_cast<hipStream_t>(stream));
        if (st != SSE_OK) return st;
    }
    const hipError_t e = sse::launch_group(topk_idx, topk_w, cu_seqlens, num_seqs, max_seqlen, H,
                                           N, topk, static_cast<int32_t*>(workspace), seg_offsets,
                                           seg_tok, seg_slot, seg_w,
                                           static_cast<hipStream_t>(stream));
    return debug_finish(hip_status(e), stream);
}

}  // extern "C"
