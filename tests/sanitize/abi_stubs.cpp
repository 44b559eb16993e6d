// Launcher stubs for the host-only sanitizer build of the C-ABI layer
// (sse_api.hip): argument validation, workspace carving and the status
// paths are exercised under AddressSanitizer / UndefinedBehaviorSanitizer on
// a machine without a GPU.  Every stub reports a failed launch; the tests
// that use this build only make calls that the host checks reject, plus
// calls with nothing to do.
#include "sse_launch.h"

namespace sse {

static hipError_t stub() { return hipErrorInvalidValue; }

hipError_t launch_router_rows(const void*, int, int64_t, int, int, int32_t*, float*, hipStream_t) {
    return stub();
}
hipError_t launch_route_count(const void*, const void*, int, const int32_t*, int, int, int64_t,
                              int, int, int, int, int32_t*, float*, int32_t*, uint2*, float*,
                              hipStream_t) {
    return stub();
}
hipError_t launch_group(const int32_t*, const float*, const int32_t*, int, int, int, int, int,
                        int32_t*, int32_t*, int32_t*, int32_t*, float*, hipStream_t) {
    return stub();
}
hipError_t launch_group_fwd(const uint2*, const int32_t*, int, int, int64_t, int, int, int,
                            int32_t*, int32_t*, const float*, SegRec*, hipStream_t) {
    return stub();
}
hipError_t launch_seg_debug(const SegRec*, const int32_t*, int64_t, int64_t, int, int, int32_t*,
                            int32_t*, int32_t*, hipStream_t) {
    return stub();
}
hipError_t launch_chunk_local(const ChunkArgs&, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_piece_state(const ChunkArgs&, int, int, hipStream_t) { return stub(); }
hipError_t launch_chunk_shared(const ChunkArgs&, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_chunk_routed(const ChunkArgs&, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_chunk_f64(int, const ChunkArgs&, int, int, hipStream_t) { return stub(); }
hipError_t launch_chunk_masked(const ChunkArgs&, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_key_norm(const void*, int, int64_t, int, float*, hipStream_t) { return stub(); }
hipError_t launch_rowsparse_mask(const void*, const void*, int, int64_t, int, int, int, void*,
                                 void*, hipStream_t) {
    return stub();
}
hipError_t launch_backward(const BwdArgs&, int, int, int, hipStream_t) { return stub(); }
hipError_t launch_decode(const void*, const void*, const void*, const void*, const void*, int, int,
                         int, int, int, int, int, float*, float*, int32_t*, hipStream_t) {
    return stub();
}

hipError_t launch_decode_ex(const void*, const void*, const void*, const void*, const void*,
                            const void*, const void*, const void*, int, int, int, int, int, int,
                            int, int, float*, float*, int32_t*, int32_t*, hipStream_t) {
    return stub();
}

}  // namespace sse
