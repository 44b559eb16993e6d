"""Python binding of the gfx950 Sparse State Expansion (SSE) library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libsse_amd.so`` (built in-tree by ``sparse_state_linear_amd.build``),
reached through the C ABI of ``include/sse.h``.  PyTorch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
missing, every entry point raises.

Names mirror the C entry points: ``sse_forward``, ``sse_decode_step``,
``sse_router_topk``, ``sse_group_by_partition`` and the workspace queries.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SSE_LIB_PATH selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("SSE_LIB_PATH") or os.path.join(_PKG, "libsse_amd.so")

SSE_OK, SSE_ERR_INVALID_ARG, SSE_ERR_UNSUPPORTED, SSE_ERR_WORKSPACE, SSE_ERR_HIP = range(5)
SSE_F32, SSE_BF16 = 0, 1
SSE_SCHEDULE_VARLEN, SSE_SCHEDULE_MASKED = 0, 1
SCHEDULES = {"varlen": SSE_SCHEDULE_VARLEN, "masked": SSE_SCHEDULE_MASKED}

EXPORTED = ("sse_status_string", "sse_version", "sse_forward_workspace_bytes", "sse_forward",
            "sse_forward_noalloc_max_bytes", "sse_forward_noalloc",
            "sse_forward_ex_workspace_bytes", "sse_forward_ex",
            "sse_backward_workspace_bytes", "sse_backward",
            "sse_decode_step", "sse_decode_step_ex", "sse_router_topk", "sse_group_workspace_bytes",
            "sse_group_by_partition", "sse_rowsparse_workspace_bytes", "sse_rowsparse_forward",
            "sse_trace_enable", "sse_trace_read", "sse_debug_checks")

_lib = None


class SSEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def lib():
    """Load libsse_amd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_state_linear_amd.build` "
            "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.sse_status_string.argtypes = [I]
    L.sse_status_string.restype = ctypes.c_char_p
    L.sse_version.argtypes = []
    L.sse_version.restype = I
    L.sse_forward_workspace_bytes.argtypes = [I64, I, I, I, I, I, I, I]
    L.sse_forward_workspace_bytes.restype = SZ
    L.sse_forward.argtypes = [P, P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P, P, P,
                              P, P, P, SZ, P]
    L.sse_forward.restype = I
    L.sse_forward_ex_workspace_bytes.argtypes = [I64, I, I, I, I, I, I, I, I]
    L.sse_forward_ex_workspace_bytes.restype = SZ
    L.sse_forward_ex.argtypes = [P, P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, I, I, P,
                                 P, P, P, P, P, P, P, P, P, SZ, P]
    L.sse_forward_ex.restype = I
    L.sse_backward_workspace_bytes.argtypes = [I64, I, I, I, I, I, I, I]
    L.sse_backward_workspace_bytes.restype = SZ
    L.sse_backward.argtypes = [P, P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P, P, P,
                               P, P, P, P, SZ, P]
    L.sse_backward.restype = I
    L.sse_forward_noalloc_max_bytes.argtypes = []
    L.sse_forward_noalloc_max_bytes.restype = SZ
    L.sse_forward_noalloc.argtypes = [P, P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P,
                                      P, P]
    L.sse_forward_noalloc.restype = I
    L.sse_decode_step.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, P, P, P]
    L.sse_decode_step.restype = I
    L.sse_decode_step_ex.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, P, P, I, P, P, P, P,
                                     P]
    L.sse_decode_step_ex.restype = I
    L.sse_router_topk.argtypes = [P, I, I64, I, I, P, P, P]
    L.sse_router_topk.restype = I
    L.sse_group_workspace_bytes.argtypes = [I64, I, I, I, I, I]
    L.sse_group_workspace_bytes.restype = SZ
    L.sse_group_by_partition.argtypes = [P, P, P, I, I, I64, I, I, I, P, P, P, P, P, SZ, P]
    L.sse_group_by_partition.restype = I
    L.sse_rowsparse_workspace_bytes.argtypes = [I64, I, I, I, I, I]
    L.sse_rowsparse_workspace_bytes.restype = SZ
    L.sse_rowsparse_forward.argtypes = [P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P,
                                        SZ, P]
    L.sse_rowsparse_forward.restype = I
    L.sse_trace_enable.argtypes = [I]
    L.sse_trace_enable.restype = I
    L.sse_debug_checks.argtypes = [I]
    L.sse_debug_checks.restype = I
    L.sse_trace_read.argtypes = [P, I, P]
    L.sse_trace_read.restype = I
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().sse_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SSE_OK:
        raise SSEError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSE_BF16
    if t.dtype == torch.float32:
        return SSE_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _need(t, shape, dtype, name, device):
    if t.shape != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def sse_forward_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk) -> int:
    return int(lib().sse_forward_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d, N,
                                                 topk))


def sse_forward(q, key_logits, v, log_alpha, router_logits, N, topk, cu_seqlens, max_seqlen=None,
                initial_states=None, *, o=None, final_states=None, topk_idx=None, topk_w=None,
                seg_offsets=None, seg_tok=None, seg_slot=None, workspace=None):
    """Varlen SSE forward.  q/key_logits/log_alpha [T,H,c], v [T,H,d],
    router_logits [T,H,N] (bf16 or fp32, one dtype), cu_seqlens int32
    [S+1] on the device.  Returns (o [T,H,d] fp32, final_states
    [S,H,N+1,c,d] fp32).  Optional preallocated outputs/workspace avoid
    allocation; ``max_seqlen`` (host int) avoids a device->host read.
    ``seg_offsets`` [S*H*N+1], ``seg_tok`` / ``seg_slot`` [T*H*topk] (int32,
    optional) receive the grouping this call ran."""
    dev = q.device
    T, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (T, H, c), "q"), (key_logits, (T, H, c), "key_logits"),
                       (log_alpha, (T, H, c), "log_alpha"), (v, (T, H, d), "v"),
                       (router_logits, (T, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S > 0 else 0
    if initial_states is not None:
        _need(initial_states, (S, H, N + 1, c, d), torch.float32, "initial_states", dev)
    if o is None:
        o = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    if final_states is None:
        final_states = torch.empty((S, H, N + 1, c, d), dtype=torch.float32, device=dev)
    for t, n_, nm in ((seg_offsets, S * H * N + 1, "seg_offsets"),
                      (seg_tok, T * H * topk, "seg_tok"), (seg_slot, T * H * topk, "seg_slot")):
        if t is not None:
            _need(t, (n_,), torch.int32, nm, dev)
    for t, nm in ((topk_idx, "topk_idx"), (topk_w, "topk_w")):
        if t is not None:
            _need(t, (T, H, topk), torch.int32 if nm == "topk_idx" else torch.float32, nm, dev)
    ws_bytes = sse_forward_workspace_bytes(T, S, max_seqlen, H, c, d, N, topk)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sse_forward(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                           _ptr(router_logits), _dtype_code(q), _ptr(cu_seqlens), S,
                           int(max_seqlen), T, H, c, d, N, topk, _ptr(initial_states), _ptr(o),
                           _ptr(final_states), _ptr(topk_idx), _ptr(topk_w), _ptr(seg_offsets),
                           _ptr(seg_tok), _ptr(seg_slot), _ptr(workspace), workspace.numel(),
                           _stream(dev))
    _check(st, "sse_forward")
    return o, final_states


def sse_forward_ex_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk,
                                   read_topk=0) -> int:
    return int(lib().sse_forward_ex_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d,
                                                    N, topk, read_topk))


def sse_forward_ex(q, key_logits, v, log_alpha, router_logits, N, topk, cu_seqlens,
                   max_seqlen=None, initial_states=None, *, q_shared=None, key_logits_shared=None,
                   read_router_logits=None, read_topk=None, schedule="varlen", o=None,
                   final_states=None, topk_idx=None, topk_w=None, read_topk_idx=None,
                   seg_offsets=None, seg_tok=None, seg_slot=None, workspace=None):
    """General forward: the shared partition's own q / key logits, read sets
    from their own router logits (masked schedule), and the choice of the
    varlen or masked schedule.  Returns (o, final_states) as sse_forward."""
    dev = q.device
    T, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (T, H, c), "q"), (key_logits, (T, H, c), "key_logits"),
                       (log_alpha, (T, H, c), "log_alpha"), (v, (T, H, d), "v"),
                       (router_logits, (T, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    for t, shp, nm in ((q_shared, (T, H, c), "q_shared"),
                       (key_logits_shared, (T, H, c), "key_logits_shared"),
                       (read_router_logits, (T, H, N), "read_router_logits")):
        if t is not None:
            _need(t, shp, dt, nm, dev)
    kr = 0 if read_router_logits is None else int(read_topk)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S > 0 else 0
    if initial_states is not None:
        _need(initial_states, (S, H, N + 1, c, d), torch.float32, "initial_states", dev)
    if o is None:
        o = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    if final_states is None:
        final_states = torch.empty((S, H, N + 1, c, d), dtype=torch.float32, device=dev)
    nbytes = sse_forward_ex_workspace_bytes(T, S, max_seqlen, H, c, d, N, topk, kr)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sse_forward_ex(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                              _ptr(router_logits), _dtype_code(q), _ptr(cu_seqlens), S,
                              int(max_seqlen), T, H, c, d, N, topk, _ptr(q_shared),
                              _ptr(key_logits_shared), _ptr(read_router_logits), kr,
                              SCHEDULES[schedule], _ptr(initial_states), _ptr(o),
                              _ptr(final_states), _ptr(topk_idx), _ptr(topk_w),
                              _ptr(read_topk_idx), _ptr(seg_offsets), _ptr(seg_tok),
                              _ptr(seg_slot), _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "sse_forward_ex")
    return o, final_states


def sse_backward_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d, N, topk) -> int:
    return int(lib().sse_backward_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d, N,
                                                  topk))


def sse_backward(q, key_logits, v, log_alpha, router_logits, N, topk, cu_seqlens, d_o,
                 max_seqlen=None, initial_states=None, d_final_states=None, *,
                 want_dinitial=False, workspace=None, out=None):
    """Gradients of <d_o, o> + <d_final_states, final_states> of sse_forward.
    Returns a dict of fp32 tensors dq, dkey_logits, dlog_alpha [T,H,c], dv
    [T,H,d], drouter_logits [T,H,N] and (want_dinitial) dinitial_states
    [S,H,N+1,c,d].  ``out`` may hold preallocated tensors under those names."""
    dev = q.device
    T, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (T, H, c), "q"), (key_logits, (T, H, c), "key_logits"),
                       (log_alpha, (T, H, c), "log_alpha"), (v, (T, H, d), "v"),
                       (router_logits, (T, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    _need(d_o, (T, H, d), torch.float32, "d_o", dev)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S > 0 else 0
    for t, nm in ((initial_states, "initial_states"), (d_final_states, "d_final_states")):
        if t is not None:
            _need(t, (S, H, N + 1, c, d), torch.float32, nm, dev)
    shapes = {"dq": (T, H, c), "dkey_logits": (T, H, c), "dlog_alpha": (T, H, c),
              "dv": (T, H, d), "drouter_logits": (T, H, N)}
    if want_dinitial:
        shapes["dinitial_states"] = (S, H, N + 1, c, d)
    res = {}
    for nm, shp in shapes.items():
        t = None if out is None else out.get(nm)
        if t is None:
            t = torch.empty(shp, dtype=torch.float32, device=dev)
        _need(t, shp, torch.float32, nm, dev)
        res[nm] = t
    nbytes = sse_backward_workspace_bytes(T, S, max_seqlen, H, c, d, N, topk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sse_backward(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                            _ptr(router_logits), _dtype_code(q), _ptr(cu_seqlens), S,
                            int(max_seqlen), T, H, c, d, N, topk, _ptr(initial_states),
                            _ptr(d_o), _ptr(d_final_states), _ptr(res["dq"]),
                            _ptr(res["dkey_logits"]), _ptr(res["dv"]), _ptr(res["dlog_alpha"]),
                            _ptr(res["drouter_logits"]), _ptr(res.get("dinitial_states")),
                            _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "sse_backward")
    return res


def sse_forward_noalloc_max_bytes() -> int:
    return int(lib().sse_forward_noalloc_max_bytes())


def sse_forward_noalloc(q, key_logits, v, log_alpha, router_logits, N, topk, cu_seqlens,
                        max_seqlen, o, final_states, initial_states=None, *, topk_idx=None,
                        topk_w=None):
    """sse_forward with the library's static workspace: the caller passes
    every output (o [T,H,d], final_states [S,H,N+1,c,d] fp32) and the host
    max_seqlen, and nothing is allocated.  Raises SSEError
    (SSE_ERR_WORKSPACE) when the sizes need more than
    sse_forward_noalloc_max_bytes() of workspace."""
    dev = q.device
    T, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (T, H, c), "q"), (key_logits, (T, H, c), "key_logits"),
                       (log_alpha, (T, H, c), "log_alpha"), (v, (T, H, d), "v"),
                       (router_logits, (T, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    _need(o, (T, H, d), torch.float32, "o", dev)
    _need(final_states, (S, H, N + 1, c, d), torch.float32, "final_states", dev)
    if initial_states is not None:
        _need(initial_states, (S, H, N + 1, c, d), torch.float32, "initial_states", dev)
    st = lib().sse_forward_noalloc(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                                   _ptr(router_logits), _dtype_code(q), _ptr(cu_seqlens), S,
                                   int(max_seqlen), T, H, c, d, N, topk, _ptr(initial_states),
                                   _ptr(o), _ptr(final_states), _ptr(topk_idx), _ptr(topk_w),
                                   _stream(dev))
    _check(st, "sse_forward_noalloc")
    return o, final_states


def sse_decode_step(q, key_logits, v, log_alpha, router_logits, N, topk, states, *, o=None,
                    topk_idx=None):
    """One decode token per (b, h).  Inputs [B,H,.]; ``states``
    [B,H,N+1,c,d] fp32 is updated in place.  Returns o [B,H,d] fp32."""
    dev = q.device
    B, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (B, H, c), "q"), (key_logits, (B, H, c), "key_logits"),
                       (log_alpha, (B, H, c), "log_alpha"), (v, (B, H, d), "v"),
                       (router_logits, (B, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    _need(states, (B, H, N + 1, c, d), torch.float32, "states", dev)
    if o is None:
        o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    st = lib().sse_decode_step(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                               _ptr(router_logits), _dtype_code(q), B, H, c, d, N, topk,
                               _ptr(states), _ptr(o), _ptr(topk_idx), _stream(dev))
    _check(st, "sse_decode_step")
    return o


def sse_decode_step_ex(q, key_logits, v, log_alpha, router_logits, N, topk, states, *,
                       q_shared=None, key_logits_shared=None, read_router_logits=None,
                       read_topk=0, o=None, topk_idx=None, read_topk_idx=None):
    """Decode step with the shared partition's own query / key logits and a
    read set from its own router logits (each optional).  ``states``
    [B,H,N+1,c,d] fp32 is updated in place.  Returns o [B,H,d] fp32."""
    dev = q.device
    B, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (B, H, c), "q"), (key_logits, (B, H, c), "key_logits"),
                       (log_alpha, (B, H, c), "log_alpha"), (v, (B, H, d), "v"),
                       (router_logits, (B, H, N), "router_logits")):
        _need(t, shp, dt, nm, dev)
    for t, shp, nm in ((q_shared, (B, H, c), "q_shared"),
                       (key_logits_shared, (B, H, c), "key_logits_shared"),
                       (read_router_logits, (B, H, N), "read_router_logits")):
        if t is not None:
            _need(t, shp, dt, nm, dev)
    _need(states, (B, H, N + 1, c, d), torch.float32, "states", dev)
    if o is None:
        o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    st = lib().sse_decode_step_ex(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                                  _ptr(router_logits), _dtype_code(q), B, H, c, d, N, topk,
                                  _ptr(q_shared), _ptr(key_logits_shared),
                                  _ptr(read_router_logits), int(read_topk), _ptr(states),
                                  _ptr(o), _ptr(topk_idx), _ptr(read_topk_idx), _stream(dev))
    _check(st, "sse_decode_step_ex")
    return o


def sse_router_topk(router_logits, topk):
    """Router alone: [rows, N] logits -> (topk_idx int32, topk_w fp32) [rows, topk]."""
    dev = router_logits.device
    N = router_logits.shape[-1]
    z = router_logits.reshape(-1, N)
    if not z.is_contiguous():
        raise ValueError("router_logits must be contiguous")
    rows = z.shape[0]
    idx = torch.empty((rows, topk), dtype=torch.int32, device=dev)
    w = torch.empty((rows, topk), dtype=torch.float32, device=dev)
    st = lib().sse_router_topk(_ptr(z), _dtype_code(z), rows, N, topk, _ptr(idx), _ptr(w),
                               _stream(dev))
    _check(st, "sse_router_topk")
    return idx, w


def sse_group_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, N, topk) -> int:
    return int(lib().sse_group_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, N, topk))


def sse_group_by_partition(topk_idx, topk_w, cu_seqlens, N, max_seqlen=None):
    """Stable grouping of [T,H,k] top-k choices into (sequence, head,
    partition) segments.  Returns (seg_offsets, seg_tok, seg_slot, seg_w)."""
    dev = topk_idx.device
    T, H, K = topk_idx.shape
    _need(topk_idx, (T, H, K), torch.int32, "topk_idx", dev)
    if topk_w is not None:
        _need(topk_w, (T, H, K), torch.float32, "topk_w", dev)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S > 0 else 0
    off = torch.empty(S * H * N + 1, dtype=torch.int32, device=dev)
    tok = torch.empty(T * H * K, dtype=torch.int32, device=dev)
    slot = torch.empty(T * H * K, dtype=torch.int32, device=dev)
    sw = torch.empty(T * H * K, dtype=torch.float32, device=dev) if topk_w is not None else None
    nbytes = sse_group_workspace_bytes(T, S, max_seqlen, H, N, K)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sse_group_by_partition(_ptr(topk_idx), _ptr(topk_w), _ptr(cu_seqlens), S,
                                      int(max_seqlen), T, H, N, K, _ptr(off), _ptr(tok),
                                      _ptr(slot), _ptr(sw), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "sse_group_by_partition")
    return off, tok, slot, sw


def sse_rowsparse_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d) -> int:
    return int(lib().sse_rowsparse_workspace_bytes(total_tokens, num_seqs, max_seqlen, H, c, d))


def sse_rowsparse_forward(q, key_logits, v, log_alpha, row_topk, cu_seqlens, max_seqlen=None,
                          initial_states=None, identity_unselected=True, *, o=None,
                          final_states=None, workspace=None):
    """Row-sparse top-k key variant: one state per head, key = softmax over
    the row_topk largest key logits, unselected rows keep their state
    (identity_unselected) or decay.  q/key_logits/log_alpha [T,H,c], v [T,H,d]
    (bf16 or fp32), cu_seqlens int32 [S+1].  Returns (o [T,H,d], final_states
    [S,H,c,d]) in fp32."""
    dev = q.device
    T, H, c = q.shape
    d = v.shape[2]
    dt = q.dtype
    for t, shp, nm in ((q, (T, H, c), "q"), (key_logits, (T, H, c), "key_logits"),
                       (log_alpha, (T, H, c), "log_alpha"), (v, (T, H, d), "v")):
        _need(t, shp, dt, nm, dev)
    S = cu_seqlens.shape[0] - 1
    _need(cu_seqlens, (S + 1,), torch.int32, "cu_seqlens", dev)
    if max_seqlen is None:
        max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if S > 0 else 0
    if initial_states is not None:
        _need(initial_states, (S, H, c, d), torch.float32, "initial_states", dev)
    if o is None:
        o = torch.empty((T, H, d), dtype=torch.float32, device=dev)
    if final_states is None:
        final_states = torch.empty((S, H, c, d), dtype=torch.float32, device=dev)
    nbytes = sse_rowsparse_workspace_bytes(T, S, max_seqlen, H, c, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = lib().sse_rowsparse_forward(_ptr(q), _ptr(key_logits), _ptr(v), _ptr(log_alpha),
                                     _dtype_code(q), _ptr(cu_seqlens), S, int(max_seqlen), T, H,
                                     c, d, int(row_topk), int(bool(identity_unselected)),
                                     _ptr(initial_states), _ptr(o), _ptr(final_states),
                                     _ptr(workspace), workspace.numel(), _stream(dev))
    _check(st, "sse_rowsparse_forward")
    return o, final_states


def sse_debug_checks(mode=None) -> bool:
    """Switch the library's debug mode on (True) or off (False), or query it
    (None): host checks of cu_seqlens before any launch and a stream
    synchronisation after every call.  Returns the mode in effect."""
    m = -1 if mode is None else int(bool(mode))
    return bool(lib().sse_debug_checks(m))


TRACE_STAGES = ("route_count", "piece_state", "group", "routed", "shared")


def sse_trace_enable(enable: bool = True):
    """Start (or stop) recording HIP events around the forward's stages."""
    _check(lib().sse_trace_enable(int(bool(enable))), "sse_trace_enable")


def sse_trace_read():
    """Summed milliseconds per forward stage since the last read, and the
    number of calls they cover (waits for those calls to finish)."""
    ms = (ctypes.c_float * len(TRACE_STAGES))()
    calls = ctypes.c_int64(0)
    _check(lib().sse_trace_read(ms, len(TRACE_STAGES), ctypes.byref(calls)), "sse_trace_read")
    return {n: float(ms[i]) for i, n in enumerate(TRACE_STAGES)}, int(calls.value)
