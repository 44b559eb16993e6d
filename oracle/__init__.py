"""Plain fp64 CPU oracle for the Sparse State Expansion (SSE) layer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``sparse_state_linear_amd``) never imports this package and shares no code
with it.

The arithmetic lives in ``sse_oracle.c`` (plain C, fp64, sequential per
(sequence, head) unit); this module only builds it with gcc and marshals
numpy arrays through ctypes.  The method follows the web page "Scaling
Linear Attention with Sparse State Expansion: 中文研读笔记", §2.3 eqs. (9)-(14),
§2.5 (shared partition) and §2.6 (identity transition of unselected
partitions, varlen grouping).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sse_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsse_oracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (IEEE fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Werror",
           *extra_flags, "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load (building first if needed) an oracle shared object."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        path = _LIB_PATH
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    I64 = ctypes.c_int64
    lib.sse_oracle_unit.argtypes = [I, P, P, P, P, P, I64, I64, I, I, I, I, I, I, P, P, P, P]
    lib.sse_oracle_unit.restype = I
    lib.sse_oracle_forward.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, I]
    lib.sse_oracle_forward.restype = I
    lib.sse_oracle_decode_step.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P]
    lib.sse_oracle_decode_step.restype = I
    lib.sse_oracle_group.argtypes = [P, P, I, I, I, I, P, P, P]
    lib.sse_oracle_group.restype = I
    lib.sse_oracle_rowsparse_forward.argtypes = [I, P, P, P, P, P, I, I, I, I, I, I, P, P, P]
    lib.sse_oracle_rowsparse_forward.restype = I
    lib.sse_oracle_forward_ex.argtypes = [I, P, P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, P,
                                          P, P, P, P]
    lib.sse_oracle_forward_ex.restype = I
    lib.sse_oracle_backward.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P,
                                        P, P, P, I]
    lib.sse_oracle_backward.restype = I
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _raw(x):
    """Return (dtype code, contiguous array) for fp32 arrays or bf16 bit arrays."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return F32, x
    if x.dtype == np.uint16:
        return BF16, x
    raise TypeError(f"oracle inputs are fp32 arrays or uint16 bf16 bit patterns, got {x.dtype}")


def forward(q, key_logits, v, log_alpha, router_logits, cu_seqlens, N, topk,
            initial_states=None, threads=1, lib=None):
    """Full varlen forward.  Inputs token-major [T_tot, H, .] (fp32 or bf16
    bits), cu_seqlens int32 [S+1].  Returns a dict of fp64 o [T_tot,H,d],
    final_states [S,H,N+1,c,d], int32 topk_idx [T_tot,H,k], fp64 topk_e."""
    lib = lib or load()
    dt, q = _raw(q)
    arrs = [_raw(a) for a in (key_logits, v, log_alpha, router_logits)]
    if any(a[0] != dt for a in arrs):
        raise TypeError("all inputs must share one dtype")
    kl, v, la, z = (a[1] for a in arrs)
    T, H, c = q.shape
    d = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    assert kl.shape == (T, H, c) and la.shape == (T, H, c) and v.shape[:2] == (T, H)
    assert z.shape == (T, H, N) and int(cu[-1]) == T
    init = None
    if initial_states is not None:
        init = np.ascontiguousarray(initial_states, dtype=np.float64)
        assert init.shape == (S, H, N + 1, c, d)
    # np.empty on purpose: the oracle must write every element itself
    o = np.empty((T, H, d), np.float64)
    fs = np.empty((S, H, N + 1, c, d), np.float64)
    idx = np.empty((T, H, topk), np.int32)
    e = np.empty((T, H, topk), np.float64)
    rc = lib.sse_oracle_forward(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(z), _ptr(cu),
                                S, H, c, d, N, topk, _ptr(init), _ptr(o), _ptr(fs), _ptr(idx),
                                _ptr(e), int(threads))
    if rc != 0:
        raise ValueError("sse_oracle_forward rejected its arguments")
    return {"o": o, "final_states": fs, "topk_idx": idx, "topk_e": e}


def unit(q, key_logits, v, log_alpha, router_logits, t0, t1, h, N, topk, state=None, lib=None):
    """One (sequence, head) unit over tokens [t0, t1) of token-major inputs.
    ``state`` [N+1,c,d] fp64 is the initial state (zeros if None).  Returns
    (o [t1-t0, d], final state, topk_idx [t1-t0,k], topk_e)."""
    lib = lib or load()
    dt, q = _raw(q)
    kl, v, la, z = (_raw(a)[1] for a in (key_logits, v, log_alpha, router_logits))
    T, H, c = q.shape
    d = v.shape[2]
    L = t1 - t0
    S = np.zeros((N + 1, c, d), np.float64) if state is None else \
        np.array(state, dtype=np.float64, order="C", copy=True)
    o = np.zeros((L, d), np.float64)
    idx = np.zeros((L, topk), np.int32)
    e = np.zeros((L, topk), np.float64)
    rc = lib.sse_oracle_unit(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(z), t0, t1, h, H,
                             c, d, N, topk, _ptr(S), _ptr(o), _ptr(idx), _ptr(e))
    if rc != 0:
        raise ValueError("sse_oracle_unit rejected its arguments")
    return o, S, idx, e


def decode_step(q, key_logits, v, log_alpha, router_logits, states, N, topk, lib=None):
    """One decode token per (b, h).  Inputs [B,H,.]; ``states`` [B,H,N+1,c,d]
    fp64 is updated IN PLACE.  Returns (o [B,H,d], topk_idx, topk_e)."""
    lib = lib or load()
    dt, q = _raw(q)
    kl, v, la, z = (_raw(a)[1] for a in (key_logits, v, log_alpha, router_logits))
    B, H, c = q.shape
    d = v.shape[2]
    assert states.dtype == np.float64 and states.flags.c_contiguous
    assert states.shape == (B, H, N + 1, c, d)
    o = np.zeros((B, H, d), np.float64)
    idx = np.zeros((B, H, topk), np.int32)
    e = np.zeros((B, H, topk), np.float64)
    rc = lib.sse_oracle_decode_step(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(z), B, H, c,
                                    d, N, topk, _ptr(states), _ptr(o), _ptr(idx), _ptr(e))
    if rc != 0:
        raise ValueError("sse_oracle_decode_step rejected its arguments")
    return o, idx, e


def group(topk_idx, cu_seqlens, N, lib=None):
    """Stable grouping of (token, slot) records into (sequence, head,
    partition) segments.  Returns (seg_offsets [S*H*N+1], seg_tok, seg_slot)."""
    lib = lib or load()
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, H, k = idx.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    off = np.zeros(S * H * N + 1, np.int32)
    tok = np.zeros(T * H * k, np.int32)
    slot = np.zeros(T * H * k, np.int32)
    lib.sse_oracle_group(_ptr(idx), _ptr(cu), S, H, N, k, _ptr(off), _ptr(tok), _ptr(slot))
    return off, tok, slot


def rowsparse_forward(q, key_logits, v, log_alpha, cu_seqlens, row_topk, identity_unselected=True,
                      initial_states=None, lib=None):
    """Row-sparse top-k key variant (single state per head).  Inputs
    [T_tot, H, .] (fp32 or bf16 bits).  Returns a dict of fp64 o [T_tot,H,d]
    and final_states [S,H,c,d]."""
    lib = lib or load()
    dt, q = _raw(q)
    arrs = [_raw(a) for a in (key_logits, v, log_alpha)]
    if any(a[0] != dt for a in arrs):
        raise TypeError("all inputs must share one dtype")
    kl, v, la = (a[1] for a in arrs)
    T, H, c = q.shape
    d = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    assert kl.shape == (T, H, c) and la.shape == (T, H, c) and int(cu[-1]) == T
    init = None
    if initial_states is not None:
        init = np.ascontiguousarray(initial_states, dtype=np.float64)
        assert init.shape == (S, H, c, d)
    o = np.empty((T, H, d), np.float64)
    fs = np.empty((S, H, c, d), np.float64)
    rc = lib.sse_oracle_rowsparse_forward(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(cu), S,
                                          H, c, d, int(row_topk), int(bool(identity_unselected)),
                                          _ptr(init), _ptr(o), _ptr(fs))
    if rc != 0:
        raise ValueError("sse_oracle_rowsparse_forward rejected its arguments")
    return {"o": o, "final_states": fs}


def forward_ex(q, key_logits, v, log_alpha, router_logits, cu_seqlens, N, topk, q_shared=None,
               key_logits_shared=None, read_router_logits=None, read_topk=None,
               initial_states=None, lib=None):
    """General forward: optional own q / key logits of the shared partition
    and optional read-set router logits (read_topk partitions read).  Returns
    a dict of fp64 o [T,H,d], final_states [S,H,N+1,c,d], int32 write_idx
    [T,H,topk] and read_idx [T,H,read_topk or topk]."""
    lib = lib or load()
    dt, q = _raw(q)
    req = [_raw(a) for a in (key_logits, v, log_alpha, router_logits)]
    opt = [None if a is None else _raw(a) for a in (q_shared, key_logits_shared,
                                                     read_router_logits)]
    if any(a[0] != dt for a in req) or any(a is not None and a[0] != dt for a in opt):
        raise TypeError("all inputs must share one dtype")
    kl, v, la, z = (a[1] for a in req)
    qs, ks, zr = (None if a is None else a[1] for a in opt)
    T, H, c = q.shape
    d = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    assert z.shape == (T, H, N) and int(cu[-1]) == T
    for a, shp in ((qs, (T, H, c)), (ks, (T, H, c)), (zr, (T, H, N))):
        assert a is None or a.shape == shp
    kr = int(read_topk) if zr is not None else int(topk)
    init = None
    if initial_states is not None:
        init = np.ascontiguousarray(initial_states, dtype=np.float64)
        assert init.shape == (S, H, N + 1, c, d)
    o = np.empty((T, H, d), np.float64)
    fs = np.empty((S, H, N + 1, c, d), np.float64)
    widx = np.empty((T, H, topk), np.int32)
    ridx = np.empty((T, H, kr), np.int32)
    rc = lib.sse_oracle_forward_ex(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(z), _ptr(qs),
                                   _ptr(ks), _ptr(zr), kr, _ptr(cu), S, H, c, d, N, topk,
                                   _ptr(init), _ptr(o), _ptr(fs), _ptr(widx), _ptr(ridx))
    if rc != 0:
        raise ValueError("sse_oracle_forward_ex rejected its arguments")
    return {"o": o, "final_states": fs, "write_idx": widx, "read_idx": ridx}


def backward(q, key_logits, v, log_alpha, router_logits, cu_seqlens, N, topk, do,
             dfinal_states=None, initial_states=None, threads=1, lib=None):
    """Gradients of L = <do, o> + <dfinal_states, final_states> with respect
    to the five inputs and the initial states (fp64).  Returns a dict of dq,
    dkey_logits, dlog_alpha [T,H,c], dv [T,H,d], drouter_logits [T,H,N] and
    dinitial_states [S,H,N+1,c,d]."""
    lib = lib or load()
    dt, q = _raw(q)
    arrs = [_raw(a) for a in (key_logits, v, log_alpha, router_logits)]
    if any(a[0] != dt for a in arrs):
        raise TypeError("all inputs must share one dtype")
    kl, v, la, z = (a[1] for a in arrs)
    T, H, c = q.shape
    d = v.shape[2]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    assert z.shape == (T, H, N) and int(cu[-1]) == T
    do = np.ascontiguousarray(do, dtype=np.float64)
    assert do.shape == (T, H, d)
    init = None if initial_states is None else np.ascontiguousarray(initial_states, np.float64)
    dfin = None if dfinal_states is None else np.ascontiguousarray(dfinal_states, np.float64)
    for a in (init, dfin):
        assert a is None or a.shape == (S, H, N + 1, c, d)
    out = {"dq": np.empty((T, H, c)), "dkey_logits": np.empty((T, H, c)),
           "dv": np.empty((T, H, d)), "dlog_alpha": np.empty((T, H, c)),
           "drouter_logits": np.empty((T, H, N)),
           "dinitial_states": np.empty((S, H, N + 1, c, d))}
    rc = lib.sse_oracle_backward(dt, _ptr(q), _ptr(kl), _ptr(v), _ptr(la), _ptr(z), _ptr(cu), S,
                                 H, c, d, N, topk, _ptr(init), _ptr(do), _ptr(dfin),
                                 _ptr(out["dq"]), _ptr(out["dkey_logits"]), _ptr(out["dv"]),
                                 _ptr(out["dlog_alpha"]), _ptr(out["drouter_logits"]),
                                 _ptr(out["dinitial_states"]), int(threads))
    if rc != 0:
        raise ValueError("sse_oracle_backward rejected its arguments")
    return out
