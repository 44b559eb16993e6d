"""Host-side calls of the C ABI that its argument checks must reject (or that
have nothing to do), with the status each must return.  No call here reaches
a device: every one returns before its first HIP call.  Used by the plain
host ABI test and by the sanitizer build of the ABI layer; it needs only
ctypes (no torch)."""
from __future__ import annotations

import ctypes

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
F32, BF16 = 0, 1
P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
FAKE = P(0x1000)   # never dereferenced: the checks reject the call first


def declare(L):
    L.sse_status_string.argtypes = [I]
    L.sse_status_string.restype = ctypes.c_char_p
    L.sse_forward_workspace_bytes.argtypes = [I64, I, I, I, I, I, I, I]
    L.sse_forward_workspace_bytes.restype = SZ
    L.sse_forward.argtypes = [P, P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P, P, P,
                              P, P, P, SZ, P]
    L.sse_forward.restype = I
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
    L.sse_rowsparse_workspace_bytes.argtypes = [I64, I, I, I, I, I]
    L.sse_rowsparse_workspace_bytes.restype = SZ
    L.sse_rowsparse_forward.argtypes = [P, P, P, P, I, P, I, I, I64, I, I, I, I, I, P, P, P, P,
                                        SZ, P]
    L.sse_rowsparse_forward.restype = I
    L.sse_trace_read.argtypes = [P, I, P]
    L.sse_trace_read.restype = I


def forward(L, **kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, z=FAKE, dtype=BF16, cu=FAKE, S=1, maxlen=16,
             T=16, H=2, c=32, d=32, N=4, k=2, init=None, o=FAKE, fs=FAKE, idx=None, w=None,
             soff=None, stok=None, sslot=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.sse_forward(a["q"], a["kl"], a["v"], a["la"], a["z"], a["dtype"], a["cu"], a["S"],
                         a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["N"], a["k"], a["init"],
                         a["o"], a["fs"], a["idx"], a["w"], a["soff"], a["stok"], a["sslot"],
                         a["ws"], a["wsb"], a["stream"])


FORWARD_REJECTS = [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(fs=None), INVALID),
    (dict(cu=None), INVALID), (dict(dtype=7), INVALID), (dict(k=5), INVALID),
    (dict(k=0), INVALID), (dict(H=0), INVALID), (dict(T=-1), INVALID), (dict(S=0), INVALID),
    (dict(S=-1), INVALID), (dict(maxlen=-1), INVALID),
    (dict(c=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(N=65, k=1), UNSUPPORTED),
    (dict(N=16, k=9), UNSUPPORTED), (dict(H=257), UNSUPPORTED),
    # 32-bit offsets of token rows and slots
    (dict(T=1 << 26, S=1, maxlen=1 << 26, H=16, c=128, d=128), UNSUPPORTED),
    (dict(T=1 << 40, S=1, maxlen=1 << 30), UNSUPPORTED),
    (dict(wsb=16), WORKSPACE), (dict(ws=None), WORKSPACE),
]


def forward_noalloc(L, **kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, z=FAKE, dtype=BF16, cu=FAKE, S=1, maxlen=16,
             T=16, H=2, c=32, d=32, N=4, k=2, init=None, o=FAKE, fs=FAKE, idx=None, w=None,
             stream=None)
    a.update(kw)
    return L.sse_forward_noalloc(a["q"], a["kl"], a["v"], a["la"], a["z"], a["dtype"], a["cu"],
                                 a["S"], a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["N"],
                                 a["k"], a["init"], a["o"], a["fs"], a["idx"], a["w"],
                                 a["stream"])


NOALLOC_REJECTS = [
    (dict(q=None), INVALID), (dict(fs=None), INVALID), (dict(k=5), INVALID),
    (dict(c=48), UNSUPPORTED),
    # workspace beyond the static array: 8 sequences x 16 heads x 8192 tokens
    (dict(T=65536, S=8, maxlen=8192, H=16, c=128, d=128, N=16), WORKSPACE),
]

def forward_ex(L, **kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, z=FAKE, dtype=BF16, cu=FAKE, S=1, maxlen=16,
             T=16, H=2, c=32, d=32, N=4, k=2, qs=None, ks=None, zr=None, kr=0, sched=0,
             init=None, o=FAKE, fs=FAKE, idx=None, w=None, ridx=None, soff=None, stok=None,
             sslot=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.sse_forward_ex(a["q"], a["kl"], a["v"], a["la"], a["z"], a["dtype"], a["cu"],
                            a["S"], a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["N"], a["k"],
                            a["qs"], a["ks"], a["zr"], a["kr"], a["sched"], a["init"], a["o"],
                            a["fs"], a["idx"], a["w"], a["ridx"], a["soff"], a["stok"],
                            a["sslot"], a["ws"], a["wsb"], a["stream"])


FORWARD_EX_REJECTS = [
    (dict(q=None), INVALID), (dict(sched=2), INVALID),
    (dict(zr=FAKE, kr=0, sched=1), INVALID), (dict(zr=FAKE, kr=5, sched=1), INVALID),
    (dict(zr=FAKE, kr=2, sched=0), UNSUPPORTED),            # read sets need the masked schedule
    (dict(N=16, zr=FAKE, kr=9, sched=1), UNSUPPORTED),
    (dict(ridx=FAKE), INVALID),                             # read choices without read logits
    (dict(sched=1, soff=FAKE), INVALID),                    # no grouping on the masked schedule
    (dict(sched=1, wsb=16), WORKSPACE),
]


def backward(L, **kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, z=FAKE, dtype=BF16, cu=FAKE, S=1, maxlen=16,
             T=16, H=2, c=32, d=32, N=4, k=2, init=None, do=FAKE, dfin=None, dq=FAKE, dkl=FAKE,
             dv=FAKE, dla=FAKE, dz=FAKE, dinit=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.sse_backward(a["q"], a["kl"], a["v"], a["la"], a["z"], a["dtype"], a["cu"], a["S"],
                          a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["N"], a["k"], a["init"],
                          a["do"], a["dfin"], a["dq"], a["dkl"], a["dv"], a["dla"], a["dz"],
                          a["dinit"], a["ws"], a["wsb"], a["stream"])


BACKWARD_REJECTS = [
    (dict(q=None), INVALID), (dict(do=None), INVALID), (dict(dz=None), INVALID),
    (dict(dla=None), INVALID), (dict(k=5), INVALID), (dict(S=0), INVALID),
    (dict(c=48), UNSUPPORTED), (dict(wsb=64), WORKSPACE), (dict(ws=None), WORKSPACE),
    (dict(T=1 << 25, S=1, maxlen=1 << 25, H=16, c=128, d=128), UNSUPPORTED),
]


def rowsparse(L, **kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, dtype=BF16, cu=FAKE, S=1, maxlen=16, T=16, H=2,
             c=32, d=32, k=8, ident=1, init=None, o=FAKE, fs=FAKE, ws=FAKE, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return L.sse_rowsparse_forward(a["q"], a["kl"], a["v"], a["la"], a["dtype"], a["cu"], a["S"],
                                   a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["k"],
                                   a["ident"], a["init"], a["o"], a["fs"], a["ws"], a["wsb"],
                                   a["stream"])


ROWSPARSE_REJECTS = [
    (dict(q=None), INVALID), (dict(la=None), INVALID), (dict(fs=None), INVALID),
    (dict(k=0), INVALID), (dict(k=33), INVALID), (dict(dtype=3), INVALID), (dict(S=0), INVALID),
    (dict(c=48), UNSUPPORTED), (dict(H=300), UNSUPPORTED), (dict(wsb=8), WORKSPACE),
    (dict(T=1 << 26, S=1, maxlen=1 << 26, H=16, c=128, d=128), UNSUPPORTED),
]

DECODE_REJECTS = [
    (dict(states=None), INVALID), (dict(B=-1), INVALID), (dict(c=16), UNSUPPORTED),
    (dict(k=3, N=2), INVALID), (dict(B=1 << 30, H=256), UNSUPPORTED),
]


def decode(L, **kw):
    a = dict(B=4, H=2, c=32, d=32, N=4, k=2, states=FAKE, dtype=F32)
    a.update(kw)
    return L.sse_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, a["dtype"], a["B"], a["H"], a["c"],
                             a["d"], a["N"], a["k"], a["states"], FAKE, None, None)


DECODE_EX_REJECTS = DECODE_REJECTS + [
    (dict(zr=FAKE, kr=0), INVALID), (dict(zr=FAKE, kr=5), INVALID),
    (dict(zr=FAKE, kr=9, N=12), UNSUPPORTED), (dict(ridx=FAKE), INVALID),
]


def decode_ex(L, **kw):
    a = dict(B=4, H=2, c=32, d=32, N=4, k=2, states=FAKE, dtype=F32, zr=None, kr=0, ridx=None)
    a.update(kw)
    return L.sse_decode_step_ex(FAKE, FAKE, FAKE, FAKE, FAKE, a["dtype"], a["B"], a["H"], a["c"],
                                a["d"], a["N"], a["k"], None, None, a["zr"], a["kr"],
                                a["states"], FAKE, None, a["ridx"], None)


def exercise(L) -> int:
    """Run every rejection case; raise AssertionError on a wrong status.
    Returns the number of calls made."""
    declare(L)
    n = 0
    for code in range(6):
        assert L.sse_status_string(code).startswith(b"SSE_")
        n += 1
    for kw, code in FORWARD_REJECTS:
        got = forward(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    assert L.sse_forward_noalloc_max_bytes() == 64 << 20
    for kw, code in NOALLOC_REJECTS:
        got = forward_noalloc(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    for kw, code in DECODE_REJECTS:
        got = decode(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    for kw, code in DECODE_EX_REJECTS:
        got = decode_ex(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    for kw, code in FORWARD_EX_REJECTS:
        got = forward_ex(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    # read sets of 3 take 3 slot rows per token instead of 2 (64 heads: the
    # varlen layout reserves no routed piece states)
    assert L.sse_forward_ex_workspace_bytes(1000, 2, 600, 64, 64, 64, 8, 2, 3) > \
        L.sse_forward_ex_workspace_bytes(1000, 2, 600, 64, 64, 64, 8, 2, 0) > 0
    assert L.sse_forward_ex_workspace_bytes(1000, 2, 600, 4, 64, 64, 8, 2, 9) == 0
    for kw, code in BACKWARD_REJECTS:
        got = backward(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    assert L.sse_backward_workspace_bytes(1000, 2, 600, 4, 64, 64, 8, 2) > 0
    assert L.sse_backward_workspace_bytes(1000, 2, 600, 4, 48, 64, 8, 2) == 0
    for kw, code in ROWSPARSE_REJECTS:
        got = rowsparse(L, **kw)
        assert got == code, (kw, got, code)
        n += 1
    # workspace queries, including sizes that overflow the kernels' indexing
    assert L.sse_forward_workspace_bytes(32768, 4, 8192, 16, 128, 128, 16, 2) > 0
    assert L.sse_forward_workspace_bytes(1 << 40, 4, 1 << 30, 16, 128, 128, 16, 2) == 0
    assert L.sse_forward_workspace_bytes(100, 1, 100, 1, 48, 32, 4, 1) == 0
    assert L.sse_forward_workspace_bytes(-1, 1, 100, 1, 32, 32, 4, 1) == 0
    assert L.sse_forward_workspace_bytes(100, -3, 100, 1, 32, 32, 4, 1) == 0
    assert L.sse_forward_workspace_bytes(0, 0, 0, 1, 32, 32, 4, 1) > 0
    assert L.sse_group_workspace_bytes(100, 1, 100, 2, 4, 1) > 0
    assert L.sse_group_workspace_bytes(100, 1, 100, 2, 65, 1) == 0
    assert L.sse_group_workspace_bytes(1 << 40, 1, 1 << 30, 2, 4, 1) == 0
    n += 9
    assert L.sse_router_topk(FAKE, 0, 10, 4, 5, FAKE, FAKE, None) == INVALID
    assert L.sse_router_topk(None, 0, 10, 4, 2, FAKE, FAKE, None) == INVALID
    assert L.sse_router_topk(FAKE, 0, 10, 80, 2, FAKE, FAKE, None) == UNSUPPORTED
    assert L.sse_router_topk(FAKE, 0, -1, 4, 2, FAKE, FAKE, None) == INVALID
    assert L.sse_group_by_partition(FAKE, None, FAKE, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, None,
                                    FAKE, 0, None) == WORKSPACE
    assert L.sse_group_by_partition(FAKE, None, FAKE, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, FAKE,
                                    FAKE, 1 << 20, None) == INVALID
    assert L.sse_group_by_partition(FAKE, None, None, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, None,
                                    FAKE, 1 << 20, None) == INVALID
    n += 7
    ms = (ctypes.c_float * 5)()
    calls = ctypes.c_int64(0)
    assert L.sse_trace_read(None, 5, ctypes.byref(calls)) == INVALID
    assert L.sse_trace_read(ms, 9, ctypes.byref(calls)) == INVALID
    n += 2
    return n
