"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sse.h, and rejects bad arguments on the host before any
launch (every call below returns before its first HIP call)."""
import ctypes
import os
import re

import pytest

import sparse_state_linear_amd as sse

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sse_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sse.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"libsse_amd.so does not export {n}"
    assert set(names) == set(sse.EXPORTED)


def test_status_strings_and_version():
    for code in range(5):
        assert sse.status_string(code).startswith("SSE_")
    assert sse.status_string(99) == "SSE_ERR_UNKNOWN"
    assert sse.lib().sse_version() >= 100


def test_workspace_queries():
    ws = sse.sse_forward_workspace_bytes(32768, 4, 8192, 16, 128, 128, 16, 2)
    assert ws >= 4 * 32768 * 16 * 2 * 4 and ws % 256 == 0
    assert sse.sse_forward_workspace_bytes(100, 1, 100, 1, 48, 32, 4, 1) == 0   # c unsupported
    assert sse.sse_forward_workspace_bytes(100, 1, 100, 1, 32, 32, 4, 5) == 0   # topk > N
    assert sse.sse_forward_workspace_bytes(-1, 1, 100, 1, 32, 32, 4, 1) == 0
    assert sse.sse_group_workspace_bytes(100, 1, 100, 2, 4, 1) > 0
    assert sse.sse_group_workspace_bytes(100, 1, 100, 2, 65, 1) == 0


P = ctypes.c_void_p
FAKE = P(0x1000)  # never dereferenced: every call below fails validation first


def fwd(**kw):
    a = dict(q=FAKE, kl=FAKE, v=FAKE, la=FAKE, z=FAKE, dtype=sse.SSE_BF16, cu=FAKE, S=1,
             maxlen=16, T=16, H=2, c=32, d=32, N=4, k=2, init=None, o=FAKE, fs=FAKE, idx=None,
             w=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return sse.lib().sse_forward(a["q"], a["kl"], a["v"], a["la"], a["z"], a["dtype"], a["cu"],
                                 a["S"], a["maxlen"], a["T"], a["H"], a["c"], a["d"], a["N"],
                                 a["k"], a["init"], a["o"], a["fs"], a["idx"], a["w"], a["ws"],
                                 a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), sse.SSE_ERR_INVALID_ARG),
    (dict(o=None), sse.SSE_ERR_INVALID_ARG),
    (dict(fs=None), sse.SSE_ERR_INVALID_ARG),
    (dict(cu=None), sse.SSE_ERR_INVALID_ARG),
    (dict(dtype=7), sse.SSE_ERR_INVALID_ARG),
    (dict(k=5), sse.SSE_ERR_INVALID_ARG),
    (dict(k=0), sse.SSE_ERR_INVALID_ARG),
    (dict(H=0), sse.SSE_ERR_INVALID_ARG),
    (dict(T=-1), sse.SSE_ERR_INVALID_ARG),
    (dict(S=0), sse.SSE_ERR_INVALID_ARG),
    (dict(c=48), sse.SSE_ERR_UNSUPPORTED),
    (dict(d=256), sse.SSE_ERR_UNSUPPORTED),
    (dict(N=65, k=1), sse.SSE_ERR_UNSUPPORTED),
    (dict(N=16, k=9), sse.SSE_ERR_UNSUPPORTED),
    (dict(wsb=16), sse.SSE_ERR_WORKSPACE),
    (dict(ws=None), sse.SSE_ERR_WORKSPACE),
])
def test_forward_rejects(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(states=None), sse.SSE_ERR_INVALID_ARG),
    (dict(B=-1), sse.SSE_ERR_INVALID_ARG),
    (dict(c=16), sse.SSE_ERR_UNSUPPORTED),
    (dict(k=3, N=2), sse.SSE_ERR_INVALID_ARG),
])
def test_decode_rejects(kw, code):
    a = dict(B=4, H=2, c=32, d=32, N=4, k=2, states=FAKE)
    a.update(kw)
    st = sse.lib().sse_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, sse.SSE_F32, a["B"], a["H"],
                                   a["c"], a["d"], a["N"], a["k"], a["states"], FAKE, None, None)
    assert st == code


def test_router_and_group_reject():
    L = sse.lib()
    assert L.sse_router_topk(FAKE, 0, 10, 4, 5, FAKE, FAKE, None) == sse.SSE_ERR_INVALID_ARG
    assert L.sse_router_topk(None, 0, 10, 4, 2, FAKE, FAKE, None) == sse.SSE_ERR_INVALID_ARG
    assert L.sse_router_topk(FAKE, 0, 10, 80, 2, FAKE, FAKE, None) == sse.SSE_ERR_UNSUPPORTED
    assert L.sse_group_by_partition(FAKE, None, FAKE, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, None,
                                    FAKE, 0, None) == sse.SSE_ERR_WORKSPACE
    assert L.sse_group_by_partition(FAKE, None, FAKE, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, FAKE,
                                    FAKE, 1 << 20, None) == sse.SSE_ERR_INVALID_ARG
    assert L.sse_group_by_partition(FAKE, None, None, 1, 16, 16, 2, 4, 2, FAKE, FAKE, None, None,
                                    FAKE, 1 << 20, None) == sse.SSE_ERR_INVALID_ARG


def test_product_path_does_not_touch_the_oracle():
    """The HIP binding must not import, load or call the oracle."""
    pkg = os.path.join(ROOT, "sparse_state_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"
