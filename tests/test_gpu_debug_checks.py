"""Debug mode on the GPU: the host checks of cu_seqlens reject a bad array
before any launch, and a valid call gives the same bits as without debug
mode.

The invalid arrays are only passed while the test has confirmed that debug
mode is on, and the first one is harmless even if it were launched (its
last entry is below total_tokens, so the kernels would just skip the
tail): if the check did not work, that case fails first and the riskier
ones (a negative length, a length above max_seqlen) never run.
"""
import pytest
import torch

import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, announce, nan_like, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seed=431):
    w = si.Workload("dbg", "bf16", H=2, c=64, d=64, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[300, 71], seed=seed)
    return w, inp, {n: to_dev(inp[n]) for n in NAMES}


@pytest.fixture
def debug_mode():
    before = sse.sse_debug_checks()
    assert sse.sse_debug_checks(True) is True
    try:
        yield
    finally:
        sse.sse_debug_checks(before)


def _forward(w, d, cu, max_seqlen):
    T = d["q"].shape[0]
    S = cu.shape[0] - 1
    o = nan_like((T, w.H, w.d))
    fs = nan_like((S, w.H, w.N + 1, w.c, w.d))
    sse.sse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"], w.N,
                    w.topk, cu, max_seqlen, o=o, final_states=fs)
    torch.cuda.synchronize()
    return o, fs


def _rejects(fn):
    with pytest.raises(sse.SSEError) as exc:
        fn()
    assert exc.value.status == sse.SSE_ERR_INVALID_ARG


def test_debug_mode_same_bits(debug_mode):
    w, inp, d = _inputs()
    cu = to_dev(inp["cu_seqlens"])
    announce("debug mode: valid forward, both modes", w.name)
    o1, f1 = _forward(w, d, cu, 300)
    sse.sse_debug_checks(False)
    o0, f0 = _forward(w, d, cu, 300)
    sse.sse_debug_checks(True)
    assert torch.equal(o1, o0) and torch.equal(f1, f0)
    assert not torch.isnan(o1).any()


def test_debug_mode_rejects_bad_cu_seqlens(debug_mode):
    w, inp, d = _inputs()
    T = d["q"].shape[0]
    assert T == 371
    o_probe = nan_like((T, w.H, w.d))

    def fwd(cu_list, max_seqlen):
        cu = torch.tensor(cu_list, dtype=torch.int32, device="cuda")
        S = len(cu_list) - 1
        fs = nan_like((S, w.H, w.N + 1, w.c, w.d))
        sse.sse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"],
                        w.N, w.topk, cu, max_seqlen, o=o_probe, final_states=fs)

    # harmless if launched: ends before total_tokens
    announce("debug mode: cu_seqlens ends early")
    assert sse.sse_debug_checks() is True
    _rejects(lambda: fwd([0, 300, 360], 300))
    torch.cuda.synchronize()
    assert torch.isnan(o_probe).all(), "a rejected call wrote its output"
    announce("debug mode: cu_seqlens does not start at 0")
    _rejects(lambda: fwd([5, 300, 371], 300))
    announce("debug mode: cu_seqlens decreases")
    _rejects(lambda: fwd([0, 300, 200, 371], 300))
    announce("debug mode: a sequence longer than max_seqlen")
    _rejects(lambda: fwd([0, 300, 371], 299))
    torch.cuda.synchronize()
    assert torch.isnan(o_probe).all(), "a rejected call wrote its output"

    bad = torch.tensor([0, 300, 200, 371], dtype=torch.int32, device="cuda")
    announce("debug mode: backward with a decreasing cu_seqlens")
    d_o = torch.ones((T, w.H, w.d), dtype=torch.float32, device="cuda")
    _rejects(lambda: sse.sse_backward(d["q"], d["key_logits"], d["v"], d["log_alpha"],
                                      d["router_logits"], w.N, w.topk, bad, d_o, max_seqlen=300))
    announce("debug mode: row-sparse forward with a decreasing cu_seqlens")
    _rejects(lambda: sse.sse_rowsparse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"],
                                               8, bad, max_seqlen=300))
    announce("debug mode: grouping with a decreasing cu_seqlens")
    idx = torch.zeros((T, w.H, w.topk), dtype=torch.int32, device="cuda")
    idx[..., 1] = 1
    _rejects(lambda: sse.sse_group_by_partition(idx, None, bad, w.N, max_seqlen=300))
    torch.cuda.synchronize()
