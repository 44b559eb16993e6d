"""sse_forward_noalloc (workspace in the library's static device array)
against sse_forward (caller workspace), through the C ABI.

Two calls in a row, the second on a smaller input, then the same two inputs
through sse_forward: outputs, final states and top-k choices must be the
same bits (same kernels, same order of operations) and within the oracle's
bar; sizes beyond the array are rejected with SSE_ERR_WORKSPACE."""
import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, TOL, announce, nan_like, oracle_threads, rel_err, sentinel_int, to_dev

pytestmark = pytest.mark.gpu


def _outputs(T, S, w):
    return (nan_like((T, w.H, w.d)), nan_like((S, w.H, w.N + 1, w.c, w.d)),
            sentinel_int((T, w.H, w.topk)))


def _call(inp, w, noalloc, init=None):
    d = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max())
    o, fs, idx = _outputs(T, S, w)
    init_d = None if init is None else torch.from_numpy(init).cuda()
    args = [d[n] for n in NAMES]
    if noalloc:
        sse.sse_forward_noalloc(*args, w.N, w.topk, d["cu_seqlens"], max_len, o, fs, init_d,
                                topk_idx=idx)
    else:
        sse.sse_forward(*args, w.N, w.topk, d["cu_seqlens"], max_len, init_d, o=o,
                        final_states=fs, topk_idx=idx)
    return o, fs, idx


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_forward_two_calls(dtype):
    wa = si.Workload(f"noalloc_a_{dtype}", dtype, H=4, c=128, d=128, N=16, topk=2, router_std=1.5)
    wb = si.Workload(f"noalloc_b_{dtype}", dtype, H=2, c=64, d=64, N=8, topk=3)
    inp_a = si.forward_inputs(wa, lengths=[1500, 700, 1], seed=91)
    inp_b = si.forward_inputs(wb, lengths=[300, 41], seed=92)
    rng = np.random.default_rng(93)
    init_b = (0.5 * rng.standard_normal((2, wb.H, wb.N + 1, wb.c, wb.d))).astype(np.float32)
    need_a = sse.sse_forward_workspace_bytes(2201, 3, 1500, wa.H, wa.c, wa.d, wa.N, wa.topk)
    assert 0 < need_a <= sse.sse_forward_noalloc_max_bytes()
    announce("noalloc", dtype, "sse_forward_noalloc x2 then sse_forward x2")
    got_a = _call(inp_a, wa, True)
    got_b = _call(inp_b, wb, True, init_b)          # second call, smaller input
    torch.cuda.synchronize()
    ref_a = _call(inp_a, wa, False)
    ref_b = _call(inp_b, wb, False, init_b)
    torch.cuda.synchronize()
    for got, ref in ((got_a, ref_a), (got_b, ref_b)):
        for g, r in zip(got, ref):
            assert torch.equal(g.view(torch.uint8), r.view(torch.uint8))
    for w, inp, init, got in ((wa, inp_a, None, got_a), (wb, inp_b, init_b, got_b)):
        orc = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                             initial_states=None if init is None else init.astype(np.float64),
                             threads=oracle_threads())
        assert np.array_equal(got[2].cpu().numpy(), orc["topk_idx"])
        assert rel_err(got[0].cpu().numpy(), orc["o"]) <= TOL[dtype]
        assert rel_err(got[1].cpu().numpy(), orc["final_states"]) <= TOL[dtype]


def test_noalloc_rejects_oversized_workspace():
    w = si.Workload("noalloc_big", "bf16", H=16, c=128, d=128, N=16, topk=2)
    T, S, L = 65536, 8, 8192
    assert sse.sse_forward_workspace_bytes(T, S, L, w.H, w.c, w.d, w.N, w.topk) > \
        sse.sse_forward_noalloc_max_bytes()
    dummy = torch.zeros((T, w.H, w.c), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((T, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros((T, w.H, w.N), dtype=torch.bfloat16, device="cuda")
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    o = torch.empty((T, w.H, w.d), dtype=torch.float32, device="cuda")
    fs = torch.empty((S, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    with pytest.raises(sse.SSEError) as e:
        sse.sse_forward_noalloc(dummy, dummy, v, dummy, z, w.N, w.topk, cu, L, o, fs)
    assert e.value.status == sse.SSE_ERR_WORKSPACE
