"""Stage tracing (sse_trace_enable / sse_trace_read) on the GPU: it counts the
forwards it recorded, its stage times are non-negative and fit inside the
wall-clock time of those calls, a read starts a fresh record, a disabled
trace records nothing, and a traced forward gives the same bits as an
untraced one."""
import time

import pytest
import torch

import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, announce, to_dev

pytestmark = pytest.mark.gpu


def test_trace_counts_calls_and_keeps_results():
    w = si.Workload("trace", "bf16", H=4, c=128, d=128, N=16, topk=2)
    lengths = [1500, 300]
    inp = si.forward_inputs(w, lengths=lengths, seed=821)
    d = {n: to_dev(inp[n]) for n in NAMES}
    cu = to_dev(inp["cu_seqlens"])
    ml = max(lengths)
    announce("trace", w.name, lengths, "sse_forward x5, sse_trace_*")
    o0, f0 = sse.sse_forward(*(d[n] for n in NAMES), w.N, w.topk, cu, ml)
    torch.cuda.synchronize()
    sse.sse_trace_enable(True)
    try:
        t0 = time.perf_counter()
        for _ in range(3):
            o1, f1 = sse.sse_forward(*(d[n] for n in NAMES), w.N, w.topk, cu, ml)
        torch.cuda.synchronize()
        wall_ms = 1e3 * (time.perf_counter() - t0)
        stages, calls = sse.sse_trace_read()
        print("  stages (ms over 3 calls):", {k: round(v, 4) for k, v in stages.items()},
              f"wall {wall_ms:.3f} ms", flush=True)
        assert calls == 3
        assert all(v >= 0.0 for v in stages.values()), stages
        assert stages["routed"] > 0.0 and stages["shared"] > 0.0, stages
        assert sum(stages.values()) <= wall_ms * 1.05 + 0.05, (stages, wall_ms)
        assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
        assert torch.equal(f0.view(torch.int32), f1.view(torch.int32))
        # a read starts a fresh record
        stages2, calls2 = sse.sse_trace_read()
        assert calls2 == 0 and all(v == 0.0 for v in stages2.values())
        # nothing is recorded while tracing is off
        sse.sse_trace_enable(False)
        sse.sse_forward(*(d[n] for n in NAMES), w.N, w.topk, cu, ml)
        torch.cuda.synchronize()
        _, calls3 = sse.sse_trace_read()
        assert calls3 == 0
    finally:
        sse.sse_trace_enable(False)
