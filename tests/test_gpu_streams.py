"""Calls on a side stream.  Every entry point takes a stream and launches
all of its work there (the binding passes torch's current stream), so work
queued on that stream before the call is finished before the call's kernels
read their inputs.  Each test fills fresh input buffers with NaN on a side
stream, queues about 10 ms of matrix products there, then the copy of the
real inputs, then the call; a kernel on any other stream would read the
NaNs.  The results must equal those of the same call on the default stream,
bit for bit.

Only value inputs are held back this way (q, key logits, v, log decay, the
output gradient, decode states): cu_seqlens and the router logits, which
decide indices, are ready before the side stream starts, so even a
misplaced launch would only compute with NaN values."""
import numpy as np
import pytest
import torch

import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, announce, to_dev

pytestmark = pytest.mark.gpu

DELAYED = ("q", "key_logits", "v", "log_alpha")


def _delayed(src: dict, s: torch.cuda.Stream) -> dict:
    """On stream s: NaN-filled copies of the tensors in src, written with
    their values only after ~10 ms of other work on s."""
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dst = {k: torch.full_like(v, float("nan")) for k, v in src.items()}
        m = torch.randn((2048, 2048), device="cuda") / 45.25
        x = m
        for _ in range(40):
            x = x @ m
        for k in dst:
            dst[k].copy_(src[k])
    return dst


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and bool(
        torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)))


def _fwd_case():
    w = si.Workload("stream_fwd", "bf16", H=2, c=64, d=64, N=8, topk=2)
    lengths = [300, 77, 129]
    inp = si.forward_inputs(w, lengths=lengths, seed=811)
    d = {n: to_dev(inp[n]) for n in NAMES}
    cu = to_dev(inp["cu_seqlens"])
    return w, lengths, d, cu


def test_forward_on_side_stream():
    w, lengths, d, cu = _fwd_case()
    ml = max(lengths)
    announce("side stream", w.name, lengths, "sse_forward")
    o0, f0 = sse.sse_forward(*(d[n] for n in NAMES), w.N, w.topk, cu, ml)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    dd = _delayed({n: d[n] for n in DELAYED}, s)
    with torch.cuda.stream(s):
        args = [dd.get(n, d[n]) for n in NAMES]
        o1, f1 = sse.sse_forward(*args, w.N, w.topk, cu, ml)
    s.synchronize()
    assert not torch.isnan(o0).any()
    assert _bits_equal(o0, o1) and _bits_equal(f0, f1)


def test_backward_on_side_stream():
    w, lengths, d, cu = _fwd_case()
    ml = max(lengths)
    T = int(sum(lengths))
    g = torch.from_numpy(
        np.random.default_rng(812).standard_normal((T, w.H, w.d)).astype(np.float32)).cuda()
    announce("side stream", w.name, lengths, "sse_backward")
    r0 = sse.sse_backward(*(d[n] for n in NAMES), w.N, w.topk, cu, g, ml)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    src = {n: d[n] for n in DELAYED}
    src["d_o"] = g
    dd = _delayed(src, s)
    with torch.cuda.stream(s):
        args = [dd.get(n, d[n]) for n in NAMES]
        r1 = sse.sse_backward(*args, w.N, w.topk, cu, dd["d_o"], ml)
    s.synchronize()
    for k in r0:
        assert not torch.isnan(r0[k]).any(), k
        assert _bits_equal(r0[k], r1[k]), k


def test_decode_on_side_stream():
    w = si.Workload("stream_dec", "bf16", H=2, c=64, d=64, N=8, topk=2, B=4, seed=0)
    B, steps = 4, 3
    states = torch.from_numpy(np.stack([si.decode_states(w, b) for b in range(B)])).cuda()
    toks = si.decode_inputs(w, steps=steps, B=B, seed=813)
    d = {n: to_dev(toks[n]) for n in NAMES}
    announce("side stream", w.name, "B", B, "steps", steps, "sse_decode_step")
    st0 = states.clone()
    o0 = [sse.sse_decode_step(*(d[n][t] for n in NAMES), w.N, w.topk, st0) for t in range(steps)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    src = {n: d[n] for n in DELAYED}
    src["states"] = states
    dd = _delayed(src, s)
    with torch.cuda.stream(s):
        st1 = dd["states"]
        o1 = [sse.sse_decode_step(*(dd.get(n, d[n])[t] for n in NAMES), w.N, w.topk, st1)
              for t in range(steps)]
    s.synchronize()
    for t in range(steps):
        assert not torch.isnan(o0[t]).any()
        assert _bits_equal(o0[t], o1[t]), t
    assert _bits_equal(st0, st1)
