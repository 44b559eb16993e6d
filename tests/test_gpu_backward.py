"""GPU parity of the backward (sse_backward) against the fp64 oracle's
backward: every element of dq, dkey_logits, dv, dlog_alpha, drouter_logits
and dinitial_states.

Bars (max|err| / rms(ref), per tensor): 5e-3 for bf16 inputs (the bar of the
forward's bf16 outputs; some of their products run on bf16 MFMA with
two-term splits, about 2^-16 relative).  With fp32 inputs the backward
computes in fp32 throughout, so they get a bar derived from fp32 arithmetic
rather than the forward's 1e-5: unit roundoff u = 2^-24 = 6e-8; a gradient element sums
O(n) terms (n up to a segment's records, ~1e3 here), each carried through
up to n/16 chunk steps, so the rounding error grows like sqrt(n) u ~ 2e-6
of the largest term; the max/rms ratio of the tensors (~5) and the
cancellations in the softmax Jacobians (dkappa - kappa.dkappa) and in the
decay gradient (Qt.dQt - Kh.dKh) amplify it by up to ~20: 2e-4."""
import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, announce, nan_like, oracle_threads, rel_err, rel_err_big, to_dev

pytestmark = pytest.mark.gpu
BWD_TOL = {"bf16": 5e-3, "f32": 2e-4}
GRADS = ("dq", "dkey_logits", "dv", "dlog_alpha", "drouter_logits", "dinitial_states")


def _grad_inputs(w, lengths, seed, with_init=True, with_dfinal=True):
    rng = np.random.default_rng(seed + 900)
    T, S = int(sum(lengths)), len(lengths)
    do = rng.standard_normal((T, w.H, w.d)).astype(np.float32)
    dfin = rng.standard_normal((S, w.H, w.N + 1, w.c, w.d)).astype(np.float32) if with_dfinal else None
    init = (0.5 * rng.standard_normal((S, w.H, w.N + 1, w.c, w.d))).astype(np.float32) if with_init else None
    return do, dfin, init


def _run(inp, w, do, dfin, init):
    d = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max()) if S else 0
    out = {"dq": nan_like((T, w.H, w.c)), "dkey_logits": nan_like((T, w.H, w.c)),
           "dlog_alpha": nan_like((T, w.H, w.c)), "dv": nan_like((T, w.H, w.d)),
           "drouter_logits": nan_like((T, w.H, w.N)),
           "dinitial_states": nan_like((S, w.H, w.N + 1, w.c, w.d))}
    nbytes = sse.sse_backward_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk)
    ws = torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device="cuda")
    dev = lambda a: None if a is None else torch.from_numpy(a).cuda()
    sse.sse_backward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"], w.N,
                     w.topk, d["cu_seqlens"], dev(do), max_len, dev(init), dev(dfin),
                     want_dinitial=True, workspace=ws, out=out)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    del out, ws
    return res


def _check(w, lengths, seed, inp=None, with_init=True, with_dfinal=True, tag=None):
    if inp is None:
        inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    do, dfin, init = _grad_inputs(w, lengths, seed, with_init, with_dfinal)
    announce(tag or w.name, "lengths", lengths if len(lengths) < 12 else len(lengths), "N", w.N,
             "k", w.topk, "init", with_init, "dfinal", with_dfinal, "sse_backward")
    got = _run(inp, w, do, dfin, init)
    ref = oracle.backward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                          do.astype(np.float64),
                          dfinal_states=None if dfin is None else dfin.astype(np.float64),
                          initial_states=None if init is None else init.astype(np.float64),
                          threads=oracle_threads())
    errs = {}
    for name in GRADS:
        assert np.isfinite(got[name]).all(), f"{name} has unwritten or non-finite elements"
        errs[name] = rel_err(got[name], ref[name])
    print("  " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) +
          f"  (tol {BWD_TOL[w.dtype]})", flush=True)
    for name, e in errs.items():
        assert e <= BWD_TOL[w.dtype], (name, e)
    return got, ref


def test_backward_small_bf16():
    w = si.Workload("bwd_small_bf16", "bf16", H=2, c=64, d=64, N=8, topk=2)
    _check(w, [300, 77, 1, 0, 129], seed=701)


def test_backward_tiny_f32():
    w = si.WORKLOADS["tiny_f32"]
    _check(w, [w.T], seed=702)


@pytest.mark.parametrize("c,d", [(128, 128), (32, 64), (64, 128), (128, 32)])
def test_backward_shapes_bf16(c, d):
    w = si.Workload(f"bwd_bf16_{c}x{d}", "bf16", H=2, c=c, d=d, N=6, topk=2, router_std=1.5)
    _check(w, [200, 33, 64], seed=703 + c + d)


@pytest.mark.parametrize("c,d", [(32, 32), (64, 32), (128, 128)])
def test_backward_shapes_f32(c, d):
    w = si.Workload(f"bwd_f32_{c}x{d}", "f32", H=2, c=c, d=d, N=4, topk=2)
    _check(w, [150, 40, 17], seed=710 + c + d)


@pytest.mark.parametrize("dtype,N,k", [("bf16", 64, 8), ("bf16", 1, 1), ("bf16", 5, 5),
                                       ("f32", 16, 3)])
def test_backward_partition_extremes(dtype, N, k):
    w = si.Workload(f"bwd_{dtype}_n{N}k{k}", dtype, H=3, c=64, d=64, N=N, topk=k)
    _check(w, [250, 1, 70], seed=720 + N + k)


def test_backward_without_init_or_dfinal():
    w = si.Workload("bwd_plain", "bf16", H=2, c=128, d=128, N=16, topk=2, router_std=1.5)
    _check(w, [600, 90], seed=730, with_init=False, with_dfinal=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_gate_limit(dtype):
    """log_alpha = -1.24 on every row (strong decay near the documented
    limit)."""
    w = si.Workload(f"bwd_gate_{dtype}", dtype, H=2, c=64, d=64, N=4, topk=2)
    lengths = [400, 61]
    inp = si.forward_inputs(w, lengths=lengths, seed=740)
    la = np.full(inp["log_alpha"].shape, -1.24, np.float32)
    inp["log_alpha"] = si.f32_to_bf16_bits(la) if dtype == "bf16" else la
    _check(w, lengths, 740, inp=inp)


def test_backward_tied_router_logits():
    w = si.Workload("bwd_ties", "bf16", H=2, c=64, d=64, N=8, topk=3)
    lengths = [300, 20]
    inp = si.forward_inputs(w, lengths=lengths, seed=750)
    rng = np.random.default_rng(751)
    z = rng.integers(-2, 3, inp["router_logits"].shape).astype(np.float32)
    z[(z == 0) & (rng.random(z.shape) < 0.5)] = -0.0   # -0 ties with +0
    inp["router_logits"] = si.f32_to_bf16_bits(z)
    _check(w, lengths, 750, inp=inp)


def test_backward_long_segments():
    """Sequences of 2-3 thousand tokens (shared chains of ~150 chunks)."""
    w = si.Workload("bwd_long", "bf16", H=2, c=64, d=64, N=4, topk=1)
    _check(w, [2500, 2049], seed=760)


def test_backward_run_twice_bitwise():
    w = si.Workload("bwd_twice", "bf16", H=4, c=128, d=128, N=16, topk=2)
    lengths = [700, 129]
    inp = si.forward_inputs(w, lengths=lengths, seed=770)
    do, dfin, init = _grad_inputs(w, lengths, 770)
    announce("backward run twice")
    a = _run(inp, w, do, dfin, init)
    b = _run(inp, w, do, dfin, init)
    for k in GRADS:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_backward_main_full_size():
    """The main workload (B=4, H=16, T=8192, c=d=128, N=16, k=2) in one
    backward call, every element of every gradient against the oracle (all
    64 (sequence, head) units, on the host threads)."""
    w = si.WORKLOADS["main_bf16"]
    inp = si.forward_inputs(w)
    lengths = [w.T] * w.B
    do, _, _ = _grad_inputs(w, lengths, 780, with_init=False, with_dfinal=False)
    announce("main_bf16 backward full size")
    got = _run(inp, w, do, None, None)
    announce("main_bf16 backward full size: oracle")
    ref = oracle.backward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                          do.astype(np.float64), threads=oracle_threads())
    for name in GRADS:
        e = rel_err_big(got[name], ref[name])
        print(f"  {name} rel err {e:.3e}", flush=True)
        assert e <= BWD_TOL["bf16"], (name, e)


@pytest.mark.parametrize("dtype,c,d", [("bf16", 64, 64), ("f32", 32, 32)])
def test_backward_many_slots(dtype, c, d):
    """N = 64, k = 8 over 2,200 tokens: about 1,500 chunk slots, far more
    than the chunk pass's resident blocks, many of them empty (the spare
    slot after each of the 256 routed segments), so every block walks
    several slots, prefetching the next one's records and rows, and skips
    empty ones on the way."""
    w = si.Workload(f"bwd_many_slots_{dtype}", dtype, H=2, c=c, d=d, N=64, topk=8)
    _check(w, [1500, 700], seed=790 + c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_all_sequences_empty(dtype):
    """Every sequence empty: no records, every chunk slot empty.  The
    initial-state gradient is d_final_states passed through unchanged (bit
    for bit, as the oracle gives), and the token gradients are empty."""
    w = si.Workload(f"bwd_empty_{dtype}", dtype, H=2, c=64, d=64, N=8, topk=2)
    lengths = [0, 0]
    inp = si.forward_inputs(w, lengths=lengths, seed=795)
    do, dfin, init = _grad_inputs(w, lengths, 795)
    announce(w.name, "lengths", lengths, "sse_backward")
    got = _run(inp, w, do, dfin, init)
    ref = oracle.backward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                          do.astype(np.float64), dfinal_states=dfin.astype(np.float64),
                          initial_states=init.astype(np.float64), threads=oracle_threads())
    for name in GRADS[:-1]:
        assert got[name].size == 0 and ref[name].size == 0, name
    assert np.array_equal(ref["dinitial_states"], dfin.astype(np.float64))
    assert np.array_equal(got["dinitial_states"].view(np.uint32), dfin.view(np.uint32))
