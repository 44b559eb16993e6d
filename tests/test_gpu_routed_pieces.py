"""GPU parity of the routed pass when long routed segments are split into
pieces (bf16 inputs, fewer (sequence, head, partition) segments than the
chip's 256 compute units): the gathered piece states, the scan of the piece
start states and the pieces of the routed pass, against the fp64 oracle on
every element of o and the final states (5e-3 of the reference rms).

The split rule (only with fewer than 256 segments holding 512 records or
more on average; records per piece P: the smallest power of two from 64 up,
capped at 2048, that gives at most 256 pieces in all and at most 16 per
segment; no split when no segment can exceed P) is restated here only to
make sure each case below does split."""
import numpy as np
import pytest

import sse_inputs as si
from gpu_util import TOL, announce
from test_gpu_parity import _compare, _oracle_forward, _run_forward

pytestmark = pytest.mark.gpu


def _piece_len(T, S, max_len, H, N, K):
    if S * H * N >= 256 or T * H * K < 512 * S * H * N:
        return 0
    p = 64
    while p < 2048 and (T * H * K // p > 256 or -(-max_len // p) > 16):
        p *= 2
    return p if max_len > p else 0


def _check(w, lengths, seed, init_scale=0.5, inp=None, expect_split=True):
    if inp is None:
        inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    T, S = int(sum(lengths)), len(lengths)
    P = _piece_len(T, S, max(lengths), w.H, w.N, w.topk)
    if expect_split:
        assert P > 0, "this case must split its routed segments"
    init = None
    if init_scale:
        rng = np.random.default_rng(seed + 5)
        init = (init_scale * rng.standard_normal((S, w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    announce(w.name, "lengths", lengths, "N", w.N, "k", w.topk, "piece", P, "sse_forward")
    got = _run_forward(inp, w, init)
    ref = _oracle_forward(inp, w, init)
    _compare(w, inp, got, ref)
    return got, ref


def test_routed_pieces_random():
    w = si.Workload("rpieces_rand", "bf16", H=2, c=128, d=128, N=4, topk=1)
    _check(w, [6000, 3400, 5], seed=801)


@pytest.mark.parametrize("c,d,k", [(64, 64, 2), (32, 128, 2), (128, 32, 3), (64, 128, 1), (32, 32, 1)])
def test_routed_pieces_shapes(c, d, k):
    w = si.Workload(f"rpieces_{c}x{d}", "bf16", H=3, c=c, d=d, N=6, topk=k)
    _check(w, [5200, 1800], seed=810 + c + d + k)


def test_routed_pieces_exact_boundaries():
    """Router logits that give one head's partitions 1024 (four whole
    pieces), 1025 (four pieces and one record), 1 and 0 records, with
    P = 256."""
    w = si.Workload("rpieces_edges", "bf16", H=1, c=128, d=128, N=4, topk=1)
    counts = [1024, 1025, 1, 0]
    T = sum(counts)
    inp = si.forward_inputs(w, lengths=[T], seed=820)
    part = np.concatenate([np.full(n, p) for p, n in enumerate(counts)])
    np.random.default_rng(821).shuffle(part)
    z = np.random.default_rng(822).standard_normal((T, 1, w.N)).astype(np.float32)
    z[np.arange(T), 0, part] = 8.0
    inp["router_logits"] = si.f32_to_bf16_bits(z)
    assert _piece_len(T, 1, T, 1, w.N, 1) == 256
    got, ref = _check(w, [T], seed=820, inp=inp)
    assert np.array_equal(np.bincount(got["idx"].ravel(), minlength=w.N), counts)


def test_routed_pieces_fig6_setting():
    """The setting of the page's Fig. 6 at L = 16K: H = 8, N = 4, k = 1, two
    sequences of 8192 tokens (segments of about 2,048 records, 4 pieces of
    512)."""
    w = si.Workload("rpieces_fig6", "bf16", H=8, c=128, d=128, N=4, topk=1)
    _check(w, [8192, 8192], seed=830, init_scale=0)


def test_routed_pieces_gate_limit():
    """log_alpha = -1.24 per row on every token: the piece decays underflow
    toward zero and the start states must still match."""
    w = si.Workload("rpieces_gate", "bf16", H=2, c=64, d=64, N=4, topk=2)
    lengths = [2100, 700]
    inp = si.forward_inputs(w, lengths=lengths, seed=840)
    inp["log_alpha"] = si.f32_to_bf16_bits(np.full(inp["log_alpha"].shape, -1.24, np.float32))
    _check(w, lengths, seed=840, inp=inp)


def test_routed_pieces_run_twice_bitwise():
    w = si.Workload("rpieces_twice", "bf16", H=2, c=128, d=128, N=4, topk=2)
    inp = si.forward_inputs(w, lengths=[2500, 1100], seed=850)
    announce("routed pieces run twice")
    a = _run_forward(inp, w)
    b = _run_forward(inp, w)
    for k in ("o", "fs"):
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_routed_pieces_long_sequence():
    """One sequence of 40,000 tokens, H = 1, N = 1, k = 1: one segment of
    every token, cut into 20 pieces of 2048 records (past the 16-piece aim:
    the longest prologue)."""
    w = si.Workload("rpieces_long", "bf16", H=1, c=64, d=64, N=1, topk=1)
    assert _piece_len(40000, 1, 40000, 1, 1, 1) == 2048
    _check(w, [40000], seed=860)


def test_routed_pieces_with_own_shared_query_key():
    """Split routed segments beside a shared partition with its own query
    and key logits: the routed pieces' states come from the routed keys in
    the same launch as the shared pieces', which use the shared keys."""
    from test_gpu_forward_ex import _check as check_ex
    w = si.Workload("rpieces_own", "bf16", H=2, c=128, d=128, N=4, topk=2)
    lengths = [4000, 2600]
    assert _piece_len(sum(lengths), 2, max(lengths), w.H, w.N, w.topk) == 256
    rng = np.random.default_rng(870)
    init = (0.5 * rng.standard_normal((2, w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    check_ex(w, lengths, "varlen", seed=871, init=init, own_shared=True)
