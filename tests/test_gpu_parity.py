"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: top-k indices and grouping arrays bit-exact; o and final states within
max|err|/rms(ref) <= 5e-3 for bf16 inputs and <= 1e-5 for fp32 inputs;
states of partitions that are not selected byte-identical.
Small cases are compared element by element; the full-size workloads are run
in the launch configuration the benchmark times and compared on sampled
(sequence, head) units the oracle recomputes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _dev_inputs(inp):
    return {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}


def _run_forward(inp, w, init=None, max_seqlen=None):
    d = _dev_inputs(inp)
    T = d["q"].shape[0]
    idx = torch.empty((T, w.H, w.topk), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.H, w.topk), dtype=torch.float32, device="cuda")
    init_d = None if init is None else torch.from_numpy(init).cuda()
    if max_seqlen is None:
        cu = inp["cu_seqlens"]
        max_seqlen = int((cu[1:] - cu[:-1]).max()) if len(cu) > 1 else 0
    o, fs = sse.sse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"],
                            w.N, w.topk, d["cu_seqlens"], max_seqlen, init_d, topk_idx=idx,
                            topk_w=wt)
    torch.cuda.synchronize()
    return o.cpu().numpy(), fs.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()


def _check_states_per_partition(fs, ref_fs, tol):
    """Final states checked one partition state at a time: every
    (sequence, head, partition) c x d state within tol of its own rms, and
    states the oracle leaves at zero exactly zero."""
    err = np.abs(fs - ref_fs).max(axis=(3, 4))
    rms = np.sqrt(np.mean(ref_fs * ref_fs, axis=(3, 4)))
    zero = rms == 0
    assert (err[zero] == 0).all(), "a state the oracle leaves at zero is not zero"
    worst = float((err[~zero] / rms[~zero]).max()) if (~zero).any() else 0.0
    print(f"  worst per-partition state rel err {worst:.3e}  (tol {tol})", flush=True)
    assert worst <= tol


def _check_full(w, lengths, seed=0, init=None, tag="", states_per_partition=False):
    inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    announce(tag or w.name, "seed", seed, "lengths", lengths, "H", w.H, "c", w.c, "d", w.d,
             "N", w.N, "k", w.topk, "sse_forward")
    o, fs, idx, wt = _run_forward(inp, w, init)
    ref = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                         initial_states=init, threads=8)
    tol = TOL[w.dtype]
    assert np.array_equal(idx, ref["topk_idx"]), "top-k indices differ"
    assert rel_err(wt, ref["topk_e"]) < 1e-5
    eo, es = rel_err(o, ref["o"]), rel_err(fs, ref["final_states"])
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}  (tol {tol})", flush=True)
    assert eo <= tol
    if states_per_partition:
        _check_states_per_partition(fs, ref["final_states"], tol)
    else:
        assert es <= tol
    return inp, o, fs, ref


# ---------------------------------------------------------------- small, full
def test_tiny_f32_full():
    w = si.WORKLOADS["tiny_f32"]
    _check_full(w, [w.T] * w.B)


def test_small_bf16_full():
    w = si.WORKLOADS["small_bf16"]
    _check_full(w, [w.T] * w.B)


def test_main_shape_ragged():
    """c=d=128, N=16, k=2 (the main workload's shapes and distributions) at
    lengths that span many chunks, a ragged tail, length 1 and an empty sequence."""
    w = si.Workload("main_small", "bf16", H=2, c=128, d=128, N=16, topk=2, router_std=1.5)
    _check_full(w, [1000, 77, 0, 1, 333], seed=3)


def test_varlen_shape_ragged():
    w = si.Workload("varlen_small", "bf16", H=2, c=128, d=128, N=32, topk=4)
    _check_full(w, [700, 129, 64, 63], seed=5)


@pytest.mark.parametrize("c,d", [(128, 128), (64, 32), (32, 128), (128, 64)])
def test_f32_other_shapes(c, d):
    w = si.Workload(f"f32_{c}x{d}", "f32", H=2, c=c, d=d, N=4, topk=2)
    _check_full(w, [150, 40, 65], seed=11)


@pytest.mark.parametrize("c,d", [(64, 128), (128, 32), (32, 64)])
def test_bf16_other_shapes(c, d):
    w = si.Workload(f"bf16_{c}x{d}", "bf16", H=3, c=c, d=d, N=6, topk=3)
    _check_full(w, [300, 5, 128], seed=12)


@pytest.mark.parametrize("c,d", [(32, 64), (64, 128), (128, 32), (128, 128)])
def test_multi_piece_with_initial_states(c, d):
    """Sequences spanning several pieces of the shared partition (piece
    states combined with random initial states; with this few (sequence,
    head) units the pieces are 256 tokens), lengths at and just past a piece
    boundary, a 3-token and an empty sequence; every element checked."""
    w = si.Workload(f"pieces_{c}x{d}", "bf16", H=2, c=c, d=d, N=8, topk=2)
    lengths = [2100, 1024, 1025, 3, 0]
    rng = np.random.default_rng(41)
    init = (0.5 * rng.standard_normal((len(lengths), w.H, w.N + 1, c, d))).astype(np.float32)
    _check_full(w, lengths, seed=40, init=init, tag=w.name)


def test_sixteen_shared_pieces():
    """The deepest chain of shared pieces the piece-length rule allows: two
    (sequence, head) units per sequence and 4,096 tokens give 16 pieces of
    256 tokens (the second sequence ends in a 161-token piece), so the last
    piece's input state combines 15 piece aggregates with the initial
    state; every element checked."""
    w = si.Workload("pieces16", "bf16", H=2, c=128, d=128, N=4, topk=1)
    lengths = [4096, 4001]
    rng = np.random.default_rng(43)
    init = (0.5 * rng.standard_normal((len(lengths), w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    _check_full(w, lengths, seed=42, init=init, tag=w.name)


@pytest.mark.parametrize("dtype,N,k,H,cd", [("bf16", 64, 8, 5, 64), ("f32", 64, 8, 3, 32),
                                           ("bf16", 1, 1, 2, 128), ("f32", 1, 1, 2, 32),
                                           ("bf16", 6, 6, 5, 64)])
def test_forward_partition_extremes(dtype, N, k, H, cd):
    """Largest router (N = 64, k = 8), the degenerate single partition
    (N = k = 1: routed and shared states both equal the GLA state), every
    partition selected (k = N), and head counts that leave a partial group of
    the router's 4-head blocks; ragged lengths, every element checked.
    With fp32 inputs and N = 64 the shared state is an order of magnitude
    larger than the 64 routed ones (it takes every token with weight 1), so
    its fp32 rounding alone reaches 1e-5 of the rms of the whole states
    tensor: there the states are checked one partition state at a time."""
    w = si.Workload(f"extreme_{dtype}_n{N}k{k}", dtype, H=H, c=cd, d=cd, N=N, topk=k)
    _check_full(w, [300, 1, 70], seed=50 + N + k, states_per_partition=(dtype == "f32" and N > 8))


def test_initial_states_and_unselected_partition():
    """Random initial states; partition 7 is never chosen (its logit is the
    row minimum), so its final state must equal its initial state byte for
    byte, in every sequence and head."""
    w = si.Workload("init_unsel", "bf16", H=2, c=64, d=64, N=8, topk=2)
    lengths = [200, 90]
    inp = si.forward_inputs(w, lengths=lengths, seed=21)
    z = si.bf16_bits_to_f32(inp["router_logits"])
    z[..., 7] = -30.0
    inp["router_logits"] = si.f32_to_bf16_bits(z)
    rng = np.random.default_rng(22)
    init = rng.standard_normal((2, w.H, w.N + 1, w.c, w.d)).astype(np.float32)
    announce("init_unsel", "sse_forward")
    o, fs, idx, _ = _run_forward(inp, w, init)
    assert not (idx == 7).any()
    assert np.array_equal(fs[:, :, 7].view(np.uint32), init[:, :, 7].view(np.uint32))
    ref = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                         initial_states=init.astype(np.float64))
    assert rel_err(o, ref["o"]) <= TOL["bf16"]
    assert rel_err(fs, ref["final_states"]) <= TOL["bf16"]


def test_resume_matches_one_pass():
    w = si.Workload("resume", "bf16", H=2, c=128, d=128, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[500], seed=31)
    announce("resume", "sse_forward x3")
    o_all, fs_all, _, _ = _run_forward(inp, w)
    a = 230
    p1 = {n: inp[n][:a] for n in NAMES}
    p1["cu_seqlens"] = np.array([0, a], np.int32)
    p2 = {n: inp[n][a:] for n in NAMES}
    p2["cu_seqlens"] = np.array([0, 500 - a], np.int32)
    o1, fs1, _, _ = _run_forward(p1, w)
    o2, fs2, _, _ = _run_forward(p2, w, init=fs1)
    assert rel_err(np.concatenate([o1, o2]), o_all) <= TOL["bf16"]
    assert rel_err(fs2, fs_all) <= TOL["bf16"]


# ------------------------------------------------------------ router, groups
@pytest.mark.parametrize("dtype,N,k", [("bf16", 16, 2), ("bf16", 32, 4), ("f32", 4, 1),
                                       ("bf16", 64, 8), ("f32", 7, 3)])
def test_router_bitexact(dtype, N, k):
    w = si.Workload("router", dtype, H=3, c=1, d=1, N=N, topk=k)
    inp = si.forward_inputs(w, lengths=[4000], seed=41)
    announce("router", dtype, N, k, "sse_router_topk")
    idx, wt = sse.sse_router_topk(to_dev(inp["router_logits"]), k)
    torch.cuda.synchronize()
    ref = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], N, k)
    assert np.array_equal(idx.cpu().numpy().reshape(ref["topk_idx"].shape), ref["topk_idx"])
    assert rel_err(wt.cpu().numpy().reshape(ref["topk_e"].shape), ref["topk_e"]) < 1e-5


@pytest.mark.parametrize("lengths,H,N,k", [([8192] * 4, 16, 16, 2), ([300, 0, 1, 257, 256], 3, 5, 2),
                                           ([14090, 10808, 1277], 4, 32, 4)])
def test_grouping_bitexact(lengths, H, N, k):
    rng = np.random.default_rng(51)
    T = int(sum(lengths))
    idx = np.argsort(rng.random((T, H, N)), axis=-1)[..., :k].astype(np.int32)
    wts = rng.random((T, H, k)).astype(np.float32)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    announce("grouping", lengths, H, N, k, "sse_group_by_partition")
    off, tok, slot, sw = sse.sse_group_by_partition(to_dev(idx), to_dev(wts), to_dev(cu), N,
                                                    max(lengths))
    torch.cuda.synchronize()
    r_off, r_tok, r_slot = oracle.group(idx, cu, N)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(tok.cpu().numpy(), r_tok)
    assert np.array_equal(slot.cpu().numpy(), r_slot)
    seg_of = np.repeat(np.arange(len(r_off) - 1), np.diff(r_off))
    head = (seg_of // N) % H
    assert np.array_equal(sw.cpu().numpy(), wts[r_tok, head, r_slot])


# -------------------------------------------------------- full-size, sampled
def _sampled_units_check(w, inp, o, fs, idx, units):
    cu = inp["cu_seqlens"]
    tol = TOL[w.dtype]
    for (s, h) in units:
        t0, t1 = int(cu[s]), int(cu[s + 1])
        ro, rS, ridx, _ = oracle.unit(*(inp[n] for n in NAMES), t0, t1, h, w.N, w.topk)
        assert np.array_equal(idx[t0:t1, h], ridx), (s, h)
        eo, es = rel_err(o[t0:t1, h], ro), rel_err(fs[s, h], rS)
        print(f"  unit s={s} h={h}: o {eo:.3e} states {es:.3e}", flush=True)
        assert eo <= tol and es <= tol, (s, h, eo, es)


def test_main_full_size_sampled():
    w = si.WORKLOADS["main_bf16"]
    inp = si.forward_inputs(w)
    announce("main_bf16 full size", "B", w.B, "T", w.T, "sse_forward")
    o, fs, idx, _ = _run_forward(inp, w, max_seqlen=w.T)
    _sampled_units_check(w, inp, o, fs, idx, [(0, 0), (3, 15), (1, 7)])


def test_varlen_full_size_sampled():
    w = si.WORKLOADS["varlen_bf16"]
    inp = si.forward_inputs(w)
    lens = np.diff(inp["cu_seqlens"])
    announce("varlen_bf16 full size", "lengths", lens.tolist(), "sse_forward")
    o, fs, idx, _ = _run_forward(inp, w)
    longest = int(np.argmax(lens))
    _sampled_units_check(w, inp, o, fs, idx, [(longest, 3), (len(lens) - 1, 15), (2, 0)])


# ------------------------------------------------------------------- decode
def _decode_check(w, B, steps, units, seed=0):
    announce("decode", w.name, "B", B, "steps", steps, "sse_decode_step")
    states = np.stack([si.decode_states(w, b) for b in range(B)])
    toks = si.decode_inputs(w, steps=steps, B=B, seed=seed)
    st_d = torch.from_numpy(states).cuda()
    d_in = {n: to_dev(toks[n]) for n in NAMES}
    outs = []
    idxs = []
    for t in range(steps):
        idx = torch.empty((B, w.H, w.topk), dtype=torch.int32, device="cuda")
        if t < 2:
            before = st_d.clone()
        o = sse.sse_decode_step(*(d_in[n][t] for n in NAMES), w.N, w.topk, st_d, topk_idx=idx)
        if t < 2:
            # unselected routed partitions must keep every bit
            sel = torch.zeros((B, w.H, w.N + 1), dtype=torch.bool, device="cuda")
            sel.scatter_(2, idx.long(), True)
            sel[..., w.N] = True
            same = (before.view(torch.int32) == st_d.view(torch.int32)).flatten(3).all(-1)
            assert bool((same | sel).all()), "an unselected state changed"
            assert not bool((same & sel).any()), "a selected state did not change"
            del before
        outs.append(o)
        idxs.append(idx)
    torch.cuda.synchronize()
    o_all = torch.stack(outs).cpu().numpy()        # [steps, B, H, d]
    i_all = torch.stack(idxs).cpu().numpy()
    fs = st_d.cpu().numpy()
    tol = TOL[w.dtype]
    for (b, h) in units:
        seq = {n: np.ascontiguousarray(toks[n][:, b]) for n in NAMES}   # [steps, H, .]
        ro, rS, ridx, _ = oracle.unit(*(seq[n] for n in NAMES), 0, steps, h, w.N, w.topk,
                                      state=states[b, h].astype(np.float64))
        assert np.array_equal(i_all[:, b, h], ridx)
        eo, es = rel_err(o_all[:, b, h], ro), rel_err(fs[b, h], rS)
        print(f"  decode unit b={b} h={h}: o {eo:.3e} states {es:.3e}", flush=True)
        assert eo <= tol and es <= tol


@pytest.mark.parametrize("dtype,N,k,cd", [("bf16", 64, 8, 64), ("bf16", 1, 1, 128), ("f32", 64, 8, 32)])
def test_decode_partition_extremes(dtype, N, k, cd):
    w = si.Workload(f"decode_{dtype}_n{N}k{k}", dtype, H=3, c=cd, d=cd, N=N, topk=k, B=4, seed=0)
    _decode_check(w, 4, 5, [(b, h) for b in range(4) for h in range(3)])


def test_decode_small():
    w = si.Workload("decode_small", "bf16", H=3, c=64, d=128, N=6, topk=2, B=5, seed=0)
    _decode_check(w, 5, 9, [(b, h) for b in range(5) for h in range(3)])


def test_decode_f32():
    w = si.Workload("decode_f32", "f32", H=2, c=32, d=32, N=4, topk=1, B=3, seed=0)
    _decode_check(w, 3, 20, [(b, h) for b in range(3) for h in range(2)])


def test_decode_full_size_sampled():
    w = si.WORKLOADS["decode_bf16"]
    _decode_check(w, w.B, w.decode_steps, [(0, 0), (255, 15), (100, 6)])


def test_decode_matches_forward():
    """Decoding a sequence token by token equals the forward over it."""
    w = si.Workload("dec_vs_fwd", "bf16", H=2, c=128, d=128, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[150], seed=61)
    announce("decode vs forward", "sse_forward + sse_decode_step")
    o_f, fs_f, _, _ = _run_forward(inp, w)
    st = torch.zeros((1, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    d_in = {n: to_dev(inp[n]) for n in NAMES}
    outs = [sse.sse_decode_step(*(d_in[n][t:t + 1] for n in NAMES), w.N, w.topk, st)
            for t in range(150)]
    o_d = torch.cat(outs).cpu().numpy()
    assert rel_err(o_d, o_f) <= TOL["bf16"]
    assert rel_err(st.cpu().numpy()[0], fs_f[0]) <= TOL["bf16"]
