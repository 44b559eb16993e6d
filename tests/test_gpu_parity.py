"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: top-k indices and the forward's own grouping (segment offsets, record
tokens and ranks) bit-exact; o and final states within max|err|/rms(ref) <=
5e-3 for bf16 inputs and <= 1e-5 for fp32 inputs, per tensor; states of
partitions that are not selected byte-identical.  Every case is compared
element by element, the full-size workloads included (the oracle runs them
on the host threads in seconds).  Outputs start as NaN and the workspace as
0xff bytes, so an element the kernels never write fails the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import (NAMES, TOL, announce, nan_like, oracle_threads, rel_err, rel_err_big,
                      sentinel_int, to_dev)

pytestmark = pytest.mark.gpu


def _dev_inputs(inp):
    return {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}


def _max_len(cu):
    return int((cu[1:] - cu[:-1]).max()) if len(cu) > 1 else 0


def _run_forward(inp, w, init=None, max_seqlen=None):
    """One sse_forward with sentinel-filled outputs; returns host arrays of
    o, final states, top-k indices and weights and the grouping outputs."""
    d = _dev_inputs(inp)
    T = d["q"].shape[0]
    S = len(inp["cu_seqlens"]) - 1
    R = T * w.H * w.topk
    if max_seqlen is None:
        max_seqlen = _max_len(inp["cu_seqlens"])
    idx = sentinel_int((T, w.H, w.topk))
    wt = nan_like((T, w.H, w.topk))
    soff = sentinel_int((S * w.H * w.N + 1,))
    stok = sentinel_int((R,))
    sslot = sentinel_int((R,))
    o = nan_like((T, w.H, w.d))
    fs = nan_like((S, w.H, w.N + 1, w.c, w.d))
    nbytes = sse.sse_forward_workspace_bytes(T, S, max_seqlen, w.H, w.c, w.d, w.N, w.topk)
    ws = torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device="cuda")
    init_d = None if init is None else torch.from_numpy(np.ascontiguousarray(init, np.float32)).cuda()
    sse.sse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"], w.N,
                    w.topk, d["cu_seqlens"], max_seqlen, init_d, o=o, final_states=fs,
                    topk_idx=idx, topk_w=wt, seg_offsets=soff, seg_tok=stok, seg_slot=sslot,
                    workspace=ws)
    torch.cuda.synchronize()
    out = {"o": o.cpu().numpy(), "fs": fs.cpu().numpy(), "idx": idx.cpu().numpy(),
           "w": wt.cpu().numpy(), "seg_offsets": soff.cpu().numpy(),
           "seg_tok": stok.cpu().numpy(), "seg_slot": sslot.cpu().numpy()}
    del o, fs, ws
    return out


def _oracle_forward(inp, w, init=None):
    return oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                          initial_states=None if init is None else np.asarray(init, np.float64),
                          threads=oracle_threads())


def _compare(w, inp, got, ref, big=False):
    tol = TOL[w.dtype]
    assert np.array_equal(got["idx"], ref["topk_idx"]), "top-k indices differ"
    assert rel_err(got["w"], ref["topk_e"]) < 1e-5
    # the grouping the forward ran, bit for bit against the oracle's counting sort
    r_off, r_tok, r_slot = oracle.group(ref["topk_idx"], inp["cu_seqlens"], w.N)
    assert np.array_equal(got["seg_offsets"], r_off), "segment offsets differ"
    assert np.array_equal(got["seg_tok"], r_tok), "record tokens differ"
    assert np.array_equal(got["seg_slot"], r_slot), "record ranks differ"
    err = rel_err_big if big else rel_err
    eo, es = err(got["o"], ref["o"]), err(got["fs"], ref["final_states"])
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}  (tol {tol})", flush=True)
    assert np.isfinite(got["o"]).all() and np.isfinite(got["fs"]).all()
    assert eo <= tol, eo
    assert es <= tol, es
    return eo, es


def _check_full(w, lengths, seed=0, init=None, tag="", inp=None):
    if inp is None:
        inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    announce(tag or w.name, "seed", seed, "lengths", lengths, "H", w.H, "c", w.c, "d", w.d,
             "N", w.N, "k", w.topk, "sse_forward")
    got = _run_forward(inp, w, init)
    ref = _oracle_forward(inp, w, init)
    _compare(w, inp, got, ref)
    return inp, got, ref


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
    rng = np.random.default_rng(13)
    init = (0.5 * rng.standard_normal((3, w.H, w.N + 1, c, d))).astype(np.float32)
    _check_full(w, [150, 40, 65], seed=11, init=init)


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


def _piece_len(S, H, max_len):
    """The shared-piece length rule of the forward for bf16 inputs: 1024
    tokens, halved down to 256 while fewer than 512 (sequence, head, piece)
    blocks would run and a sequence would keep at most 16 pieces."""
    p = 1024
    pieces = lambda pl: max(1, -(-max_len // pl))
    while p > 256 and S * H * pieces(p) < 512 and pieces(p // 2) <= 16:
        p //= 2
    return p


@pytest.mark.parametrize("n_seq,expect", [(16, 1024), (8, 512)])
def test_long_pieces_with_initial_states(n_seq, expect):
    """Enough (sequence, head) units that the piece-length rule keeps 1024-
    or 512-token pieces (the lengths the main and varlen workloads run),
    random initial states, ragged lengths of 2-3 pieces; every element."""
    w = si.Workload(f"longpieces{expect}", "bf16", H=16, c=32, d=32, N=8, topk=2)
    rng = np.random.default_rng(44 + n_seq)
    lengths = [int(x) for x in rng.integers(2050, 2600, n_seq)]
    assert _piece_len(n_seq, w.H, max(lengths)) == expect
    init = (0.5 * rng.standard_normal((n_seq, w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    _check_full(w, lengths, seed=45 + n_seq, init=init, tag=w.name)


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
    the router's 4-head blocks; ragged lengths, every element checked, the
    final states as one tensor."""
    w = si.Workload(f"extreme_{dtype}_n{N}k{k}", dtype, H=H, c=cd, d=cd, N=N, topk=k)
    _check_full(w, [300, 1, 70], seed=50 + N + k)


# ------------------------------------------------ edges of the input domain
def _block_decay(inp, w, lengths, value):
    """log_alpha = value on every row of tokens whose in-sequence index lies in
    an even 32-token block, 0 on the odd blocks: each chunk of a partition that
    sees every token then decays by 32 |value| in total, and any 64
    consecutive records by at most that much."""
    T = int(sum(lengths))
    pos = np.concatenate([np.arange(L) for L in lengths]) if T else np.zeros(0, int)
    la = np.where(((pos // 32) % 2 == 0)[:, None, None], value, 0.0) * np.ones((T, w.H, w.c))
    inp["log_alpha"] = si.f32_to_bf16_bits(la.astype(np.float32)) if w.dtype == "bf16" \
        else la.astype(np.float32)
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_limit_chunk_decay(dtype):
    """The strongest decay the documented domain allows: every partition sees
    every token (k = N) and 32-token blocks alternate between log_alpha =
    -2.45 per row and 0, so a whole 32-record chunk decays by e^-78.5 (the
    factorisation multiplies by e^+78.5 inside the chunk) while 64
    consecutive records stay above -80; random initial states."""
    w = si.Workload(f"gate_limit_{dtype}", dtype, H=2, c=128, d=128, N=2, topk=2)
    lengths = [700, 130, 33]
    inp = _block_decay(si.forward_inputs(w, lengths=lengths, seed=71), w, lengths, -2.45)
    rng = np.random.default_rng(72)
    init = (0.5 * rng.standard_normal((len(lengths), w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    _check_full(w, lengths, init=init, inp=inp, tag=w.name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_limit_uniform_decay(dtype):
    """Uniform strong decay near the limit: log_alpha = -1.24 on every row of
    every token (64 records of a partition decay by e^-79.4), N = 8, k = 2."""
    w = si.Workload(f"gate_uniform_{dtype}", dtype, H=2, c=64, d=64, N=8, topk=2)
    lengths = [900, 257]
    inp = si.forward_inputs(w, lengths=lengths, seed=73)
    la = np.full((sum(lengths), w.H, w.c), -1.24, np.float32)
    inp["log_alpha"] = si.f32_to_bf16_bits(la) if dtype == "bf16" else la
    _check_full(w, lengths, inp=inp, tag=w.name)


def _tied_router(inp, w, rng):
    """Integer-valued router logits in [-2, 2]: most rows hold equal values,
    so the order of equal logits (lower index first) decides the top-k.  Half
    the zeros are -0, which ties with +0 (they are the same value)."""
    z = rng.integers(-2, 3, inp["router_logits"].shape).astype(np.float32)
    z[(z == 0) & (rng.random(z.shape) < 0.5)] = -0.0
    inp["router_logits"] = si.f32_to_bf16_bits(z) if w.dtype == "bf16" else z
    return inp


@pytest.mark.parametrize("dtype,N,k", [("bf16", 16, 2), ("f32", 8, 3), ("bf16", 32, 4)])
def test_forward_tied_router_logits(dtype, N, k):
    w = si.Workload(f"ties_{dtype}_n{N}", dtype, H=3, c=64, d=64, N=N, topk=k)
    lengths = [400, 65, 1]
    inp = _tied_router(si.forward_inputs(w, lengths=lengths, seed=74), w,
                       np.random.default_rng(75))
    z = inp["router_logits"]
    zf = si.bf16_bits_to_f32(z) if dtype == "bf16" else z
    srt = np.sort(zf.reshape(-1, N), axis=1)
    assert (srt[:, 1:] == srt[:, :-1]).any(axis=1).mean() > 0.9   # ties everywhere
    _check_full(w, lengths, inp=inp, tag=w.name)


@pytest.mark.parametrize("dtype,N,k", [("bf16", 16, 2), ("f32", 7, 3), ("bf16", 64, 8)])
def test_router_tied_logits(dtype, N, k):
    w = si.Workload("router_ties", dtype, H=3, c=1, d=1, N=N, topk=k)
    inp = _tied_router(si.forward_inputs(w, lengths=[3000], seed=76), w,
                       np.random.default_rng(77))
    announce("router ties", dtype, N, k, "sse_router_topk")
    idx, wt = sse.sse_router_topk(to_dev(inp["router_logits"]), k)
    torch.cuda.synchronize()
    ref = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], N, k)
    assert np.array_equal(idx.cpu().numpy().reshape(ref["topk_idx"].shape), ref["topk_idx"])
    assert rel_err(wt.cpu().numpy().reshape(ref["topk_e"].shape), ref["topk_e"]) < 1e-5


def test_slot_dynamic_range():
    """Routed reads whose 32-column groups span a wide range: in every token
    one column of v in each 32-column group is scaled by 2^8, so a group's
    small values sit 2^8 below its largest one (they are carried at a step of
    2^-15 of the largest); every element checked."""
    w = si.Workload("slot_range", "bf16", H=2, c=128, d=128, N=8, topk=2)
    lengths = [600, 90]
    inp = si.forward_inputs(w, lengths=lengths, seed=78)
    v = si.bf16_bits_to_f32(inp["v"]).copy()
    v[..., ::32] *= 256.0
    inp["v"] = si.f32_to_bf16_bits(v)
    _check_full(w, lengths, inp=inp, tag=w.name)


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
    _, got, _ = _check_full(w, lengths, init=init, inp=inp, tag="init_unsel")
    assert not (got["idx"] == 7).any()
    assert np.array_equal(got["fs"][:, :, 7].view(np.uint32), init[:, :, 7].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_all_sequences_empty(dtype):
    """Every sequence empty: o is empty and every final state equals its
    initial state byte for byte (each partition keeps an identity
    transition)."""
    w = si.Workload(f"fwd_empty_{dtype}", dtype, H=2, c=64, d=64, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[0, 0, 0], seed=23)
    init = np.random.default_rng(24).standard_normal((3, w.H, w.N + 1, w.c, w.d)).astype(np.float32)
    d = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    announce(w.name, "lengths [0, 0, 0]", "sse_forward")
    fs = nan_like((3, w.H, w.N + 1, w.c, w.d))
    o = nan_like((0, w.H, w.d))
    sse.sse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"], w.N,
                    w.topk, d["cu_seqlens"], 0, torch.from_numpy(init).cuda(), o=o, final_states=fs)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert np.array_equal(fs.cpu().numpy().view(np.uint32), init.view(np.uint32))


def test_resume_matches_one_pass():
    w = si.Workload("resume", "bf16", H=2, c=128, d=128, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[500], seed=31)
    announce("resume", "sse_forward x3")
    full = _run_forward(inp, w)
    a = 230
    p1 = {n: inp[n][:a] for n in NAMES}
    p1["cu_seqlens"] = np.array([0, a], np.int32)
    p2 = {n: inp[n][a:] for n in NAMES}
    p2["cu_seqlens"] = np.array([0, 500 - a], np.int32)
    r1 = _run_forward(p1, w)
    r2 = _run_forward(p2, w, init=r1["fs"])
    assert rel_err(np.concatenate([r1["o"], r2["o"]]), full["o"]) <= TOL["bf16"]
    assert rel_err(r2["fs"], full["fs"]) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_run_twice_bitwise(dtype):
    """o and the final states are the same bits on every run (no atomics)."""
    w = si.Workload(f"twice_{dtype}", dtype, H=4, c=128, d=128, N=16, topk=2, router_std=1.5)
    inp = si.forward_inputs(w, lengths=[1500, 300, 1], seed=79)
    announce("run twice", dtype, "sse_forward x2")
    a = _run_forward(inp, w)
    b = _run_forward(inp, w)
    for key in ("o", "fs", "idx", "seg_tok"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


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


# ------------------------------------------------------ full size, every unit
def _check_full_size(w, inp, max_seqlen):
    got = _run_forward(inp, w, max_seqlen=max_seqlen)
    ref = _oracle_forward(inp, w)
    _compare(w, inp, got, ref, big=True)


def test_main_full_size():
    """The benchmark's main workload in the launch configuration it times;
    all 64 (sequence, head) units, every element of o and the final states."""
    w = si.WORKLOADS["main_bf16"]
    inp = si.forward_inputs(w)
    announce("main_bf16 full size", "B", w.B, "T", w.T, "sse_forward")
    _check_full_size(w, inp, w.T)


def test_varlen_full_size():
    """The packed varlen workload (8 sequences, N = 32, k = 4), every unit."""
    w = si.WORKLOADS["varlen_bf16"]
    inp = si.forward_inputs(w)
    lens = np.diff(inp["cu_seqlens"])
    announce("varlen_bf16 full size", "lengths", lens.tolist(), "sse_forward")
    _check_full_size(w, inp, int(lens.max()))


# ------------------------------------------------------------------- decode
def _decode_run(w, B, steps, states, toks, check_untouched=2):
    st_d = torch.from_numpy(states).cuda()
    d_in = {n: to_dev(toks[n]) for n in NAMES}
    outs, idxs = [], []
    for t in range(steps):
        idx = sentinel_int((B, w.H, w.topk))
        o = nan_like((B, w.H, w.d))
        if t < check_untouched:
            before = st_d.clone()
        sse.sse_decode_step(*(d_in[n][t] for n in NAMES), w.N, w.topk, st_d, o=o, topk_idx=idx)
        if t < check_untouched:
            # unselected routed partitions keep every bit
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
    del st_d, outs
    return o_all, i_all, fs


def _decode_oracle(w, B, steps, states, toks):
    """The decode steps of every (b, h) as one forward over B sequences of
    `steps` tokens from the given states (threads over units)."""
    seq = {n: np.ascontiguousarray(np.swapaxes(toks[n], 0, 1).reshape((B * steps,) +
                                                                      toks[n].shape[2:]))
           for n in NAMES}
    cu = (np.arange(B + 1) * steps).astype(np.int32)
    ref = oracle.forward(*(seq[n] for n in NAMES), cu, w.N, w.topk,
                         initial_states=states.astype(np.float64), threads=oracle_threads())
    o = np.swapaxes(ref["o"].reshape(B, steps, w.H, w.d), 0, 1)
    idx = np.swapaxes(ref["topk_idx"].reshape(B, steps, w.H, w.topk), 0, 1)
    return o, idx, ref["final_states"]


def _decode_check(w, B, steps, seed=0, states=None, toks=None):
    announce("decode", w.name, "B", B, "steps", steps, "sse_decode_step")
    if states is None:
        states = np.stack([si.decode_states(w, b) for b in range(B)])
    if toks is None:
        toks = si.decode_inputs(w, steps=steps, B=B, seed=seed)
    o_all, i_all, fs = _decode_run(w, B, steps, states, toks)
    r_o, r_idx, r_fs = _decode_oracle(w, B, steps, states, toks)
    tol = TOL[w.dtype]
    assert np.array_equal(i_all, r_idx), "decode top-k indices differ"
    eo, es = rel_err_big(o_all, r_o), rel_err_big(fs, r_fs)
    print(f"  decode o rel err {eo:.3e}  states rel err {es:.3e}  (tol {tol})", flush=True)
    assert np.isfinite(o_all).all()
    assert eo <= tol and es <= tol, (eo, es)
    return o_all, fs


@pytest.mark.parametrize("dtype,N,k,cd", [("bf16", 64, 8, 64), ("bf16", 1, 1, 128), ("f32", 64, 8, 32)])
def test_decode_partition_extremes(dtype, N, k, cd):
    w = si.Workload(f"decode_{dtype}_n{N}k{k}", dtype, H=3, c=cd, d=cd, N=N, topk=k, B=4, seed=0)
    _decode_check(w, 4, 5)


def test_decode_small():
    w = si.Workload("decode_small", "bf16", H=3, c=64, d=128, N=6, topk=2, B=5, seed=0)
    _decode_check(w, 5, 9)


def test_decode_f32():
    w = si.Workload("decode_f32", "f32", H=2, c=32, d=32, N=4, topk=1, B=3, seed=0)
    _decode_check(w, 3, 20)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_tied_router_logits(dtype):
    w = si.Workload(f"decode_ties_{dtype}", dtype, H=3, c=64, d=64, N=16, topk=3, B=6, seed=0)
    toks = si.decode_inputs(w, steps=6, B=6, seed=3)
    _tied_router(toks, w, np.random.default_rng(80))
    _decode_check(w, 6, 6, toks=toks)


def test_decode_gate_limit():
    """log_alpha = -1.24 per row at every step (the decode has no chunked
    factorisation, so this only checks the plain decay at strength)."""
    w = si.Workload("decode_gate", "bf16", H=2, c=128, d=128, N=8, topk=2, B=4, seed=0)
    toks = si.decode_inputs(w, steps=8, B=4, seed=4)
    toks["log_alpha"] = si.f32_to_bf16_bits(np.full(toks["log_alpha"].shape, -1.24, np.float32))
    _decode_check(w, 4, 8, toks=toks)


def test_decode_full_size():
    """The benchmark's decode workload: 256 sequences x 16 heads, 64 steps;
    every step's o (all 4,096 units) and every final state compared."""
    w = si.WORKLOADS["decode_bf16"]
    _decode_check(w, w.B, w.decode_steps)


def test_decode_run_twice_bitwise():
    w = si.Workload("decode_twice", "bf16", H=4, c=128, d=128, N=16, topk=2, B=8, seed=0)
    states = np.stack([si.decode_states(w, b) for b in range(8)])
    toks = si.decode_inputs(w, steps=4, B=8, seed=5)
    announce("decode run twice", "sse_decode_step")
    o1, _, f1 = _decode_run(w, 8, 4, states, toks, check_untouched=0)
    o2, _, f2 = _decode_run(w, 8, 4, states, toks, check_untouched=0)
    assert np.array_equal(o1.view(np.uint8), o2.view(np.uint8))
    assert np.array_equal(f1.view(np.uint8), f2.view(np.uint8))


def test_decode_matches_forward():
    """Decoding a sequence token by token equals the forward over it."""
    w = si.Workload("dec_vs_fwd", "bf16", H=2, c=128, d=128, N=8, topk=2)
    inp = si.forward_inputs(w, lengths=[150], seed=61)
    announce("decode vs forward", "sse_forward + sse_decode_step")
    full = _run_forward(inp, w)
    st = torch.zeros((1, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    d_in = {n: to_dev(inp[n]) for n in NAMES}
    outs = [sse.sse_decode_step(*(d_in[n][t:t + 1] for n in NAMES), w.N, w.topk, st)
            for t in range(150)]
    o_d = torch.cat(outs).cpu().numpy()
    assert rel_err(o_d, full["o"]) <= TOL["bf16"]
    assert rel_err(st.cpu().numpy()[0], full["fs"][0]) <= TOL["bf16"]
