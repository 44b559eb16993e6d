"""GPU parity of the general decode step (sse_decode_step_ex: the shared
partition's own query and key logits, a read set from its own router
logits) against the fp64 oracle's general forward over the same tokens as
sequences of `steps` tokens from the same states (a decode step is the
forward recurrence advanced by one token).  Every step's o and the final
states are compared, within 5e-3 (bf16 inputs) / 1e-5 (fp32 inputs) of
the reference rms; the chosen write and read sets must match exactly.
States that are neither written nor read must keep every bit, written
states must change, and read-only states must keep every bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import NAMES, TOL, announce, nan_like, oracle_threads, rel_err, rel_err_big, \
    sentinel_int, to_dev

pytestmark = pytest.mark.gpu


def _extra(w, B, steps, seed, own_qk, read_topk):
    """Extra token inputs: own shared q / key logits, read-router logits."""
    rng = np.random.default_rng(seed + 40)
    enc = si.f32_to_bf16_bits if w.dtype == "bf16" else (lambda a: a)
    ex = {}
    if own_qk:
        ex["q_shared"] = enc((rng.standard_normal((steps, B, w.H, w.c)) / np.sqrt(w.c))
                             .astype(np.float32))
        ex["key_logits_shared"] = enc(rng.standard_normal((steps, B, w.H, w.c))
                                      .astype(np.float32))
    if read_topk:
        ex["read_router_logits"] = enc((w.router_std * rng.standard_normal((steps, B, w.H, w.N)))
                                       .astype(np.float32))
    return ex


def _run(w, B, steps, states, toks, ex, read_topk, check_sets=2):
    st_d = torch.from_numpy(states).cuda()
    d_in = {n: to_dev(toks[n]) for n in NAMES}
    d_ex = {n: to_dev(a) for n, a in ex.items()}
    kr = read_topk or w.topk
    outs, widx, ridx = [], [], []
    for t in range(steps):
        wi = sentinel_int((B, w.H, w.topk))
        ri = sentinel_int((B, w.H, kr)) if read_topk else None
        o = nan_like((B, w.H, w.d))
        before = st_d.clone() if t < check_sets else None
        sse.sse_decode_step_ex(*(d_in[n][t] for n in NAMES), w.N, w.topk, st_d,
                               q_shared=d_ex["q_shared"][t] if "q_shared" in d_ex else None,
                               key_logits_shared=(d_ex["key_logits_shared"][t]
                                                  if "key_logits_shared" in d_ex else None),
                               read_router_logits=(d_ex["read_router_logits"][t]
                                                   if "read_router_logits" in d_ex else None),
                               read_topk=read_topk, o=o, topk_idx=wi, read_topk_idx=ri)
        if before is not None:
            wr = torch.zeros((B, w.H, w.N + 1), dtype=torch.bool, device="cuda")
            wr.scatter_(2, wi.long(), True)
            wr[..., w.N] = True
            same = (before.view(torch.int32) == st_d.view(torch.int32)).flatten(3).all(-1)
            assert bool((same | wr).all()), "a state outside the write set changed"
            assert not bool((same & wr).any()), "a written state did not change"
            del before
        outs.append(o)
        widx.append(wi)
        ridx.append(ri if ri is not None else wi)
    torch.cuda.synchronize()
    res = (torch.stack(outs).cpu().numpy(), torch.stack(widx).cpu().numpy(),
           torch.stack(ridx).cpu().numpy(), st_d.cpu().numpy())
    del st_d, outs
    return res


def _seq(a, B, steps):
    """[steps, B, H, x] -> [B*steps, H, x] (sequence-major tokens)."""
    return np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape((B * steps,) + a.shape[2:]))


def _oracle(w, B, steps, states, toks, ex, read_topk):
    cu = (np.arange(B + 1) * steps).astype(np.int32)
    seq = {n: _seq(toks[n], B, steps) for n in NAMES}
    sx = {n: _seq(a, B, steps) for n, a in ex.items()}
    ref = oracle.forward_ex(*(seq[n] for n in NAMES), cu, w.N, w.topk,
                            q_shared=sx.get("q_shared"),
                            key_logits_shared=sx.get("key_logits_shared"),
                            read_router_logits=sx.get("read_router_logits"),
                            read_topk=read_topk or None,
                            initial_states=states.astype(np.float64))
    back = lambda a: np.swapaxes(a.reshape((B, steps) + a.shape[1:]), 0, 1)
    return back(ref["o"]), back(ref["write_idx"]), back(ref["read_idx"]), ref["final_states"]


def _check(w, B, steps, own_qk, read_topk, seed=0, toks=None):
    announce("decode_ex", w.name, "B", B, "steps", steps, "own_qk", own_qk, "read_topk",
             read_topk, "sse_decode_step_ex")
    states = np.stack([si.decode_states(w, b) for b in range(B)])
    if toks is None:
        toks = si.decode_inputs(w, steps=steps, B=B, seed=seed)
    ex = _extra(w, B, steps, seed, own_qk, read_topk)
    o, wi, ri, fs = _run(w, B, steps, states, toks, ex, read_topk)
    r_o, r_wi, r_ri, r_fs = _oracle(w, B, steps, states, toks, ex, read_topk)
    assert np.array_equal(wi, r_wi), "write sets differ"
    assert np.array_equal(ri, r_ri), "read sets differ"
    eo, es = rel_err_big(o, r_o), rel_err_big(fs, r_fs)
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}  (tol {TOL[w.dtype]})", flush=True)
    assert np.isfinite(o).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)


@pytest.mark.parametrize("own_qk,read_topk", [(True, 0), (False, 3), (True, 4), (True, 1)])
def test_decode_ex_bf16(own_qk, read_topk):
    w = si.Workload("decode_ex_bf16", "bf16", H=3, c=64, d=128, N=8, topk=2, B=5, seed=0)
    _check(w, 5, 6, own_qk, read_topk, seed=11)


@pytest.mark.parametrize("c,d", [(32, 32), (128, 64)])
def test_decode_ex_f32(c, d):
    w = si.Workload(f"decode_ex_f32_{c}x{d}", "f32", H=2, c=c, d=d, N=6, topk=3, B=3, seed=0)
    _check(w, 3, 8, True, 2, seed=12)


@pytest.mark.parametrize("N,k,kr", [(64, 8, 8), (1, 1, 1), (5, 5, 5), (16, 1, 8)])
def test_decode_ex_partition_extremes(N, k, kr):
    w = si.Workload(f"decode_ex_n{N}k{k}r{kr}", "bf16", H=2, c=128, d=128, N=N, topk=k, B=4,
                    seed=0)
    _check(w, 4, 4, True, kr, seed=13 + N)


def test_decode_ex_tied_logits():
    """Integer router and read logits in [-2, 2]: ties everywhere, lower
    indices first on both sides."""
    w = si.Workload("decode_ex_ties", "bf16", H=3, c=64, d=64, N=16, topk=3, B=6, seed=0)
    toks = si.decode_inputs(w, steps=5, B=6, seed=14)
    rng = np.random.default_rng(15)
    toks["router_logits"] = si.f32_to_bf16_bits(
        rng.integers(-2, 3, toks["router_logits"].shape).astype(np.float32))
    announce("decode_ex ties")
    states = np.stack([si.decode_states(w, b) for b in range(6)])
    ex = _extra(w, 6, 5, 14, True, 4)
    ex["read_router_logits"] = si.f32_to_bf16_bits(
        rng.integers(-2, 3, ex["read_router_logits"].shape).astype(np.float32))
    o, wi, ri, fs = _run(w, 6, 5, states, toks, ex, 4)
    r_o, r_wi, r_ri, r_fs = _oracle(w, 6, 5, states, toks, ex, 4)
    assert np.array_equal(wi, r_wi) and np.array_equal(ri, r_ri)
    assert rel_err_big(o, r_o) <= TOL["bf16"] and rel_err_big(fs, r_fs) <= TOL["bf16"]


def test_decode_ex_defaults_match_decode_step():
    """With every option NULL the general step computes the default step."""
    w = si.Workload("decode_ex_default", "bf16", H=4, c=128, d=128, N=16, topk=2, B=8, seed=0)
    states = np.stack([si.decode_states(w, b) for b in range(8)])
    toks = si.decode_inputs(w, steps=3, B=8, seed=16)
    announce("decode_ex vs decode_step")
    a = torch.from_numpy(states).cuda()
    b = a.clone()
    d_in = {n: to_dev(toks[n]) for n in NAMES}
    for t in range(3):
        oa = sse.sse_decode_step(*(d_in[n][t] for n in NAMES), w.N, w.topk, a)
        ob = sse.sse_decode_step_ex(*(d_in[n][t] for n in NAMES), w.N, w.topk, b)
        assert rel_err(ob.cpu().numpy(), oa.cpu().numpy()) <= 1e-6
    assert rel_err(b.cpu().numpy(), a.cpu().numpy()) <= 1e-6


def test_decode_ex_matches_forward_ex():
    """Decoding token by token equals sse_forward_ex (masked schedule, own
    shared q/k, read sets) over the same sequence."""
    w = si.Workload("decode_ex_vs_fwd", "bf16", H=2, c=64, d=64, N=8, topk=2)
    T = 120
    inp = si.forward_inputs(w, lengths=[T], seed=17)
    ex = {n: a[:, 0] for n, a in _extra(w, 1, T, 17, True, 3).items()}
    announce("decode_ex vs forward_ex", "sse_forward_ex + sse_decode_step_ex")
    d_in = {n: to_dev(inp[n]) for n in NAMES}
    d_ex = {n: to_dev(a) for n, a in ex.items()}
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o_f, fs_f = sse.sse_forward_ex(d_in["q"], d_in["key_logits"], d_in["v"], d_in["log_alpha"],
                                   d_in["router_logits"], w.N, w.topk, cu, max_seqlen=T,
                                   q_shared=d_ex["q_shared"],
                                   key_logits_shared=d_ex["key_logits_shared"],
                                   read_router_logits=d_ex["read_router_logits"], read_topk=3,
                                   schedule="masked")
    st = torch.zeros((1, w.H, w.N + 1, w.c, w.d), dtype=torch.float32, device="cuda")
    outs = [sse.sse_decode_step_ex(*(d_in[n][t:t + 1] for n in NAMES), w.N, w.topk, st,
                                   q_shared=d_ex["q_shared"][t:t + 1],
                                   key_logits_shared=d_ex["key_logits_shared"][t:t + 1],
                                   read_router_logits=d_ex["read_router_logits"][t:t + 1],
                                   read_topk=3)
            for t in range(T)]
    o_d = torch.cat(outs).cpu().numpy()
    assert rel_err(o_d, o_f.cpu().numpy()) <= TOL["bf16"]
    assert rel_err(st.cpu().numpy()[0], fs_f.cpu().numpy()[0]) <= TOL["bf16"]
