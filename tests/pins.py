"""Pins of the fp64 oracle against facts fixed by the page and by mathematics.

Each pin takes an oracle shared object (``oracle.load(path)``) and raises
AssertionError when the oracle disagrees.  They are run against the real
oracle (test_oracle_pins.py) and against deliberately broken copies of it
(test_oracle_mutants.py), where at least one pin must fail per mutant.

Page: "Scaling Linear Attention with Sparse State Expansion: 中文研读笔记".
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from brute import f64, gla, masked_linear_attention, quadratic_form, route, softmax
from sse_inputs import Workload, forward_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale) if a.size else 0.0


def _case(T, c, d, N, k, dtype="f32", seed=0, router_std=1.0, S=1, H=1):
    w = Workload("pin", dtype, H=H, c=c, d=d, N=N, topk=k, router_std=router_std, seed=seed)
    return forward_inputs(w, lengths=[T] * S if isinstance(T, int) else T)


def _unit(inp, s, h):
    cu = inp["cu_seqlens"]
    sl = slice(int(cu[s]), int(cu[s + 1]))
    return [inp[n][sl, h] for n in ("q", "key_logits", "v", "log_alpha", "router_logits")]


def pin_bruteforce_quadratic_form(lib):
    """Oracle == unrolled closed form of §2.4 with cumulative gate products
    (plus shared partition and initial state), several shapes and dtypes."""
    cases = [(1, 4, 3, 2, 1, "f32"), (37, 8, 5, 4, 1, "f32"), (64, 16, 8, 4, 2, "bf16"),
             (100, 8, 12, 5, 3, "bf16"), (50, 6, 6, 3, 3, "f32")]
    for n, (T, c, d, N, k, dt) in enumerate(cases):
        inp = _case([T, T // 2 + 1], c, d, N, k, dt, seed=10 + n, H=2)
        rng = np.random.default_rng(100 + n)
        init = rng.standard_normal((2, 2, N + 1, c, d))
        for use_init in (False, True):
            out = oracle.forward(*(inp[x] for x in ("q", "key_logits", "v", "log_alpha",
                                                    "router_logits")), inp["cu_seqlens"], N, k,
                                 initial_states=init if use_init else None, lib=lib)
            for s in range(2):
                for h in range(2):
                    q, kl, v, la, z = _unit(inp, s, h)
                    o_ref, st_ref = quadratic_form(q, kl, v, la, z, N, k,
                                                   init=init[s, h] if use_init else None)
                    cu = inp["cu_seqlens"]
                    o = out["o"][cu[s]:cu[s + 1], h]
                    assert _rel(o, o_ref) < 1e-11, ("o", T, c, d, N, k, dt, use_init)
                    assert _rel(out["final_states"][s, h], st_ref) < 1e-11, ("S", T, N, k)


def pin_gla_reduction(lib):
    """N = 1, k = 1: e = 1, the routed and the shared partition both run
    single-state GLA (eq. (6) with diagonal decay), so o = 2 o_GLA and both
    final states equal the GLA state."""
    for n, (T, c, d) in enumerate([(1, 3, 2), (40, 8, 8), (97, 16, 4)]):
        inp = _case(T, c, d, 1, 1, "bf16", seed=20 + n)
        q, kl, v, la, z = _unit(inp, 0, 0)
        rng = np.random.default_rng(7 + n)
        S0 = rng.standard_normal((c, d))
        init = np.stack([S0, S0])[None, None]
        out = oracle.forward(inp["q"], inp["key_logits"], inp["v"], inp["log_alpha"],
                             inp["router_logits"], inp["cu_seqlens"], 1, 1, initial_states=init,
                             lib=lib)
        o_g, S_g = gla(f64(q), softmax(f64(kl)), f64(v), f64(la), S0)
        assert _rel(out["o"][:, 0], 2 * o_g) < 1e-12
        assert _rel(out["final_states"][0, 0, 0], S_g) < 1e-12
        assert _rel(out["final_states"][0, 0, 1], S_g) < 1e-12
        assert np.all(out["topk_idx"] == 0) and np.all(out["topk_e"] == 1.0)


def pin_unselected_identity(lib):
    """§2.6 must-have: partitions a token does not select keep their state
    bit for bit (no decay, no write); checked step by step with decode."""
    w = Workload("pin", "bf16", H=3, c=8, d=6, N=6, topk=2, B=4, seed=3)
    rng = np.random.default_rng(3)
    states = rng.standard_normal((4, 3, 7, 8, 6))
    from sse_inputs import decode_inputs
    steps = decode_inputs(w, steps=12, B=4)
    for t in range(12):
        before = states.copy()
        _, idx, _ = oracle.decode_step(*(steps[n][t] for n in ("q", "key_logits", "v",
                                                                 "log_alpha", "router_logits")),
                                       states, 6, 2, lib=lib)
        for b in range(4):
            for h in range(3):
                sel = set(idx[b, h].tolist())
                assert len(sel) == 2
                for p in range(6):
                    same = np.array_equal(before[b, h, p].view(np.uint64),
                                          states[b, h, p].view(np.uint64))
                    assert same == (p not in sel), (t, b, h, p)
                assert not np.array_equal(before[b, h, 6], states[b, h, 6])


def pin_local_clock_example(lib):
    """The page's worked example (§2.4): one write, then 100 steps of decay
    0.99 with v = 0; the shared partition decays every step (0.366), the
    routed partition is active on 10 of those steps only (0.904)."""
    with open(os.path.join(GOLDEN, "local_clock_example.json")) as f:
        g = json.load(f)
    steps, active, a = g["steps"], g["active_steps"], g["decay_per_step"]
    T, c, d, N = steps + 1, 4, 3, 2
    act = set(np.linspace(5, steps - 3, active).astype(int).tolist())
    assert len(act) == active
    z = np.zeros((T, 1, N), np.float32)
    for t in range(T):
        z[t, 0] = [1.0, 0.0] if (t == 0 or t in act) else [0.0, 1.0]
    rng = np.random.default_rng(1)
    q = rng.standard_normal((T, 1, c)).astype(np.float32)
    kl = rng.standard_normal((T, 1, c)).astype(np.float32)
    v = np.zeros((T, 1, d), np.float32)
    v[0, 0] = [1.0, -2.0, 0.5]
    la = np.full((T, 1, c), np.log(a), np.float32)
    out = oracle.forward(q, kl, v, la, z, np.array([0, T], np.int32), N, 1, lib=lib)
    kappa0 = softmax(kl[0, 0].astype(np.float64))
    e0 = softmax(np.array([1.0, 0.0]))[0]
    first = np.outer(kappa0, v[0, 0].astype(np.float64))
    r_part = out["final_states"][0, 0, 0] / (e0 * first)
    r_shared = out["final_states"][0, 0, N] / first
    nd = g["printed_decimals"]
    assert np.allclose(r_part, r_part.flat[0]) and np.allclose(r_shared, r_shared.flat[0])
    assert round(float(r_part.flat[0]), nd) == g["printed_partition_clock"]
    assert round(float(r_shared.flat[0]), nd) == g["printed_always_decayed"]
    assert np.allclose(out["final_states"][0, 0, 1], 0.0)


def pin_prop4_closed_form(lib):
    """Appendix A Prop. 4 as summarised in §2.7: with q = 1 and keys all
    equal (kappa = 1/c), N = 1, k = 1, the output is
    o_t = (2/c) sum_{s<=t} p_ts v_s with p_ts = sum_j prod_{u=s+1..t} alpha_uj
    (routed + shared partition, each with weight 1)."""
    T, c, d = 30, 5, 4
    rng = np.random.default_rng(4)
    q = np.ones((T, 1, c), np.float32)
    kl = np.full((T, 1, c), 0.25, np.float32)
    v = rng.standard_normal((T, 1, d)).astype(np.float32)
    la = np.log(rng.uniform(0.5, 1.0, (T, 1, c))).astype(np.float32)
    z = np.zeros((T, 1, 1), np.float32)
    out = oracle.forward(q, kl, v, la, z, np.array([0, T], np.int32), 1, 1, lib=lib)
    alpha = np.exp(la[:, 0].astype(np.float64))
    ref = np.zeros((T, d))
    for t in range(T):
        for s in range(t + 1):
            p = np.sum(np.prod(alpha[s + 1:t + 1], axis=0))
            ref[t] += (2.0 / c) * p * v[s, 0]
    assert _rel(out["o"][:, 0], ref) < 1e-12


def pin_masked_linear_attention(lib):
    """alpha = 1: the layer is partition-gated linear attention (§一 / §2.4
    with Lambda = I), o = ((Q K^T) * M) V with co-selection weights."""
    for n, (T, c, d, N, k) in enumerate([(48, 8, 8, 4, 1), (33, 6, 10, 6, 2)]):
        inp = _case(T, c, d, N, k, "f32", seed=40 + n)
        inp["log_alpha"] = np.zeros_like(inp["log_alpha"])
        out = oracle.forward(inp["q"], inp["key_logits"], inp["v"], inp["log_alpha"],
                             inp["router_logits"], inp["cu_seqlens"], N, k, lib=lib)
        q, kl, v, _, z = _unit(inp, 0, 0)
        assert _rel(out["o"][:, 0], masked_linear_attention(q, kl, v, z, N, k)) < 1e-12


def pin_router(lib):
    """eqs. (9)-(10): e is a softmax over N (sums to 1), the selection is the
    stable descending order of the logits (equal logits -> lower index), and
    §2.3's remark: the selected weights sum to at most 1 (no renormalisation)."""
    rng = np.random.default_rng(5)
    T, N, k = 200, 8, 3
    z = rng.integers(-3, 4, (T, 1, N)).astype(np.float32)   # many exact ties on purpose
    q = rng.standard_normal((T, 1, 4)).astype(np.float32)
    v = rng.standard_normal((T, 1, 2)).astype(np.float32)
    la = np.full((T, 1, 4), -0.1, np.float32)
    out = oracle.forward(q, q, v, la, z, np.array([0, T], np.int32), N, k, lib=lib)
    e_all, sel = route(z[:, 0].astype(np.float64), k)
    assert np.array_equal(out["topk_idx"][:, 0], sel)
    assert _rel(out["topk_e"][:, 0], np.take_along_axis(e_all, sel, 1)) < 1e-15
    assert np.all(out["topk_e"].sum(-1) <= 1.0 + 1e-15)
    assert np.allclose(e_all.sum(-1), 1.0)


def pin_grouping(lib):
    """§2.6 varlen grouping: records sorted by (sequence, head, partition)
    with time order kept inside a segment == a stable sort on that key."""
    rng = np.random.default_rng(6)
    lengths = [5, 0, 17, 1, 9]
    H, N, k = 3, 5, 2
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    idx = np.stack([np.stack([rng.permutation(N)[:k] for _ in range(H)]) for _ in range(T)])
    off, tok, slot = oracle.group(idx.astype(np.int32), cu, N, lib=lib)
    seq = np.repeat(np.arange(len(lengths)), lengths)
    t_, h_, j_ = np.meshgrid(np.arange(T), np.arange(H), np.arange(k), indexing="ij")
    key = (seq[t_] * H + h_) * N + idx
    order = np.argsort(key.ravel(), kind="stable")            # flat order is (t, h, j)
    assert np.array_equal(tok, t_.ravel()[order]) and np.array_equal(slot, j_.ravel()[order])
    counts = np.bincount(key.ravel(), minlength=len(lengths) * H * N)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))


def pin_split_consistency(lib):
    """Resume from final states == one pass; packed varlen == separate runs;
    decode token by token == forward (all bit-exact in fp64)."""
    inp = _case([23, 41], 8, 6, 4, 2, "bf16", seed=8, H=2)
    names = ("q", "key_logits", "v", "log_alpha", "router_logits")
    full = oracle.forward(*(inp[n] for n in names), inp["cu_seqlens"], 4, 2, lib=lib)
    for s, (a, b) in enumerate([(0, 23), (23, 64)]):
        one = oracle.forward(*(inp[n][a:b] for n in names), np.array([0, b - a], np.int32), 4,
                             2, lib=lib)
        assert np.array_equal(one["o"], full["o"][a:b])
        assert np.array_equal(one["final_states"][0], full["final_states"][s])
        m = a + 9
        p1 = oracle.forward(*(inp[n][a:m] for n in names), np.array([0, m - a], np.int32), 4, 2,
                            lib=lib)
        p2 = oracle.forward(*(inp[n][m:b] for n in names), np.array([0, b - m], np.int32), 4, 2,
                            initial_states=p1["final_states"], lib=lib)
        assert np.array_equal(np.concatenate([p1["o"], p2["o"]]), full["o"][a:b])
        assert np.array_equal(p2["final_states"][0], full["final_states"][s])
    # decode of sequence 0 token by token
    states = np.zeros((1, 2, 5, 8, 6))
    for t in range(23):
        o, idx, e = oracle.decode_step(*(inp[n][t:t + 1] for n in names), states, 4, 2, lib=lib)
        assert np.array_equal(o[0], full["o"][t]) and np.array_equal(idx[0], full["topk_idx"][t])
    assert np.array_equal(states[0], full["final_states"][0])


PINS = [pin_bruteforce_quadratic_form, pin_gla_reduction, pin_unselected_identity,
        pin_local_clock_example, pin_prop4_closed_form, pin_masked_linear_attention,
        pin_router, pin_grouping, pin_split_consistency]
