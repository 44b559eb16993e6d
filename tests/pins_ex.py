"""Pins of the oracle's general form (the shared partition's own query and
key, §2.5; read sets that differ from write sets, §2.3, of "Scaling Linear
Attention with Sparse State Expansion: 中文研读笔记") against formulations that
do not walk its recurrence.  Each pin raises AssertionError on a mismatch."""
from __future__ import annotations

import numpy as np

import oracle
from brute import f64, route, softmax
from sse_inputs import Workload, _tie_free_router, forward_inputs

NAMES = ("q", "key_logits", "v", "log_alpha", "router_logits")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _weights(z, N, k):
    """om[t, i] = softmax(z_t)_i if i is among the k largest logits of z_t."""
    e, sel = route(z, k)
    om = np.zeros((z.shape[0], N))
    rows = np.arange(z.shape[0])[:, None]
    om[rows, sel] = e[rows, sel]
    return om


def quadratic_form_ex(q, kl, v, la, z, N, k, qs=None, ks=None, zr=None, kr=None, init=None):
    """Unrolled closed form for one (sequence, head) with write weights
    ww[s, i] (router z, top-k) and read weights wr[t, i] (read logits zr,
    top-kr; = ww when zr is None).  With G^i_j(t) = sum over writes u <= t of
    partition i of log alpha_uj (all u for the shared partition):
        o_t = sum_i wr[t,i] [sum_{s<=t} ww[s,i] sum_j q_tj kappa_sj
                 e^{G^i_j(t) - G^i_j(s)} v_s + (q_t e^{G^i(t)}) S0^i]
              + the same for the shared partition with q_sh, kappa_sh, weight 1."""
    q, kl, v, la, z = (f64(a) for a in (q, kl, v, la, z))
    qs = q if qs is None else f64(qs)
    ks = kl if ks is None else f64(ks)
    T, c = q.shape
    d = v.shape[1]
    ww = _weights(z, N, k)
    wr = ww if zr is None else _weights(f64(zr), N, kr)
    kap, kaps = softmax(kl), softmax(ks)
    S0 = np.zeros((N + 1, c, d)) if init is None else np.asarray(init, np.float64)
    o = np.zeros((T, d))
    ST = np.zeros((N + 1, c, d))
    for i in range(N + 1):
        shared = i == N
        wrt = np.ones(T) if shared else (ww[:, i] > 0).astype(float)
        G = np.cumsum(la * wrt[:, None], axis=0)
        wwi = np.ones(T) if shared else ww[:, i]
        wri = np.ones(T) if shared else wr[:, i]
        qq, kk = (qs, kaps) if shared else (q, kap)
        for t in range(T):
            if wri[t] == 0:
                continue
            a = (qq[t][None, :] * kk[:t + 1] * np.exp(G[t][None, :] - G[:t + 1])).sum(axis=1)
            o[t] += wri[t] * ((a * wwi[:t + 1]) @ v[:t + 1] + (qq[t] * np.exp(G[t])) @ S0[i])
        if T:
            ST[i] = ((kk * wwi[:, None]) * np.exp(G[-1][None, :] - G)).T @ v + \
                np.exp(G[-1])[:, None] * S0[i]
        else:
            ST[i] = S0[i]
    return o, ST


def _inputs(lengths, c, d, N, k, dt, seed, H=2):
    w = Workload("ex", dt, H=H, c=c, d=d, N=N, topk=k, seed=seed)
    inp = forward_inputs(w, lengths=lengths, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    T = int(sum(lengths))
    cast = (lambda x: x.astype(np.float32)) if dt == "f32" else \
        (lambda x: __import__("sse_inputs").f32_to_bf16_bits(x.astype(np.float32)))
    inp["q_sh"] = cast(rng.standard_normal((T, H, c)))
    inp["kl_sh"] = cast(rng.standard_normal((T, H, c)))
    inp["z_r"] = _tie_free_router(rng, (T, H, N), 1.0, dt)
    return inp


def pin_ex_defaults_are_the_forward(lib):
    """With no optional inputs, and with shared q/k = q/k and read logits =
    router logits, the general form gives the pinned forward's bits."""
    for n, (dt, N, k) in enumerate((("f32", 4, 1), ("bf16", 6, 3), ("f32", 1, 1))):
        inp = _inputs([30, 1, 0, 17], 8, 6, N, k, dt, 400 + n)
        init = np.random.default_rng(n).standard_normal((4, 2, N + 1, 8, 6))
        ref = oracle.forward(*(inp[x] for x in NAMES), inp["cu_seqlens"], N, k,
                             initial_states=init, lib=lib)
        for extra in ({}, dict(q_shared=inp["q"], key_logits_shared=inp["key_logits"],
                                read_router_logits=inp["router_logits"], read_topk=k)):
            out = oracle.forward_ex(*(inp[x] for x in NAMES), inp["cu_seqlens"], N, k,
                                    initial_states=init, lib=lib, **extra)
            assert np.array_equal(out["o"], ref["o"]) and \
                np.array_equal(out["final_states"], ref["final_states"]), (n, extra.keys())
            assert np.array_equal(out["write_idx"], ref["topk_idx"])
            assert np.array_equal(out["read_idx"], ref["topk_idx"])


def pin_ex_quadratic_form(lib):
    """Own shared q/k and separate read sets against the closed form, with
    and without initial states, read sets larger and smaller than the
    write sets."""
    cases = [([25, 9], 6, 5, 5, 2, 3, "f32"), ([33], 8, 4, 4, 1, 4, "bf16"),
             ([20, 11], 5, 6, 6, 3, 1, "f32")]
    for n, (lengths, c, d, N, k, kr, dt) in enumerate(cases):
        inp = _inputs(lengths, c, d, N, k, dt, 420 + n)
        init = np.random.default_rng(430 + n).standard_normal((len(lengths), 2, N + 1, c, d))
        cu = inp["cu_seqlens"]
        for ini in (None, init):
            out = oracle.forward_ex(*(inp[x] for x in NAMES), cu, N, k, inp["q_sh"],
                                    inp["kl_sh"], inp["z_r"], kr, initial_states=ini, lib=lib)
            for s in range(len(lengths)):
                sl = slice(int(cu[s]), int(cu[s + 1]))
                for h in range(2):
                    o_ref, S_ref = quadratic_form_ex(
                        *(inp[x][sl, h] for x in NAMES), N, k, inp["q_sh"][sl, h],
                        inp["kl_sh"][sl, h], inp["z_r"][sl, h], kr,
                        None if ini is None else ini[s, h])
                    assert _rel(out["o"][sl, h], o_ref) < 1e-12, (n, s, h)
                    assert _rel(out["final_states"][s, h], S_ref) < 1e-12, (n, s, h)


def pin_ex_read_only_partition(lib):
    """A partition that is read at every token but never written returns
    e_r q S0 from its initial state (identity transition while not written,
    no decay) and keeps that state bit for bit; the rest of o is the shared
    partition's read."""
    c, d, N = 4, 3, 3
    inp = _inputs([12], c, d, N, 1, "f32", 440, H=1)
    z = inp["router_logits"].copy()
    z[..., 2] = -40.0                      # never written
    inp["router_logits"] = z
    zr = inp["z_r"].copy()
    zr[..., 2] = 40.0                      # the only partition read
    init = np.zeros((1, 1, N + 1, c, d))
    init[0, 0, 2] = np.random.default_rng(441).standard_normal((c, d))
    out = oracle.forward_ex(*(inp[x] for x in NAMES), inp["cu_seqlens"], N, 1, None, None, zr, 1,
                            initial_states=init, lib=lib)
    er = softmax(f64(zr[:, 0]))[:, 2]
    expect = er[:, None] * (f64(inp["q"][:, 0]) @ init[0, 0, 2]) + _shared_read(inp)
    assert _rel(out["o"][:, 0], expect) < 1e-12
    assert np.array_equal(out["final_states"][0, 0, 2], init[0, 0, 2])
    assert (out["read_idx"] == 2).all()


def _shared_read(inp):
    """q_t S^sh_t of the shared partition alone (plain GLA with weight 1)."""
    q, kl, v, la = (f64(inp[x][:, 0]) for x in ("q", "key_logits", "v", "log_alpha"))
    kap = softmax(kl)
    T = q.shape[0]
    G = np.cumsum(la, axis=0)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        a = (q[t][None, :] * kap[:t + 1] * np.exp(G[t][None, :] - G[:t + 1])).sum(axis=1)
        o[t] = a @ v[:t + 1]
    return o


EX_PINS = [pin_ex_defaults_are_the_forward, pin_ex_quadratic_form, pin_ex_read_only_partition]
