"""Pins of the oracle's backward (gradients of L = <do, o> + <dS_final,
S_final>) against (1) torch autograd through an independent, plain PyTorch
fp64 implementation of §2.3 eqs. (9)-(14) with the shared partition of §2.5
("Scaling Linear Attention with Sparse State Expansion: 中文研读笔记"), and
(2) central finite differences of the oracle's own forward.  Each pin raises
AssertionError on a mismatch; the mutant tests run them on broken copies."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from brute import f64
from sse_inputs import Workload, forward_inputs

NAMES = ("q", "key_logits", "v", "log_alpha", "router_logits")
GRADS = ("dq", "dkey_logits", "dv", "dlog_alpha", "drouter_logits")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def torch_unit(q, kl, v, la, z, N, k, init):
    """One (sequence, head) unit: token loop in torch fp64 (autograd-able).
    Top-k is taken on detached logits (stable order: equal logits -> lower
    index); the router weights e flow through the softmax."""
    T, c = q.shape
    S = [init[p] for p in range(N + 1)]
    outs = []
    for t in range(T):
        e = torch.softmax(z[t], dim=0)
        sel = torch.argsort(-z[t].detach(), stable=True)[:k].tolist()
        kap = torch.softmax(kl[t], dim=0)
        alpha = torch.exp(la[t])
        o = torch.zeros(v.shape[1], dtype=torch.float64)
        for r, p in enumerate(sel + [N]):
            w = e[p] if r < k else 1.0
            S[p] = alpha[:, None] * S[p] + w * torch.outer(kap, v[t])
            o = o + w * (q[t] @ S[p])
        outs.append(o)
    return torch.stack(outs) if outs else torch.zeros((0, v.shape[1]), dtype=torch.float64), \
        torch.stack(S)


def _case(lengths, c, d, N, k, dt, seed, H=2):
    w = Workload("bwd", dt, H=H, c=c, d=d, N=N, topk=k, seed=seed)
    inp = forward_inputs(w, lengths=lengths, seed=seed)
    rng = np.random.default_rng(seed + 77)
    T, S = int(sum(lengths)), len(lengths)
    do = rng.standard_normal((T, H, d))
    dfin = rng.standard_normal((S, H, N + 1, c, d))
    init = rng.standard_normal((S, H, N + 1, c, d))
    return inp, do, dfin, init


def pin_backward_autograd(lib):
    """Every gradient (inputs and initial states) equals torch autograd of
    the plain implementation, with and without initial states and final-
    state gradients; bf16 and fp32 inputs; N = k = 1, k = N, ragged."""
    cases = [([9, 4], 4, 3, 4, 2, "f32"), ([7, 1, 0], 3, 5, 3, 3, "bf16"), ([10], 5, 4, 1, 1, "f32"),
             ([6, 5], 4, 4, 6, 1, "bf16")]
    for n, (lengths, c, d, N, k, dt) in enumerate(cases):
        inp, do, dfin, init = _case(lengths, c, d, N, k, dt, 600 + n)
        cu = inp["cu_seqlens"]
        for use_extra in (False, True):
            g = oracle.backward(*(inp[x] for x in NAMES), cu, N, k, do,
                                dfinal_states=dfin if use_extra else None,
                                initial_states=init if use_extra else None, lib=lib)
            for s in range(len(lengths)):
                sl = slice(int(cu[s]), int(cu[s + 1]))
                for h in range(2):
                    ts = [torch.tensor(f64(inp[x][sl, h]), requires_grad=True) for x in NAMES]
                    ti = torch.tensor(init[s, h] if use_extra else np.zeros_like(init[s, h]),
                                      requires_grad=True)
                    o, fs = torch_unit(*ts, N, k, ti)
                    loss = (o * torch.tensor(do[sl, h])).sum() + (fs * torch.tensor(
                        dfin[s, h] if use_extra else np.zeros_like(dfin[s, h]))).sum()
                    grads = torch.autograd.grad(loss, ts + [ti], allow_unused=True)
                    for name, gr in zip(GRADS + ("dinitial_states",), grads):
                        ref = np.zeros(ts[0].shape) if gr is None else gr.numpy()
                        got = g[name][sl, h] if name != "dinitial_states" else g[name][s, h]
                        if name == "dinitial_states":
                            ref = grads[-1].numpy()
                        assert _rel(got, ref) < 1e-11, (n, use_extra, s, h, name, _rel(got, ref))


def pin_backward_finite_differences(lib):
    """Central differences of L(x) = <do, o(x)> + <dS_final, S_final(x)>
    computed with the oracle's forward, element by element on fp32 inputs
    (the perturbed input is rounded to fp32 and the difference actually
    applied is used); the top-k choice is kept (perturbations that change it
    are skipped)."""
    c, d, N, k = 3, 2, 3, 2
    inp, do, dfin, init = _case([6], c, d, N, k, "f32", 650, H=1)
    cu = inp["cu_seqlens"]

    def loss(x):
        out = oracle.forward(*(x[n] for n in NAMES), cu, N, k, initial_states=init, lib=lib)
        return float((out["o"] * do).sum() + (out["final_states"] * dfin).sum()), out["topk_idx"]

    base_idx = loss(inp)[1]
    g = oracle.backward(*(inp[x] for x in NAMES), cu, N, k, do, dfinal_states=dfin,
                        initial_states=init, lib=lib)
    for name, gname in zip(NAMES, GRADS):
        a = inp[name]
        fd = np.zeros(a.shape)
        mask = np.ones(a.shape, bool)
        for ix in np.ndindex(a.shape):
            x0 = float(a[ix])
            h = 1e-3 * max(1.0, abs(x0))
            xp, xm = np.float32(x0 + h), np.float32(x0 - h)
            vals = []
            for xv in (xp, xm):
                b = dict(inp)
                b[name] = a.copy()
                b[name][ix] = xv
                lv, idx = loss(b)
                if not np.array_equal(idx, base_idx):
                    mask[ix] = False
                vals.append(lv)
            fd[ix] = (vals[0] - vals[1]) / (float(xp) - float(xm))
        scale = max(np.sqrt(np.mean(g[gname] ** 2)), 1e-30)
        err = np.max(np.abs(fd - g[gname])[mask]) / scale
        assert err < 2e-4, (name, err)


BACKWARD_PINS = [pin_backward_autograd, pin_backward_finite_differences]
