"""Pins of the oracle's row-sparse key variant (§2.2, eqs. (7)-(8) of
"Scaling Linear Attention with Sparse State Expansion: 中文研读笔记") against
formulations that do not walk its recurrence.  Each pin raises
AssertionError on a mismatch; the mutant tests run them against broken
copies of the oracle."""
from __future__ import annotations

import numpy as np

import oracle
from brute import f64, gla, softmax
from sse_inputs import Workload, forward_inputs

NAMES4 = ("q", "key_logits", "v", "log_alpha")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    scale = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def row_topk_mask(kl, k):
    """sel[t, j]: row j is among the k largest key logits of token t (equal
    logits -> lower row first: a stable argsort of the negated logits)."""
    T, c = kl.shape
    top = np.argsort(-kl, axis=-1, kind="stable")[:, :k]
    sel = np.zeros((T, c), bool)
    sel[np.arange(T)[:, None], top] = True
    return sel


def rowsparse_quadratic_form(q, kl, v, la, k, identity, init=None):
    """Unrolled closed form for one (sequence, head): with the masked key
    kappa_s = softmax over the selected rows and cumulative log-gates
    G_j(t) = sum_{u<=t} log alpha~_uj (alpha~ = alpha on selected rows, 1 on
    the others when `identity`),
        o_t = sum_{s<=t} sum_j q_tj kappa_sj e^{G_j(t)-G_j(s)} v_s
              + sum_j q_tj e^{G_j(t)} S0_j,
        S_T = sum_s diag(e^{G(T-1)-G(s)}) kappa_s^T v_s + diag(e^{G(T-1)}) S0."""
    q, kl, v, la = (f64(x) for x in (q, kl, v, la))
    T, c = q.shape
    d = v.shape[1]
    sel = row_topk_mask(kl, k)
    z = np.where(sel, kl, -np.inf)
    kap = np.exp(z - z.max(axis=1, keepdims=True))
    kap /= kap.sum(axis=1, keepdims=True)
    lg = np.where(sel | (not identity), la, 0.0)
    G = np.cumsum(lg, axis=0)                                  # [T, c]
    S0 = np.zeros((c, d)) if init is None else np.asarray(init, np.float64)
    o = np.zeros((T, d))
    for t in range(T):
        w = q[t][None, :] * kap[:t + 1] * np.exp(G[t][None, :] - G[:t + 1])   # [s, j]
        o[t] = w.sum(axis=1) @ v[:t + 1] + (q[t] * np.exp(G[t])) @ S0
    if T:
        ST = (kap * np.exp(G[-1][None, :] - G)).T @ v + np.exp(G[-1])[:, None] * S0
    else:
        ST = S0.copy()
    return o, ST


def _case(lengths, c, d, dtype, seed, H=2):
    w = Workload("rs", dtype, H=H, c=c, d=d, N=1, topk=1, seed=seed)
    return forward_inputs(w, lengths=lengths, seed=seed)


def pin_rowsparse_quadratic_form(lib):
    """Oracle == the closed form, both transition forms, with and without
    initial states, several row counts k (1, c/4, c-1), bf16 and fp32."""
    cases = [([40, 7], 8, 5, 1, "f32"), ([33, 20], 16, 6, 4, "bf16"), ([25], 8, 8, 7, "f32"),
             ([0, 12], 12, 4, 3, "bf16")]
    for n, (lengths, c, d, k, dt) in enumerate(cases):
        inp = _case(lengths, c, d, dt, 300 + n)
        init = np.random.default_rng(310 + n).standard_normal((len(lengths), 2, c, d))
        for identity in (True, False):
            for ini in (None, init):
                out = oracle.rowsparse_forward(*(inp[x] for x in NAMES4), inp["cu_seqlens"], k,
                                               identity, ini, lib=lib)
                cu = inp["cu_seqlens"]
                for s in range(len(lengths)):
                    for h in range(2):
                        sl = slice(int(cu[s]), int(cu[s + 1]))
                        o_ref, S_ref = rowsparse_quadratic_form(
                            *(inp[x][sl, h] for x in NAMES4), k, identity,
                            None if ini is None else ini[s, h])
                        assert _rel(out["o"][sl, h], o_ref) < 1e-12, (n, identity)
                        assert _rel(out["final_states"][s, h], S_ref) < 1e-12, (n, identity)


def pin_rowsparse_all_rows_is_gla(lib):
    """k = c keeps every row: the layer is plain GLA with the softmax key
    (§2.1 eq. 6), whichever transition form."""
    inp = _case([60], 8, 5, "f32", 320, H=1)
    q, kl, v, la = (f64(inp[x][:, 0]) for x in NAMES4)
    ref, _ = gla(q, softmax(kl), v, la)
    for identity in (True, False):
        out = oracle.rowsparse_forward(*(inp[x] for x in NAMES4), inp["cu_seqlens"], 8, identity,
                                       lib=lib)
        assert _rel(out["o"][:, 0], ref) < 1e-12


def pin_rowsparse_unselected_rows_keep_state(lib):
    """Rows whose key logit is always the smallest are never selected: with
    the identity transition their state rows stay the initial ones bit for
    bit; with the plain transition they decay by the product of alpha."""
    c, d, k = 8, 4, 3
    inp = _case([50], c, d, "f32", 330, H=1)
    kl = inp["key_logits"].copy()
    kl[:, :, :2] = -30.0
    inp["key_logits"] = kl
    init = np.random.default_rng(331).standard_normal((1, 1, c, d))
    out = oracle.rowsparse_forward(*(inp[x] for x in NAMES4), inp["cu_seqlens"], k, True, init,
                                   lib=lib)
    assert np.array_equal(out["final_states"][0, 0, :2], init[0, 0, :2])
    out2 = oracle.rowsparse_forward(*(inp[x] for x in NAMES4), inp["cu_seqlens"], k, False, init,
                                    lib=lib)
    dec = np.exp(f64(inp["log_alpha"][:, 0, :2]).sum(axis=0))
    assert _rel(out2["final_states"][0, 0, :2], dec[:, None] * init[0, 0, :2]) < 1e-12


def pin_rowsparse_ties_lower_row(lib):
    """Equal key logits: the lower rows win (k = 1 with all logits equal
    writes row 0 only)."""
    c, d = 6, 3
    inp = _case([5], c, d, "f32", 340, H=1)
    inp["key_logits"] = np.zeros_like(inp["key_logits"])
    out = oracle.rowsparse_forward(*(inp[x] for x in NAMES4), inp["cu_seqlens"], 1, True, lib=lib)
    S = out["final_states"][0, 0]
    assert np.abs(S[0]).sum() > 0 and np.abs(S[1:]).sum() == 0


ROWSPARSE_PINS = [pin_rowsparse_quadratic_form, pin_rowsparse_all_rows_is_gla,
                  pin_rowsparse_unselected_rows_keep_state, pin_rowsparse_ties_lower_row]
