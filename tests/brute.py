"""Independent numpy formulations used to pin the oracle (tests only).

None of these walks the token recurrence of the oracle: each one evaluates a
different, closed form of the same quantity, all taken from the web page
"Scaling Linear Attention with Sparse State Expansion: 中文研读笔记".
"""
from __future__ import annotations

import numpy as np

from sse_inputs import bf16_bits_to_f32


def f64(a):
    """Exact fp64 view of an fp32 array or a uint16 bf16 bit array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def softmax(x, axis=-1):
    m = x.max(axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=axis, keepdims=True)


def route(z, k):
    """Router of §2.3 eqs. (9)-(10): probabilities e and the k selected
    partitions, descending by logit, equal logits -> lower index (a stable
    argsort of the negated logits)."""
    e = softmax(z)
    sel = np.argsort(-z, axis=-1, kind="stable")[..., :k]
    return e, sel


def weights_matrix(z, N, k):
    """omega[t, i]: router weight e_t^i if partition i is selected at t else 0
    (i < N), and omega[t, N] = 1 for the shared partition (§2.5)."""
    e, sel = route(z, k)
    T = z.shape[0]
    om = np.zeros((T, N + 1))
    rows = np.arange(T)[:, None]
    om[rows, sel] = e[rows, sel]
    om[:, N] = 1.0
    return om


def quadratic_form(q, kl, v, la, z, N, k, init=None):
    """Unrolled closed form of §2.4 (plus the shared partition and an
    optional initial state) for one sequence and one head, T small.

    With cumulative per-partition log-gates
        G^i_j(t) = sum over u <= t with i selected at u of log_alpha[u, j]
    (all u for the shared partition), the output is
        o_t = sum_i w^i_t [ sum_{s<=t} w^i_s (sum_j q_tj kappa_sj
                 exp(G^i_j(t) - G^i_j(s))) v_s + (q_t * exp(G^i(t))) S0^i ]
    and the final state of partition i is
        S^i = diag(exp(G^i(T-1))) S0^i
              + sum_s w^i_s diag(exp(G^i(T-1) - G^i(s))) kappa_s^T v_s.
    """
    q, kl, v, la, z = (f64(a) for a in (q, kl, v, la, z))
    T, c = q.shape
    d = v.shape[1]
    kappa = softmax(kl)
    om = weights_matrix(z, N, k)
    active = om > 0
    o = np.zeros((T, d))
    final = np.zeros((N + 1, c, d))
    causal = np.tril(np.ones((T, T), bool))
    for i in range(N + 1):
        G = np.cumsum(la * active[:, i:i + 1], axis=0)            # [T, c]
        dec = np.exp(G[:, None, :] - G[None, :, :])               # [t, s, c]
        M = np.einsum("tj,sj,tsj->ts", q, kappa, dec) * causal
        M *= om[:, i:i + 1] * om[None, :, i]
        o += M @ v
        decT = np.exp(G[-1][None, :] - G)                          # [s, c]
        final[i] = (kappa * decT * om[:, i:i + 1]).T @ v
        if init is not None:
            S0 = np.asarray(init[i], np.float64)
            o += om[:, i:i + 1] * ((q * np.exp(G)) @ S0)
            final[i] += np.exp(G[-1])[:, None] * S0
    return o, final


def gla(q, kappa, v, la, S0=None):
    """Single-state gated linear attention, eq. (6) of §2.1 with diagonal
    Lambda_t = diag(exp(log_alpha_t)): S_t = Lambda_t S_{t-1} + kappa_t^T v_t,
    o_t = q_t S_t."""
    T, c = q.shape
    d = v.shape[1]
    S = np.zeros((c, d)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, d))
    for t in range(T):
        S = np.exp(la[t])[:, None] * S + np.outer(kappa[t], v[t])
        o[t] = q[t] @ S
    return o, S


def masked_linear_attention(q, kl, v, z, N, k):
    """alpha = 1 (log_alpha = 0): the recurrence is plain linear attention of
    §一, gated per partition.  o = ((Q K^T) * M) V with
    M_ts = [s <= t] (sum over partitions selected at both t and s of
    e_t^i e_s^i, plus 1 for the shared partition)."""
    q, kl, v, z = (f64(a) for a in (q, kl, v, z))
    kappa = softmax(kl)
    om = weights_matrix(z, N, k)
    M = np.tril(om @ om.T)
    return ((q @ kappa.T) * M) @ v
