"""Seeded synthetic inputs for the SSE layer (shared by tests, smoke and bench).

This module draws random numbers and rounds them to the storage dtype.  It
holds none of the method's arithmetic: no softmax, no top-k, no recurrence.

Recipe (per workload, numpy ``default_rng``):
  * draw order: [sequence lengths for the varlen workload], q, key_logits, v,
    x, router_logits, all ``standard_normal`` in fp64;
  * log_alpha = logsigmoid(x) / 16 in fp64;
  * router_logits are scaled by the workload's standard deviation;
  * every tensor is rounded fp64 -> fp32 (round to nearest even) and, for
    bf16 workloads, fp32 -> bf16 (round to nearest even on the bit pattern);
  * router rows (token, head) that hold a repeated value after rounding are
    redrawn from the same stream until every row has N distinct values, so
    that top-k has a unique answer;
  * decode states: 0.1 * standard_normal fp32, drawn per sequence b from
    ``default_rng([seed, 4, b])``, so a single sequence can be regenerated.

bf16 tensors are returned as uint16 bit patterns (numpy has no bf16 type).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    H: int
    c: int
    d: int
    N: int
    topk: int
    B: int = 1            # fixed-length batch (forward) or sequences (decode)
    T: int = 0            # tokens per sequence (fixed-length forward)
    router_std: float = 1.0
    varlen: tuple = ()    # (num_seqs, lo, hi) for varlen draws
    decode_steps: int = 0
    seed: int = 0
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", H=1, c=32, d=32, N=4, topk=1, B=1, T=256,
                         notes="fp32, B=1 H=1 T=256 c=d=32 N=4 k=1"),
    "small_bf16": Workload("small_bf16", "bf16", H=4, c=64, d=64, N=8, topk=2, B=2, T=2048,
                           notes="bf16, B=2 H=4 T=2048 c=d=64 N=8 k=2"),
    "main_bf16": Workload("main_bf16", "bf16", H=16, c=128, d=128, N=16, topk=2, B=4, T=8192,
                          router_std=1.5,
                          notes="bf16, B=4 H=16 T=8192 c=d=128 N=16 k=2, router std 1.5"),
    "varlen_bf16": Workload("varlen_bf16", "bf16", H=16, c=128, d=128, N=32, topk=4,
                            varlen=(8, 1024, 16384),
                            notes="bf16 varlen, 8 seqs U[1024,16384], H=16 c=d=128 N=32 k=4"),
    "decode_bf16": Workload("decode_bf16", "bf16", H=16, c=128, d=128, N=16, topk=2, B=256,
                            decode_steps=64,
                            notes="decode, 256 seqs x H=16, c=d=128, N=16, k=2, 64 steps"),
}


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _as_f32(a: np.ndarray) -> np.ndarray:
    return a if a.dtype == np.float32 else bf16_bits_to_f32(a)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, -x)


def _tie_free_router(rng, shape, std, dtype) -> np.ndarray:
    z = _store(std * rng.standard_normal(shape), dtype)
    N = shape[-1]
    flat = z.reshape(-1, N)
    while True:
        srt = np.sort(_as_f32(flat), axis=1)
        bad = np.nonzero((srt[:, 1:] == srt[:, :-1]).any(axis=1))[0]
        if bad.size == 0:
            return z
        flat[bad] = _store(std * rng.standard_normal((bad.size, N)), dtype)


def token_inputs(rng, shape_prefix, w: Workload) -> dict:
    """q, key_logits, v, log_alpha, router_logits with leading dims shape_prefix."""
    sp = tuple(shape_prefix)
    out = {}
    out["q"] = _store(rng.standard_normal(sp + (w.H, w.c)), w.dtype)
    out["key_logits"] = _store(rng.standard_normal(sp + (w.H, w.c)), w.dtype)
    out["v"] = _store(rng.standard_normal(sp + (w.H, w.d)), w.dtype)
    out["log_alpha"] = _store(_logsigmoid(rng.standard_normal(sp + (w.H, w.c))) / 16.0, w.dtype)
    out["router_logits"] = _tie_free_router(rng, sp + (w.H, w.N), w.router_std, w.dtype)
    return out


def seq_lengths(w: Workload, rng=None) -> np.ndarray:
    if w.varlen:
        n, lo, hi = w.varlen
        rng = rng if rng is not None else np.random.default_rng(w.seed)
        return rng.integers(lo, hi + 1, n).astype(np.int64)
    return np.full(w.B, w.T, np.int64)


def forward_inputs(w: Workload, lengths=None, seed=None) -> dict:
    """Packed token-major inputs [T_tot, H, .] plus int32 cu_seqlens.

    ``lengths`` overrides the workload's sequence lengths (used for small
    parity cases that keep the workload's distributions)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if lengths is None:
        lengths = seq_lengths(w, rng) if w.varlen else np.full(w.B, w.T, np.int64)
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    out = token_inputs(rng, (T,), w)
    out["cu_seqlens"] = cu
    return out


def decode_states(w: Workload, b: int, seed=None) -> np.ndarray:
    """Initial fp32 states of decode sequence b: [H, N+1, c, d]."""
    rng = np.random.default_rng([w.seed if seed is None else seed, 4, b])
    s = rng.standard_normal((w.H, w.N + 1, w.c, w.d), dtype=np.float32)
    s *= np.float32(0.1)
    return s


def decode_inputs(w: Workload, steps=None, B=None, seed=None) -> dict:
    """Per-step token inputs [steps, B, H, .] (one token per sequence per step)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    steps = w.decode_steps if steps is None else steps
    B = w.B if B is None else B
    return token_inputs(rng, (steps, B), w)
