"""Helpers shared by the GPU tests: move seeded numpy inputs to the device,
compare against the oracle, print the case being run."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

NAMES = ("q", "key_logits", "v", "log_alpha", "router_logits")


def announce(*parts):
    """Name the case (test, seed, shape, entry point) before a GPU step."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dev="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def rel_err(got, ref) -> float:
    """max |got - ref| / rms(ref), computed in fp64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


TOL = {"f32": 1e-5, "bf16": 5e-3}


def oracle_threads() -> int:
    """Host threads for the oracle (the box gives a GPU job 16 cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def rel_err_big(got, ref, chunk=1 << 24) -> float:
    """rel_err over large arrays, in chunks (fp64 temporaries stay small)."""
    g = np.asarray(got).reshape(-1)
    r = np.asarray(ref).reshape(-1)
    if r.size == 0:
        return 0.0
    mx, ss = 0.0, 0.0
    for i in range(0, r.size, chunk):
        rr = r[i:i + chunk].astype(np.float64)
        gg = g[i:i + chunk].astype(np.float64)
        mx = max(mx, float(np.max(np.abs(gg - rr))))
        ss += float(np.dot(rr, rr))
    rms = (ss / r.size) ** 0.5
    return mx / max(rms, 1e-300)


def nan_like(shape, dev="cuda"):
    """fp32 output buffer pre-filled with NaN: an element the kernels never
    write stays NaN and fails every comparison."""
    return torch.full(shape, float("nan"), dtype=torch.float32, device=dev)


def sentinel_int(shape, dev="cuda"):
    return torch.full(shape, -7, dtype=torch.int32, device=dev)
