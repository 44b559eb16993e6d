"""Helpers shared by the GPU tests: move seeded numpy inputs to the device,
compare against the oracle, print the case being run."""
from __future__ import annotations

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
