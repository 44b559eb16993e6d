"""The oracle's threaded path (a work queue of (sequence, head) units over
pthreads) gives the same bits as the single-threaded path, which the pins
check against the page's formulas (CPU).  The GPU parity tests and the CPU
baseline run the threaded path."""
import numpy as np
import pytest

import oracle
import sse_inputs as si

NAMES = ("q", "key_logits", "v", "log_alpha", "router_logits")


@pytest.mark.parametrize("dtype,H,c,d,N,k,lengths", [
    ("bf16", 3, 16, 8, 8, 2, [200, 0, 1, 77, 130]),
    ("f32", 2, 8, 16, 5, 5, [64, 65, 3]),
    ("bf16", 5, 8, 8, 1, 1, [300, 31]),
])
@pytest.mark.parametrize("threads", [2, 7, 16])
def test_threaded_forward_is_bitwise_single(dtype, H, c, d, N, k, lengths, threads):
    w = si.Workload("thr", dtype, H=H, c=c, d=d, N=N, topk=k)
    inp = si.forward_inputs(w, lengths=lengths, seed=threads)
    init = np.random.default_rng(threads).standard_normal((len(lengths), H, N + 1, c, d))
    for ini in (None, init):
        one = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], N, k,
                             initial_states=ini, threads=1)
        many = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], N, k,
                              initial_states=ini, threads=threads)
        for key in one:
            assert np.array_equal(one[key].view(np.uint8), many[key].view(np.uint8)), key
