"""Seeded input generator: determinism, tie-freeness, rounding, moments (CPU)."""
import numpy as np

import sse_inputs as si


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e-30, 65504.0], np.float32)
    bits = si.f32_to_bf16_bits(x)
    back = si.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[0] == 1.0 and back[3] == -2.5
    for v, b in zip(x, back):
        assert abs(float(b) - float(v)) <= abs(float(v)) * 2.0 ** -8 + 1e-45


def test_deterministic_and_tie_free():
    w = si.WORKLOADS["small_bf16"]
    a = si.forward_inputs(w, lengths=[300, 77])
    b = si.forward_inputs(w, lengths=[300, 77])
    for k in a:
        assert np.array_equal(a[k], b[k])
    z = si.bf16_bits_to_f32(a["router_logits"]).reshape(-1, w.N)
    srt = np.sort(z, axis=1)
    assert not (srt[:, 1:] == srt[:, :-1]).any()
    la = si.bf16_bits_to_f32(a["log_alpha"])
    assert (la <= 0).all() and la.mean() < -0.02


def test_varlen_lengths_and_cu():
    w = si.WORKLOADS["varlen_bf16"]
    lens = si.seq_lengths(w)
    assert len(lens) == 8 and lens.min() >= 1024 and lens.max() <= 16384


def test_decode_states_per_sequence():
    w = si.Workload("t", "bf16", H=2, c=4, d=4, N=3, topk=1, B=3)
    s0 = si.decode_states(w, 1)
    assert s0.shape == (2, 4, 4, 4) and s0.dtype == np.float32
    assert np.array_equal(s0, si.decode_states(w, 1))
    assert not np.array_equal(s0, si.decode_states(w, 2))
