"""GPU parity of the row-sparse top-k key variant (sse_rowsparse_forward)
against the fp64 oracle: every element of o and the final states, within
5e-3 (bf16 inputs) / 1e-5 (fp32 inputs) of the reference rms; rows that are
never selected keep their initial state bit for bit (identity transition).
Outputs start as NaN and the workspace as 0xff bytes."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import TOL, announce, nan_like, oracle_threads, rel_err, rel_err_big, to_dev

pytestmark = pytest.mark.gpu
NAMES4 = ("q", "key_logits", "v", "log_alpha")


def _run(inp, w, k, identity, init=None):
    d = {n: to_dev(inp[n]) for n in NAMES4 + ("cu_seqlens",)}
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max()) if S else 0
    o = nan_like((T, w.H, w.d))
    fs = nan_like((S, w.H, w.c, w.d))
    nbytes = sse.sse_rowsparse_workspace_bytes(T, S, max_len, w.H, w.c, w.d)
    ws = torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device="cuda")
    init_d = None if init is None else torch.from_numpy(init).cuda()
    sse.sse_rowsparse_forward(d["q"], d["key_logits"], d["v"], d["log_alpha"], k,
                              d["cu_seqlens"], max_len, init_d, identity, o=o, final_states=fs,
                              workspace=ws)
    torch.cuda.synchronize()
    return o.cpu().numpy(), fs.cpu().numpy()


def _oracle(inp, w, k, identity, init=None):
    """The oracle per (sequence, head) unit on host threads."""
    cu = inp["cu_seqlens"]
    S = len(cu) - 1
    T = int(cu[-1])
    o = np.zeros((T, w.H, w.d))
    fs = np.zeros((S, w.H, w.c, w.d))

    def unit(sh):
        s, h = divmod(sh, w.H)
        sl = slice(int(cu[s]), int(cu[s + 1]))
        sub = {n: np.ascontiguousarray(inp[n][sl, h:h + 1]) for n in NAMES4}
        ini = None if init is None else init[s, h][None, None].astype(np.float64)
        r = oracle.rowsparse_forward(*(sub[n] for n in NAMES4),
                                     np.array([0, sl.stop - sl.start], np.int32), k, identity, ini)
        o[sl, h] = r["o"][:, 0]
        fs[s, h] = r["final_states"][0, 0]

    with ThreadPoolExecutor(oracle_threads()) as ex:
        list(ex.map(unit, range(S * w.H)))
    return o, fs


def _check(w, lengths, k, identity, seed, init=None, inp=None, big=False):
    if inp is None:
        inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    announce(w.name, "lengths", lengths if len(lengths) < 12 else f"{len(lengths)} seqs", "k", k,
             "identity", identity, "sse_rowsparse_forward")
    o, fs = _run(inp, w, k, identity, init)
    ro, rfs = _oracle(inp, w, k, identity, init)
    err = rel_err_big if big else rel_err
    eo, es = err(o, ro), err(fs, rfs)
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}  (tol {TOL[w.dtype]})", flush=True)
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)
    return inp, o, fs


@pytest.mark.parametrize("k", [1, 32, 128])
@pytest.mark.parametrize("identity", [True, False])
def test_rowsparse_bf16(k, identity):
    w = si.Workload(f"rowsparse_bf16_k{k}", "bf16", H=3, c=128, d=128, N=1, topk=1)
    rng = np.random.default_rng(200 + k)
    lengths = [700, 130, 0, 1]
    init = (0.5 * rng.standard_normal((len(lengths), w.H, w.c, w.d))).astype(np.float32)
    _check(w, lengths, k, identity, seed=201 + k, init=init)


@pytest.mark.parametrize("c,d,k", [(32, 32, 1), (64, 32, 8), (32, 128, 32), (128, 64, 16)])
@pytest.mark.parametrize("identity", [True, False])
def test_rowsparse_f32(c, d, k, identity):
    w = si.Workload(f"rowsparse_f32_{c}x{d}", "f32", H=2, c=c, d=d, N=1, topk=1)
    rng = np.random.default_rng(210 + k)
    lengths = [300, 17, 64]
    init = (0.5 * rng.standard_normal((len(lengths), w.H, c, d))).astype(np.float32)
    _check(w, lengths, k, identity, seed=211 + c + k, init=init)


@pytest.mark.parametrize("n_seq,H", [(2, 2), (16, 16)])
def test_rowsparse_pieces(n_seq, H):
    """Chains of several shared pieces (256-token pieces with few units,
    1024-token pieces with many), random initial states."""
    w = si.Workload(f"rowsparse_pieces_{n_seq}", "bf16", H=H, c=32 if H > 2 else 128,
                    d=32 if H > 2 else 128, N=1, topk=1)
    rng = np.random.default_rng(220 + n_seq)
    lengths = [int(x) for x in rng.integers(2050, 2600, n_seq)]
    init = (0.5 * rng.standard_normal((n_seq, H, w.c, w.d))).astype(np.float32)
    _check(w, lengths, w.c // 4, True, seed=221, init=init)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rowsparse_tied_key_logits(dtype):
    """Integer-valued key logits in [-2, 2]: the k-th largest value is tied
    in most rows, and the lower rows must win, as in the oracle.  Half the
    zeros are -0, which ties with +0."""
    w = si.Workload(f"rowsparse_ties_{dtype}", dtype, H=2, c=64, d=64, N=1, topk=1)
    lengths = [400, 33]
    inp = si.forward_inputs(w, lengths=lengths, seed=230)
    rng = np.random.default_rng(231)
    kl = rng.integers(-2, 3, inp["key_logits"].shape).astype(np.float32)
    kl[(kl == 0) & (rng.random(kl.shape) < 0.5)] = -0.0
    assert np.signbit(kl[kl == 0]).any()
    inp["key_logits"] = si.f32_to_bf16_bits(kl) if dtype == "bf16" else kl
    for k in (5, 16):
        _check(w, lengths, k, True, seed=0, inp=inp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rowsparse_strong_decay(dtype):
    """log_alpha = -1.24 on every row (the masked decay of 64 consecutive
    tokens stays above -80)."""
    w = si.Workload(f"rowsparse_decay_{dtype}", dtype, H=2, c=128, d=128, N=1, topk=1)
    lengths = [600, 70]
    inp = si.forward_inputs(w, lengths=lengths, seed=240)
    la = np.full(inp["log_alpha"].shape, -1.24, np.float32)
    inp["log_alpha"] = si.f32_to_bf16_bits(la) if dtype == "bf16" else la
    _check(w, lengths, 32, True, seed=0, inp=inp)
    _check(w, lengths, 32, False, seed=0, inp=inp)


def test_rowsparse_unselected_rows_keep_initial_state():
    w = si.Workload("rowsparse_unsel", "bf16", H=2, c=64, d=64, N=1, topk=1)
    lengths = [300, 50]
    inp = si.forward_inputs(w, lengths=lengths, seed=250)
    kl = si.bf16_bits_to_f32(inp["key_logits"]).copy()
    kl[..., :4] = -30.0
    inp["key_logits"] = si.f32_to_bf16_bits(kl)
    init = np.random.default_rng(251).standard_normal((2, w.H, w.c, w.d)).astype(np.float32)
    _, _, fs = _check(w, lengths, 16, True, seed=0, init=init, inp=inp)
    assert np.array_equal(fs[:, :, :4].view(np.uint32), init[:, :, :4].view(np.uint32))


def test_rowsparse_run_twice_bitwise():
    w = si.Workload("rowsparse_twice", "bf16", H=4, c=128, d=128, N=1, topk=1)
    inp = si.forward_inputs(w, lengths=[1500, 200], seed=260)
    announce("rowsparse run twice")
    a = _run(inp, w, 32, True)
    b = _run(inp, w, 32, True)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_rowsparse_main_shape_full_size():
    """The benchmark's row-sparse workload: B=4, H=16, T=8192, c=d=128,
    k = 32 of 128 rows (k = c/4, the setting of the page's MQAR study),
    identity transition on unselected rows; every unit compared."""
    w = si.Workload("rowsparse_main", "bf16", H=16, c=128, d=128, N=1, topk=1, B=4, T=8192)
    _check(w, [8192] * 4, 32, True, seed=0, big=True)
