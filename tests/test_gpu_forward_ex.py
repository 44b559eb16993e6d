"""GPU parity of the general forward (sse_forward_ex) against the fp64
oracle: the masked schedule, the shared partition's own query and key, and
read sets that differ from write sets.  Write and read top-k choices
bit-exact; o and final states within 5e-3 (bf16) / 1e-5 (fp32) of the
reference rms, every element; partitions that are neither written nor
(for states) touched keep their initial state bit for bit.  Outputs start
as NaN and the workspace as 0xff bytes."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sparse_state_linear_amd as sse
import sse_inputs as si
from gpu_util import (NAMES, TOL, announce, nan_like, oracle_threads, rel_err, rel_err_big,
                      sentinel_int, to_dev)

pytestmark = pytest.mark.gpu


def _extra_inputs(w, T, seed):
    """The shared partition's own q and key logits (N(0,1)) and read-set
    router logits (tie-free, like the write router's)."""
    rng = np.random.default_rng(seed)
    cast = (lambda x: x.astype(np.float32)) if w.dtype == "f32" else \
        (lambda x: si.f32_to_bf16_bits(x.astype(np.float32)))
    return {"q_sh": cast(rng.standard_normal((T, w.H, w.c))),
            "kl_sh": cast(rng.standard_normal((T, w.H, w.c))),
            "z_r": si._tie_free_router(rng, (T, w.H, w.N), 1.0, w.dtype)}


def _run(inp, w, schedule, extra=None, kr=None, init=None, own_shared=False, read_sets=False):
    d = {n: to_dev(inp[n]) for n in NAMES + ("cu_seqlens",)}
    cu = inp["cu_seqlens"]
    T, S = int(cu[-1]), len(cu) - 1
    max_len = int((cu[1:] - cu[:-1]).max()) if S else 0
    o = nan_like((T, w.H, w.d))
    fs = nan_like((S, w.H, w.N + 1, w.c, w.d))
    idx = sentinel_int((T, w.H, w.topk))
    ridx = sentinel_int((T, w.H, kr)) if read_sets else None
    nbytes = sse.sse_forward_ex_workspace_bytes(T, S, max_len, w.H, w.c, w.d, w.N, w.topk,
                                                kr if read_sets else 0)
    ws = torch.full((max(nbytes, 1),), 255, dtype=torch.uint8, device="cuda")
    kw = {}
    if own_shared:
        kw.update(q_shared=to_dev(extra["q_sh"]), key_logits_shared=to_dev(extra["kl_sh"]))
    if read_sets:
        kw.update(read_router_logits=to_dev(extra["z_r"]), read_topk=kr, read_topk_idx=ridx)
    init_d = None if init is None else torch.from_numpy(init).cuda()
    sse.sse_forward_ex(d["q"], d["key_logits"], d["v"], d["log_alpha"], d["router_logits"], w.N,
                       w.topk, d["cu_seqlens"], max_len, init_d, schedule=schedule, o=o,
                       final_states=fs, topk_idx=idx, workspace=ws, **kw)
    torch.cuda.synchronize()
    return {"o": o.cpu().numpy(), "fs": fs.cpu().numpy(), "idx": idx.cpu().numpy(),
            "ridx": None if ridx is None else ridx.cpu().numpy()}


def _oracle_ex(inp, w, extra=None, kr=None, init=None, own_shared=False, read_sets=False):
    """oracle.forward_ex per (sequence, head) unit on host threads."""
    cu = inp["cu_seqlens"]
    S, T = len(cu) - 1, int(cu[-1])
    kk = kr if read_sets else w.topk
    out = {"o": np.zeros((T, w.H, w.d)), "final_states": np.zeros((S, w.H, w.N + 1, w.c, w.d)),
           "write_idx": np.zeros((T, w.H, w.topk), np.int32),
           "read_idx": np.zeros((T, w.H, kk), np.int32)}

    def unit(sh):
        s, h = divmod(sh, w.H)
        sl = slice(int(cu[s]), int(cu[s + 1]))
        sub = lambda a: None if a is None else np.ascontiguousarray(a[sl, h:h + 1])
        r = oracle.forward_ex(
            *(sub(inp[n]) for n in NAMES), np.array([0, sl.stop - sl.start], np.int32), w.N,
            w.topk, q_shared=sub(extra["q_sh"]) if own_shared else None,
            key_logits_shared=sub(extra["kl_sh"]) if own_shared else None,
            read_router_logits=sub(extra["z_r"]) if read_sets else None, read_topk=kr,
            initial_states=None if init is None else init[s, h][None, None].astype(np.float64))
        out["o"][sl, h] = r["o"][:, 0]
        out["final_states"][s, h] = r["final_states"][0, 0]
        out["write_idx"][sl, h] = r["write_idx"][:, 0]
        out["read_idx"][sl, h] = r["read_idx"][:, 0]

    with ThreadPoolExecutor(oracle_threads()) as ex:
        list(ex.map(unit, range(S * w.H)))
    return out


def _check(w, lengths, schedule, seed, kr=None, init=None, own_shared=False, read_sets=False,
           inp=None, big=False):
    if inp is None:
        inp = si.forward_inputs(w, lengths=lengths, seed=seed)
    T = int(inp["cu_seqlens"][-1])
    extra = _extra_inputs(w, T, seed + 7)
    announce(w.name, schedule, "lengths", lengths if len(lengths) < 12 else len(lengths), "N",
             w.N, "k", w.topk, "kr", kr, "own_shared", own_shared, "read_sets", read_sets,
             "sse_forward_ex")
    got = _run(inp, w, schedule, extra, kr, init, own_shared, read_sets)
    ref = _oracle_ex(inp, w, extra, kr, init, own_shared, read_sets)
    assert np.array_equal(got["idx"], ref["write_idx"]), "write top-k differs"
    if read_sets:
        assert np.array_equal(got["ridx"], ref["read_idx"]), "read top-k differs"
    err = rel_err_big if big else rel_err
    eo, es = err(got["o"], ref["o"]), err(got["fs"], ref["final_states"])
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}  (tol {TOL[w.dtype]})", flush=True)
    assert np.isfinite(got["o"]).all() and np.isfinite(got["fs"]).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)
    return got, ref


# ------------------------------------------------------------ masked schedule
@pytest.mark.parametrize("dtype,H,cd,N,k", [("bf16", 2, 128, 16, 2), ("bf16", 3, 64, 8, 3),
                                           ("bf16", 2, 32, 64, 8), ("bf16", 2, 128, 1, 1),
                                           ("bf16", 5, 64, 6, 6), ("f32", 2, 32, 4, 1),
                                           ("f32", 3, 64, 8, 2)])
def test_masked_schedule(dtype, H, cd, N, k):
    w = si.Workload(f"masked_{dtype}_n{N}k{k}", dtype, H=H, c=cd, d=cd, N=N, topk=k,
                    router_std=1.5)
    lengths = [700, 130, 0, 1, 65]
    rng = np.random.default_rng(500 + N)
    init = (0.5 * rng.standard_normal((len(lengths), H, N + 1, cd, cd))).astype(np.float32)
    _check(w, lengths, "masked", seed=501 + N + k, init=init)


def test_masked_schedule_pieces():
    """Sequences of several shared pieces, 1024-token pieces (many units)."""
    w = si.Workload("masked_pieces", "bf16", H=16, c=32, d=32, N=8, topk=2)
    rng = np.random.default_rng(510)
    lengths = [int(x) for x in rng.integers(2050, 2600, 16)]
    init = (0.5 * rng.standard_normal((16, w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    _check(w, lengths, "masked", seed=511, init=init)


def test_masked_unselected_partition_keeps_state():
    w = si.Workload("masked_unsel", "bf16", H=2, c=64, d=64, N=8, topk=2)
    lengths = [300, 90]
    inp = si.forward_inputs(w, lengths=lengths, seed=520)
    z = si.bf16_bits_to_f32(inp["router_logits"]).copy()
    z[..., 5] = -30.0
    inp["router_logits"] = si.f32_to_bf16_bits(z)
    init = np.random.default_rng(521).standard_normal((2, w.H, w.N + 1, w.c, w.d)).astype(np.float32)
    got, _ = _check(w, lengths, "masked", seed=0, init=init, inp=inp)
    assert np.array_equal(got["fs"][:, :, 5].view(np.uint32), init[:, :, 5].view(np.uint32))


def test_masked_main_full_size():
    """The main workload (B=4, H=16, T=8192, c=d=128, N=16, k=2) on the
    masked schedule, every unit."""
    w = si.WORKLOADS["main_bf16"]
    inp = si.forward_inputs(w)
    got = _run(inp, w, "masked")
    ref = oracle.forward(*(inp[n] for n in NAMES), inp["cu_seqlens"], w.N, w.topk,
                         threads=oracle_threads())
    announce("main_bf16 masked full size")
    assert np.array_equal(got["idx"], ref["topk_idx"])
    eo, es = rel_err_big(got["o"], ref["o"]), rel_err_big(got["fs"], ref["final_states"])
    print(f"  o rel err {eo:.3e}  states rel err {es:.3e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


# ------------------------------------- the shared partition's own query/key
@pytest.mark.parametrize("schedule", ["varlen", "masked"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_own_shared_query_key(schedule, dtype):
    w = si.Workload(f"own_shared_{dtype}", dtype, H=3, c=128 if dtype == "bf16" else 64,
                    d=128 if dtype == "bf16" else 64, N=8, topk=2)
    lengths = [1200, 77, 1, 300]
    rng = np.random.default_rng(530)
    init = (0.5 * rng.standard_normal((len(lengths), w.H, w.N + 1, w.c, w.d))).astype(np.float32)
    _check(w, lengths, schedule, seed=531, init=init, own_shared=True)


# ----------------------------------------------------------------- read sets
@pytest.mark.parametrize("dtype,N,k,kr", [("bf16", 16, 2, 3), ("bf16", 8, 3, 1),
                                          ("bf16", 6, 2, 6), ("f32", 8, 2, 4), ("f32", 4, 1, 1)])
def test_read_sets(dtype, N, k, kr):
    w = si.Workload(f"rsets_{dtype}_n{N}k{k}r{kr}", dtype, H=2, c=64, d=64, N=N, topk=k)
    lengths = [500, 33, 1]
    rng = np.random.default_rng(540 + kr)
    init = (0.5 * rng.standard_normal((len(lengths), w.H, N + 1, w.c, w.d))).astype(np.float32)
    _check(w, lengths, "masked", seed=541 + N, kr=kr, init=init, read_sets=True)


def test_read_sets_with_own_shared_query_key():
    w = si.Workload("rsets_own", "bf16", H=4, c=128, d=128, N=16, topk=2)
    _check(w, [900, 200], "masked", seed=550, kr=4, own_shared=True, read_sets=True)


def test_read_only_partition():
    """A partition read at every token but never written: its state stays
    the initial one bit for bit (identity transition) while the reads use
    it."""
    w = si.Workload("read_only", "bf16", H=2, c=64, d=64, N=8, topk=2)
    lengths = [300, 40]
    inp = si.forward_inputs(w, lengths=lengths, seed=560)
    z = si.bf16_bits_to_f32(inp["router_logits"]).copy()
    z[..., 3] = -30.0
    inp["router_logits"] = si.f32_to_bf16_bits(z)
    T = sum(lengths)
    extra = _extra_inputs(w, T, 561)
    zr = si.bf16_bits_to_f32(extra["z_r"]).copy()
    zr[..., 3] = 30.0
    extra["z_r"] = si.f32_to_bf16_bits(zr)
    init = np.random.default_rng(562).standard_normal((2, w.H, w.N + 1, w.c, w.d)).astype(np.float32)
    announce("read-only partition", "sse_forward_ex masked")
    got = _run(inp, w, "masked", extra, 2, init, read_sets=True)
    ref = _oracle_ex(inp, w, extra, 2, init, read_sets=True)
    assert (got["ridx"][..., 0] == 3).all()
    assert np.array_equal(got["fs"][:, :, 3].view(np.uint32), init[:, :, 3].view(np.uint32))
    assert rel_err(got["o"], ref["o"]) <= TOL["bf16"]
    assert rel_err(got["fs"], ref["final_states"]) <= TOL["bf16"]
