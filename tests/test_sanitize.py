"""AddressSanitizer + UndefinedBehaviorSanitizer runs of the host code (CPU).

* The fp64 oracle (plain C) is rebuilt with gcc -fsanitize=address,undefined
  and driven through its whole API (varlen forward single- and
  multi-threaded, units, decode steps, grouping) on edge cases: empty and
  length-1 sequences, N = 1, k = N, initial states.  Its outputs must match
  the regular build bit for bit.
* The C-ABI layer (sse_api.hip: argument checks, workspace carving, status
  paths) is rebuilt host-only with the sanitizers (-Xarch_host) and linked
  against launcher stubs (tests/sanitize/abi_stubs.cpp), then every entry
  point is called with arguments its checks must reject and with sizes that
  overflow the 32-bit indexing.
Each run happens in a child process with the sanitizer runtime preloaded;
any report aborts it with a non-zero status.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run_child(script, env_extra, tmp_path):
    path = tmp_path / "child.py"
    path.write_text(script)
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT + os.pathsep + os.path.join(ROOT, "tests")
    r = subprocess.run([sys.executable, str(path)], env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return r.stdout


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    import oracle
    so = str(tmp_path / "libsse_oracle_asan.so")
    oracle.build(out=so, extra_flags=("-g", "-O1", "-fno-omit-frame-pointer",
                                      "-fsanitize=address,undefined",
                                      "-fno-sanitize-recover=all"))
    script = textwrap.dedent(f"""
        import numpy as np
        import oracle
        import sse_inputs as si
        asan = oracle.load({so!r})
        plain = oracle.load()
        names = ("q", "key_logits", "v", "log_alpha", "router_logits")
        cases = [("f32", 1, 1, [5, 0, 1, 9]), ("bf16", 4, 4, [33, 2]), ("bf16", 6, 2, [0]),
                 ("f32", 5, 3, [17, 1, 0, 40])]
        for n, (dt, N, k, lens) in enumerate(cases):
            w = si.Workload("asan", dt, H=2, c=8, d=6, N=N, topk=k)
            inp = si.forward_inputs(w, lengths=lens, seed=n)
            S = len(lens)
            init = np.random.default_rng(n).standard_normal((S, 2, N + 1, 8, 6))
            for threads in (1, 3):
                for ini in (None, init):
                    a = oracle.forward(*(inp[x] for x in names), inp["cu_seqlens"], N, k,
                                       initial_states=ini, threads=threads, lib=asan)
                    b = oracle.forward(*(inp[x] for x in names), inp["cu_seqlens"], N, k,
                                       initial_states=ini, threads=1, lib=plain)
                    for key in a:
                        assert np.array_equal(a[key], b[key]), key
            if sum(lens):
                o, S1, i1, e1 = oracle.unit(*(inp[x] for x in names), 0, lens[0], 1, N, k, lib=asan)
                g = oracle.group(a["topk_idx"], inp["cu_seqlens"], N, lib=asan)
                st = np.zeros((1, 2, N + 1, 8, 6))
                tok = {{x: np.ascontiguousarray(inp[x][:1]) for x in names}}
                oracle.decode_step(*(tok[x] for x in names), st, N, k, lib=asan)
        print("oracle sanitizer run ok")
    """)
    out = _run_child(script, {"LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                              "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, tmp_path)
    assert "oracle sanitizer run ok" in out


def _clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "libsse_api_asan.so")
    csrc = os.path.join(ROOT, "sparse_state_linear_amd", "csrc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "sse_api.hip"), os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
           "-o", so]
    subprocess.run(cmd, check=True, capture_output=True)
    script = textwrap.dedent(f"""
        import ctypes
        import abi_calls
        L = ctypes.CDLL({so!r})
        n = abi_calls.exercise(L)
        print("abi sanitizer run ok", n)
    """)
    out = _run_child(script, {"LD_PRELOAD": rt, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                              "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}, tmp_path)
    assert "abi sanitizer run ok" in out
