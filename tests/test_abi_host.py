"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sse.h, and rejects bad arguments on the host before any
launch (every call below returns before its first HIP call)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest  # noqa: F401

import sparse_state_linear_amd as sse

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sse.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sse_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sse.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"libsse_amd.so does not export {n}"
    assert set(names) == set(sse.EXPORTED)


def test_status_strings_and_version():
    for code in range(5):
        assert sse.status_string(code).startswith("SSE_")
    assert sse.status_string(99) == "SSE_ERR_UNKNOWN"
    assert sse.lib().sse_version() >= 100


def test_workspace_queries():
    ws = sse.sse_forward_workspace_bytes(32768, 4, 8192, 16, 128, 128, 16, 2)
    assert ws >= 4 * 32768 * 16 * 2 * 4 and ws % 256 == 0
    assert sse.sse_forward_workspace_bytes(100, 1, 100, 1, 48, 32, 4, 1) == 0   # c unsupported
    assert sse.sse_forward_workspace_bytes(100, 1, 100, 1, 32, 32, 4, 5) == 0   # topk > N
    assert sse.sse_forward_workspace_bytes(-1, 1, 100, 1, 32, 32, 4, 1) == 0
    assert sse.sse_group_workspace_bytes(100, 1, 100, 2, 4, 1) > 0
    assert sse.sse_group_workspace_bytes(100, 1, 100, 2, 65, 1) == 0


def test_host_checks_reject_bad_arguments():
    """Every rejection case of tests/abi_calls.py returns its status (the same
    battery runs under the sanitizers in test_sanitize.py)."""
    import abi_calls
    assert abi_calls.exercise(sse.lib()) > 40


def test_debug_mode_switch():
    """The debug-mode switch touches no device: set, query and restore it in
    this process; the environment variable sets the mode of a fresh one."""
    before = sse.sse_debug_checks()
    try:
        assert sse.sse_debug_checks(True) is True
        assert sse.sse_debug_checks() is True
        assert sse.sse_debug_checks(False) is False
        assert sse.sse_debug_checks() is False
    finally:
        sse.sse_debug_checks(before)
    code = "import sparse_state_linear_amd as s; print(int(s.sse_debug_checks()))"
    for val, want in (("1", "1"), ("0", "0"), ("", "0")):
        env = dict(os.environ, SSE_DEBUG_CHECKS=val, PYTHONPATH=ROOT)
        out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                             text=True, check=True, timeout=300)
        assert out.stdout.strip().splitlines()[-1] == want


def test_product_path_does_not_touch_the_oracle():
    """The HIP binding must not import, load or call the oracle."""
    pkg = os.path.join(ROOT, "sparse_state_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_binding_constants_match_header():
    """Status, dtype and schedule codes of the binding equal the header's."""
    text = open(HEADER).read()
    for name, val in (("SSE_SCHEDULE_VARLEN", sse.SSE_SCHEDULE_VARLEN),
                      ("SSE_SCHEDULE_MASKED", sse.SSE_SCHEDULE_MASKED),
                      ("SSE_F32", sse.SSE_F32), ("SSE_BF16", sse.SSE_BF16),
                      ("SSE_ERR_WORKSPACE", sse.SSE_ERR_WORKSPACE)):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == val, name
    assert sse.SCHEDULES == {"varlen": sse.SSE_SCHEDULE_VARLEN, "masked": sse.SSE_SCHEDULE_MASKED}
