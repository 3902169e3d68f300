"""The C-ABI library loads and exports every function include/wsg.h declares.

No compute calls: only argument checks that return before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wsg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def wsg():
    import warp_specialized_gemm_amd as w
    return w


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ("gemm_bias_relu", "gemm_bias_relu_bf16", "staged_copy", "gemm_bias_relu_ex", "staged_copy_ex",
              "wsg_set_stream", "wsg_last_error", "wsg_check_device_status"):
        assert n in names


def test_library_exports_every_declared_symbol(wsg):
    names = declared_functions()
    assert sorted(wsg.EXPORTS) == names
    out = subprocess.run(["nm", "-D", "--defined-only", wsg.library_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(wsg.lib, n)


def test_library_is_gfx950_code(wsg):
    data = open(wsg.library_path(), "rb").read()
    assert b"gfx950" in data


def test_version(wsg):
    assert "gfx950" in wsg.version()


def test_invalid_arguments_rejected_before_any_device_call(wsg):
    L = wsg.lib
    nul = None
    # negative dimension
    assert L.gemm_bias_relu(-1, 4, 4, nul, nul, nul, nul, 2) == wsg.WSG_EINVAL
    assert "negative" in wsg.last_error()
    # stages < 1
    assert L.gemm_bias_relu(4, 4, 4, 16, 16, 16, 16, 0) == wsg.WSG_EINVAL
    # null operands with nonzero sizes
    assert L.gemm_bias_relu(4, 4, 4, nul, nul, nul, nul, 2) == wsg.WSG_EINVAL
    # misaligned fp32 operand
    assert L.gemm_bias_relu(4, 4, 4, 0x1002, 0x2000, 0x3000, 0x40000, 2) == wsg.WSG_EINVAL
    # C overlapping A
    assert L.gemm_bias_relu(4, 4, 4, 0x10000, 0x20000, 0x30000, 0x10010, 2) == wsg.WSG_EINVAL
    assert "overlap" in wsg.last_error()
    # dtype code
    assert L.gemm_bias_relu_ex(7, 4, 4, 4, 0x10000, 0x20000, 0x30000, 0x40000, 2, None) == wsg.WSG_EINVAL
    # dimensions beyond 31 bits
    assert L.gemm_bias_relu(1 << 31, 4, 4, 0x10000, 0x20000, 0x30000, 0x40000, 2) == wsg.WSG_EUNSUPPORTED
    # empty problems are no-ops that succeed
    assert L.gemm_bias_relu(0, 4, 4, nul, nul, nul, nul, 2) == wsg.WSG_OK
    assert L.gemm_bias_relu(4, 0, 4, nul, nul, nul, nul, 2) == wsg.WSG_OK
    # copy: zero bytes, null, misaligned, overlapping, stages
    assert L.staged_copy(nul, nul, 0, 2) == wsg.WSG_OK
    assert L.staged_copy(nul, 0x1000, 16, 2) == wsg.WSG_EINVAL
    assert L.staged_copy(0x1008, 0x2000, 16, 2) == wsg.WSG_EINVAL
    assert L.staged_copy(0x1000, 0x1010, 64, 2) == wsg.WSG_EINVAL
    assert "overlap" in wsg.last_error()
    assert L.staged_copy(0x1000, 0x9000, 64, 0) == wsg.WSG_EINVAL


def test_grouped_and_attention_arguments_rejected_before_any_device_call(wsg):
    L = wsg.lib
    rows = lambda *r: (ctypes.c_int64 * max(1, len(r)))(*r)  # noqa: E731
    A, B, b, C = 0x100000, 0x200000, 0x300000, 0x400000
    g = L.grouped_gemm_bias_relu_ex
    assert g(wsg.WSG_FP32, 0, rows(), 8, 16, A, B, b, C, 2, None) == wsg.WSG_EINVAL
    assert g(wsg.WSG_FP32, wsg.WSG_MAX_GROUPS + 1, rows(*[1] * 65), 8, 16, A, B, b, C, 2, None) == \
        wsg.WSG_EUNSUPPORTED
    assert g(wsg.WSG_FP32, 2, None, 8, 16, A, B, b, C, 2, None) == wsg.WSG_EINVAL
    assert g(wsg.WSG_FP32, 2, rows(3, -1), 8, 16, A, B, b, C, 2, None) == wsg.WSG_EINVAL
    assert g(wsg.WSG_FP32, 2, rows(3, 1), 8, 16, A, B, b, C, 0, None) == wsg.WSG_EINVAL
    assert g(7, 2, rows(3, 1), 8, 16, A, B, b, C, 2, None) == wsg.WSG_EINVAL
    # C inside the second expert's block of B (2 x 16 x 8 floats from B)
    assert g(wsg.WSG_FP32, 2, rows(3, 1), 8, 16, A, B, b, B + 16 * 8 * 4 + 64, 2, None) == wsg.WSG_EINVAL
    assert "overlap" in wsg.last_error()
    # no rows, or no columns: nothing to do
    assert g(wsg.WSG_FP32, 3, rows(0, 0, 0), 8, 16, None, None, None, None, 2, None) == wsg.WSG_OK
    assert g(wsg.WSG_FP32, 2, rows(3, 1), 0, 16, None, None, None, None, 2, None) == wsg.WSG_OK

    a = L.attention_fwd
    Q, K, V, O = 0x100000, 0x200000, 0x300000, 0x400000
    assert a(-1, 1, 4, 4, 128, Q, K, V, O, 1.0, 0, 2, None) == wsg.WSG_EINVAL
    assert a(1, 1, 4, 4, 96, Q, K, V, O, 1.0, 0, 2, None) == wsg.WSG_EUNSUPPORTED
    assert a(1, 1, 4, 4, 128, Q, K, V, O, float("nan"), 0, 2, None) == wsg.WSG_EINVAL
    assert a(1, 1, 4, 4, 128, Q, K, V, O, float("inf"), 0, 2, None) == wsg.WSG_EINVAL
    # the scale must be positive and normal: zero, negative and subnormal scales are refused
    for bad in (0.0, -0.0, -1.0, 1e-40, -float("inf")):
        assert a(1, 1, 4, 4, 128, Q, K, V, O, bad, 0, 2, None) == wsg.WSG_EINVAL, bad
    assert "scale" in wsg.last_error()
    assert a(1, 1, 4, 4, 128, Q, K, V, O, 1.0, 0, 0, None) == wsg.WSG_EINVAL
    assert a(1, 1, 4, 4, 128, None, K, V, O, 1.0, 0, 2, None) == wsg.WSG_EINVAL
    assert a(1, 1, 4, 4, 128, Q + 2, K, V, O, 1.0, 0, 2, None) == wsg.WSG_EINVAL  # Q not 16-byte aligned
    assert a(1, 1, 4, 4, 128, Q, K, V, Q + 64, 1.0, 0, 2, None) == wsg.WSG_EINVAL  # O overlaps Q
    assert "overlap" in wsg.last_error()
    assert a(1, 1 << 31, 4, 4, 128, Q, K, V, O, 1.0, 0, 2, None) == wsg.WSG_EUNSUPPORTED
    # no heads or no queries: nothing to do; no keys needs no K or V
    assert a(0, 4, 4, 4, 128, None, None, None, None, 1.0, 0, 2, None) == wsg.WSG_OK
    assert a(1, 4, 0, 4, 128, None, None, None, None, 1.0, 1, 2, None) == wsg.WSG_OK


def test_stream_is_thread_local(wsg):
    import threading
    wsg.lib.wsg_set_stream(ctypes.c_void_p(0x1234))
    seen = []
    t = threading.Thread(target=lambda: seen.append(wsg.lib.wsg_get_stream()))
    t.start()
    t.join()
    assert wsg.lib.wsg_get_stream() == 0x1234
    assert seen == [None]
    wsg.lib.wsg_set_stream(None)
    assert wsg.lib.wsg_get_stream() is None


def test_config_struct_layout_matches_header(wsg):
    text = open(HEADER).read()
    body = re.search(r"typedef struct wsg_config \{(.*?)\} wsg_config;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"([A-Za-z_]+)\s*[,;]", body)
    assert fields == [f for f, _ in wsg.Config._fields_]
    assert ctypes.sizeof(wsg.Config) == 4 * len(fields)


def test_binding_constants_match_header(wsg):
    """Every WSG_* constant of the header has the same value in the binding."""
    text = open(HEADER).read()
    defs = dict(re.findall(r"^#define\s+(WSG_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", text, flags=re.M))
    assert {"WSG_OK", "WSG_EINVAL", "WSG_FP32", "WSG_BF16", "WSG_FLAG_HOMOGENEOUS"} <= set(defs)
    for name, value in defs.items():
        assert getattr(wsg, name) == int(value), name


def test_status_message_names_every_kernel(wsg):
    """Each kernel bit of the status word appears in the timeout message (host-only call)."""
    T = wsg.WSG_STATUS_TIMEOUT
    assert "no ring flag wait gave up" in wsg.status_message(0)
    for bit, name in ((wsg.WSG_STATUS_COPY, "staged_copy"), (wsg.WSG_STATUS_GEMM, "gemm"),
                      (wsg.WSG_STATUS_ATTENTION, "attention")):
        msg = wsg.status_message(T | bit)
        assert name in msg and "gave up" in msg, msg
    msg = wsg.status_message(T | wsg.WSG_STATUS_COPY | wsg.WSG_STATUS_GEMM | wsg.WSG_STATUS_ATTENTION)
    assert "staged_copy" in msg and "gemm" in msg and "attention" in msg
    assert "unnamed" in wsg.status_message(T)
