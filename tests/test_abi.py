"""The C ABI library, on the host: it loads, exports every entry point its
header declares, and the host-side checks return the documented errors.
No call here reaches the GPU."""

import ctypes
import os
import re

import pytest

import markov_draft_sampling_step_amd as m

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "markov.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.LIBRARY):
        from markov_draft_sampling_step_amd import build

        build.build()
    return m.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(markov_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("markov_sample_sequential", "markov_workspace_bytes", "markov_workspace_init",
                     "markov_why_not", "markov_status_string", "markov_debug_bias"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    handle = ctypes.CDLL(m.LIBRARY)
    missing = [n for n in declared_functions() if not hasattr(handle, n)]
    assert not missing, missing


def test_status_strings(lib):
    assert m.status_string(0) == "ok"
    for code in m.ERRORS:
        assert m.status_string(code) != "unknown status"


def test_max_rows_and_workspace(lib):
    # LDS-bound at R = 256 and 512 (160 KiB per workgroup), else the
    # one-thread-per-row prologue's 512
    assert m.max_rows(256) == 272
    assert m.max_rows(512) == 144
    for R in (16, 32, 64, 128):
        assert m.max_rows(R) == 512
    assert m.max_rows(48) == 0
    for R in (16, 64, 256, 512):
        mr = m.max_rows(R)
        assert m.why_not(mr, 4096, R, 3) is None
        assert "LDS" in m.why_not(mr + 1, 4096, R, 3)
    # the noise bound tables (25856 bytes), the transform table (a 256-byte
    # stamp, 32768 bf16 entries), the ticket block (256 bytes) and three
    # steps' eight per-row slot arrays
    assert m.NOISE_TABLES_BYTES == 25856
    assert m.TABLES_BYTES == 25856 + 256 + 65536
    assert m.workspace_bytes(64, 163840, 256, 5) == m.TABLES_BYTES + 256 + 64 * 8 * 3 * 8
    assert m.workspace_bytes(0, 163840, 256, 5) == 0
    assert m.workspace_bytes(4, 100, 256, 5) == 0        # vocab not a multiple of 8


@pytest.mark.parametrize("rows,V,R,k,why", [
    (0, 4096, 32, 3, "no requests"),
    (2, 4096, 32, 0, "no draft steps"),
    (2, 4100, 32, 3, "vocabulary"),
    (2, 0x7fff0008, 32, 3, "MARKOV_MAX_VOCAB"),
    (2, 0x7fff0000, 32, 3, None),
    (2, 4096, 48, 3, "rank"),
    (2, 4096, 1024, 3, "rank"),
    (273, 4096, 256, 3, "LDS"),
    (513, 4096, 32, 3, "LDS"),
    (2, 4096, 32, 3, None),
    (256, 163840, 256, 8, None),
])
def test_why_not(lib, rows, V, R, k, why):
    r = m.why_not(rows, V, R, k)
    if why is None:
        assert r is None
    else:
        assert r is not None and why in r


def _call(lib, shape, ptrs, k=3, ws_bytes=1 << 20):
    P = ctypes.c_void_p
    return lib.markov_sample_sequential(P(ptrs[0]), P(ptrs[1]), P(ptrs[2]), P(ptrs[3]),
                                        P(ptrs[4]), P(ptrs[5]), k, P(ptrs[6]), P(ptrs[7]),
                                        P(ptrs[8]), None, ctypes.byref(shape), P(ptrs[9]),
                                        ws_bytes)


def test_host_errors_before_any_device_work(lib):
    good = [0x10000 * (i + 1) for i in range(10)]          # never dereferenced
    sh = m.make_shape(2, 4096, 32)
    assert _call(lib, m.make_shape(0, 4096, 32), good) == -2
    assert _call(lib, m.make_shape(2, 4100, 32), good) == -2
    assert _call(lib, m.make_shape(2, 0x7fff0008, 32), good) == -8   # past MARKOV_MAX_VOCAB
    assert lib.markov_quantize_w2_fp8(ctypes.c_void_p(good[0]), ctypes.c_void_p(good[1]),
                                      ctypes.c_void_p(good[2]), 0x7fff0008, 256, None) == -8
    assert _call(lib, sh, good, k=0) == -2
    assert _call(lib, m.make_shape(2, 4096, 40), good) == -3
    assert _call(lib, m.make_shape(300, 4096, 256), good) == -5
    assert _call(lib, sh, good, ws_bytes=m.TABLES_BYTES + 256 + 2 * 24 * 8 - 1) == -6
    for i in range(10):
        bad = list(good)
        bad[i] = 0
        assert _call(lib, sh, bad) == -1, i
    for i in (0, 1, 2, 7):                                  # bf16 arrays
        bad = list(good)
        bad[i] += 2
        assert _call(lib, sh, bad) == -4, i
    assert _call(lib, sh, good, ws_bytes=8) == -6
    P = ctypes.c_void_p
    assert lib.markov_debug_bias(P(good[0]), P(good[1]), P(good[2]), P(good[3]),
                                 ctypes.byref(m.make_shape(2, 4096, 33)), None) == -3
    assert lib.markov_debug_gumbel(None, None, 4, ctypes.c_float(1.0), 1, 0, 1, None, None, None,
                                   None) == -1
    bad = list(good)
    bad[9] += 8                                             # workspace must be 16-byte aligned
    assert _call(lib, sh, bad, ws_bytes=1 << 20) == -4


def test_workspace_init_host_errors(lib):
    """markov_workspace_init rejects a NULL, misaligned or too small workspace
    before any device call (a NULL shape is allowed: no transform stamp)."""
    P = ctypes.c_void_p
    sh = m.make_shape(2, 4096, 32, 1.0, 30.0)
    need = m.workspace_bytes(2, 4096, 32, 3)
    assert lib.markov_workspace_init(None, need, ctypes.byref(sh), None) == -1
    assert lib.markov_workspace_init(P(0x10008), need, ctypes.byref(sh), None) == -4
    assert lib.markov_workspace_init(P(0x10000), 64, ctypes.byref(sh), None) == -6
    assert lib.markov_workspace_init(P(0x10000), 64, None, None) == -6
