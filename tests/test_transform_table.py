"""The output-transform table the library builds on the host (and stamps into
the workspace for the kernel's lookups) against the oracle's transform, for
every entry: the bf16 sum whose bits are i (i < 2^15, the non-negative
patterns) maps to the cached value the oracle computes for a base logit of
bits i and a zero bias. NaN entries must be NaN on both sides; everything
else bit-equal (both take tanh correctly rounded). Host code only."""

import numpy as np
import pytest

import markov_draft_sampling_step_amd as m
import oracle


def is_nan_bf16(b):
    b = np.asarray(b, dtype=np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)


@pytest.fixture(scope="module")
def libs():
    try:
        m.lib()
    except ImportError:
        pytest.skip("library not built")
    oracle.lib()


@pytest.mark.parametrize("mult,softcap", [(1.0, 30.0), (0.75, 30.0), (1.0, 0.5), (-1.5, 7.0),
                                          (0.0, 30.0), (3.0, 1e-3)])
def test_transform_table_equals_oracle(libs, mult, softcap):
    t = m.debug_transform_table(mult, softcap)
    o = np.array([oracle.cache_value(i, 0, mult, softcap) for i in range(m.TRANSFORM_ENTRIES)],
                 dtype=np.uint16)
    nt, no = is_nan_bf16(t), is_nan_bf16(o)
    assert np.array_equal(nt, no)
    bad = np.nonzero((t != o) & ~nt)[0]
    assert bad.size == 0, [(hex(i), hex(t[i]), hex(o[i])) for i in bad[:8]]


def test_transform_table_is_odd_and_saturates(libs):
    """cap = 30, mult = 1: the map is monotone and never exceeds the cap; the
    negative half (sign flipped, as the kernel applies it) mirrors it."""
    t = m.debug_transform_table(1.0, 30.0).astype(np.uint32)
    finite = np.arange(0x7F80)
    vals = (t[finite] << 16).view(np.float32)
    assert np.all(np.diff(vals) >= 0)
    assert vals.max() <= 30.0
    neg = ((t[finite] ^ 0x8000) << 16).view(np.float32)
    assert np.array_equal(neg, -vals)


def test_transform_table_rejects_no_cap(libs):
    out = np.zeros(4, dtype=np.uint16)
    import ctypes
    assert m.lib().markov_debug_transform_table(ctypes.c_float(1.0), ctypes.c_float(0.0),
                                                out.ctypes.data_as(ctypes.c_void_p), 4) == -2
