"""Sweeps over every 32-bit hash (CPU only).

* The oracle's uniform u(h) equals the exact rounding of (h + 1/2) 2^-32 to
  binary32 at all 2^32 hashes (integer rounding in ``exhaustive.c``; the
  oracle uses a binary64 product).
* The step kernel's two noise bound tables (host data, read through
  ``markov_debug_noise_table``) lie on or above the oracle's noise -lb(h) at
  all 2^32 hashes. The kernel's pruning of exact keys is sound only if this
  holds everywhere; the minimum slack of each table is printed.

Both sweeps run in ``tests/exhaustive.c``, compiled here with gcc and handed
the oracle's exports by address.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def sweep(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("exhaustive") / "libexhaustive.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out,
                           os.path.join(HERE, "exhaustive.c"), "-lm"])
    lib = ctypes.CDLL(out)
    P = ctypes.c_void_p
    lib.check_uniform_all.restype = ctypes.c_int64
    lib.check_uniform_all.argtypes = [P, ctypes.c_int, P]
    lib.check_noise_tables_all.restype = ctypes.c_int64
    lib.check_noise_tables_all.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, P, P, P, P]
    return lib


@pytest.mark.slow
def test_uniform_exact_at_every_hash(oracle_lib, sweep):
    fn = ctypes.cast(oracle_lib.lib().oracle_uniform, ctypes.c_void_p)
    first = ctypes.c_uint32()
    bad = sweep.check_uniform_all(fn, THREADS, ctypes.byref(first))
    assert bad == 0, f"{bad} hashes differ, first h = {first.value}"


@pytest.mark.slow
def test_noise_tables_bound_the_noise_at_every_hash(oracle_lib, sweep):
    import markov_draft_sampling_step_amd as m

    if not os.path.exists(m.LIBRARY):
        from markov_draft_sampling_step_amd import build

        build.build()
    table = m.debug_noise_table()                   # float32 [2050, 3]: A, B, C
    A, B, C = (np.ascontiguousarray(table[:, i]) for i in range(3))
    fn = ctypes.cast(oracle_lib.lib().oracle_gumbel_key, ctypes.c_void_p)
    ml, mc = ctypes.c_double(), ctypes.c_double()
    al, ac = ctypes.c_uint32(), ctypes.c_uint32()
    bad = sweep.check_noise_tables_all(fn, A.ctypes.data, B.ctypes.data, C.ctypes.data, len(A),
                                       THREADS, ctypes.byref(ml), ctypes.byref(al),
                                       ctypes.byref(mc), ctypes.byref(ac))
    print(f"min slack: line {ml.value:.3e} at h={al.value}, constant {mc.value:.3e} at h={ac.value}")
    assert bad == 0, bad
    assert ml.value > 0 and mc.value >= 0
