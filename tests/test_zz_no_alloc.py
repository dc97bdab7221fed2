"""The entry point that allocates nothing, against markov_sample_sequential.

markov_sample_sequential_noalloc runs the same kernels on the library's own
per-device workspace. Two calls in a row (the second smaller, with another
rank and no soft cap) must each give the bits markov_sample_sequential gives
on a workspace of its own; a shape beyond its row limit is refused.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import markov_draft_sampling_step_amd as m  # noqa: E402
from markov_draft_sampling_step_amd import workloads  # noqa: E402
from oracle import parity  # noqa: E402


def _case(V, R, rows, k, seed, temps, softcap):
    w = workloads.make("tiny", V=V, R=R, rows=rows, k=k, data_seed=seed)
    rng = np.random.default_rng(seed)
    w.name = f"noalloc{seed}"
    w.temperature = np.array([temps[r % len(temps)] for r in range(rows)], dtype=np.float32)
    w.seeds = rng.integers(-(2 ** 62), 2 ** 62, size=rows).astype(np.int64)
    w.mult, w.softcap = 1.0, softcap
    return w


def test_noalloc_matches_sample_sequential():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    for w in (_case(4104, 128, 70, 4, 61, (1.0, 0.0, 0.7), 30.0),
              _case(1000, 32, 19, 3, 62, (0.0, 1.0), 0.0)):
        print(f"case {w.name} V={w.V} R={w.R} rows={w.rows} k={w.k} cap={w.softcap}", flush=True)
        sys.stdout.flush()
        d = workloads.to_device(w, dev)
        workloads.run(w, d)
        torch.cuda.synchronize()
        c_ref, t_ref = workloads.fetch(d)
        d["cache"].zero_()
        d["tokens"].fill_(-1)
        torch.cuda.synchronize()
        m.sample_sequential_noalloc(d["base"], d["w1"], d["w2"], d["prev"], d["seeds"],
                                    d["positions"], d["temperature"], d["cache"], d["tokens"],
                                    w.mult, w.softcap)
        torch.cuda.synchronize()
        c, t = workloads.fetch(d)
        assert np.array_equal(t, t_ref)
        assert np.array_equal(c, c_ref)
        rep = parity.check_loop(w, c, t, threads=8)
        parity.assert_parity(rep)


def test_noalloc_refuses_too_many_rows():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    assert m.noalloc_max_rows() == 512
    rows, k, V, R = 600, 1, 8, 16
    z = lambda *s, dt=torch.bfloat16: torch.zeros(*s, dtype=dt, device=dev)
    with pytest.raises(m.MarkovError):
        m.sample_sequential_noalloc(z(rows, k, V), z(V, R), z(V, R), z(rows, dt=torch.int64),
                                    z(rows, dt=torch.int64), z(rows, k, dt=torch.int64),
                                    z(rows, dt=torch.float32), z(rows, k, V),
                                    z(rows, k, dt=torch.int64))
