"""Shrunk synthetic cases shared by the GPU tests (inputs only: no arithmetic
of the method)."""

import numpy as np

from markov_draft_sampling_step_amd import workloads


def custom(V, R, rows, k, seed, temps=(1.0,), softcap=0.0, mult=1.0, inject=True, prev_oob=True):
    """A shrunk workload with mixed temperatures, injected ties and NaNs and
    out-of-range feed tokens."""
    w = workloads.make("tiny", V=V, R=R, rows=rows, k=k, data_seed=seed)
    rng = np.random.default_rng(seed + 1000)
    w.name = f"custom{seed}"
    w.w1 = workloads.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.05)
    w.w2 = workloads.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.05)
    w.base = workloads.to_bf16_bits(rng.standard_normal((rows, k, V)).astype(np.float32) * 3)
    w.temperature = np.array([temps[r % len(temps)] for r in range(rows)], dtype=np.float32)
    w.seeds = rng.integers(-(2 ** 62), 2 ** 62, size=rows).astype(np.int64)
    P = rng.integers(0, 1 << 20, size=rows).astype(np.int64)
    w.positions = np.ascontiguousarray(P[:, None] + np.arange(k)[None, :])
    w.prev = rng.integers(0, V, size=rows).astype(np.int64)
    if prev_oob and rows >= 2:
        w.prev[0] = -5
        w.prev[1] = V + 17
    if inject and V >= 4:
        for r in range(0, rows, 3):
            for s in range(k):
                t1, t2 = sorted(int(t) for t in rng.choice(V, size=2, replace=False))
                val = 0x4280 if r % 2 == 0 else workloads.BF16_NAN
                w.base[r, s, t1] = w.base[r, s, t2] = val
    w.mult, w.softcap = mult, softcap
    return w
