"""Seeded synthetic inputs for the Markov draft-sampling step.

This module only draws numbers: it holds none of the step's arithmetic, and
both the HIP library's tests/benchmark and the CPU oracle take their inputs
from it. No page measures a public benchmark or dataset, so these five
workloads are the workloads. Each follows a fixed draw order from
``numpy.random.default_rng(data_seed)`` (PCG64):

    w1 -> w2 -> base -> spikes / injections -> prev -> seeds -> positions

Weights and logits are binary32 normals rounded to bf16 (nearest, ties to
even) and carried as ``uint16`` bit patterns. ``prev`` is uniform in
[0, V). A row's single position P_r gives the sample position of step s as
P_r + s.

The shapes follow the pages: the w2 table of 129280 x 256 bf16 (66 MB) and
of 163840 x 256 bf16 (84 MB) named in the vLLM kimi_k3 and deepseek_v41
Markov pages' module docstrings; rank 256; k = 5 draft steps.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BF16_NAN = 0x7FC0


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, nearest-even (input has no NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    V: int
    R: int
    rows: int
    k: int
    w1: np.ndarray            # uint16 [V, R]
    w2: np.ndarray            # uint16 [V, R]
    base: np.ndarray          # uint16 [rows, k, V]
    prev: np.ndarray          # int64 [rows]
    seeds: np.ndarray         # int64 [rows]
    positions: np.ndarray     # int64 [rows, k]
    temperature: np.ndarray   # float32 [rows]
    mult: float = 1.0
    softcap: float = 0.0
    tie_rows: list = field(default_factory=list)
    nan_rows: list = field(default_factory=list)
    injected: dict = field(default_factory=dict)   # row -> [(step, t1, t2)]

    def bytes_per_step(self) -> int:
        """Algorithmic HBM bytes of one step: the w2 table, the base read and
        cache write of one step's [rows, V] slice, and the rows' w1 rows."""
        return 2 * self.V * self.R + 4 * self.rows * self.V + 2 * self.rows * self.R


CONFIGS = {
    # name: (data_seed, V, R, rows, k)
    "tiny": (0, 4096, 32, 2, 3),
    "single": (1, 129280, 256, 1, 5),
    "small": (2, 129280, 256, 16, 5),
    "large": (3, 163840, 256, 64, 5),
    "stress": (4, 163840, 256, 256, 8),
}


def _normal_bf16(rng, shape, sigma):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(sigma)
    return to_bf16_bits(x)


def make(name: str, V: int | None = None, rows: int | None = None, k: int | None = None,
         R: int | None = None, data_seed: int | None = None) -> Workload:
    """One of the five workloads, optionally shrunk (V, rows, k, R) with the
    same distributions, for cases the oracle must finish in seconds."""
    seed0, V0, R0, rows0, k0 = CONFIGS[name]
    V = V0 if V is None else V
    R = R0 if R is None else R
    rows = rows0 if rows is None else rows
    k = k0 if k is None else k
    seed = seed0 if data_seed is None else data_seed
    rng = np.random.default_rng(seed)

    w1 = _normal_bf16(rng, (V, R), 0.02)
    w2 = _normal_bf16(rng, (V, R), 0.02)
    sigma = 2.0 if name == "tiny" else 3.0
    if name in ("single", "small"):
        x = rng.standard_normal(size=(rows, k, V), dtype=np.float32) * np.float32(sigma)
        n_spike = min(32, V)
        for r in range(rows):
            for s in range(k):
                ids = rng.choice(V, size=n_spike, replace=False)
                x[r, s, ids] += np.float32(8.0)
        base = to_bf16_bits(x)
    else:
        base = _normal_bf16(rng, (rows, k, V), sigma)

    tie_rows, nan_rows, injected = [], [], {}
    if name == "stress":
        # ceil(1% of rows) tie rows with at least one of each temperature
        # parity, and ceil(0.1% of rows) NaN rows, injected at every step.
        n_tie = max(2, int(np.ceil(0.01 * rows)))
        n_nan = max(1, int(np.ceil(0.001 * rows)))
        perm = rng.permutation(rows)
        evens = [int(r) for r in perm if r % 2 == 0]
        odds = [int(r) for r in perm if r % 2 == 1]
        tie_rows = [evens[0]] + ([odds[0]] if odds else [])
        rest = [int(r) for r in perm if int(r) not in tie_rows]
        tie_rows += rest[: max(0, n_tie - len(tie_rows))]
        rest = [r for r in rest if r not in tie_rows]
        nan_rows = rest[:n_nan]
        for r in tie_rows + nan_rows:
            injected[r] = []
            for s in range(k):
                t1, t2 = sorted(int(t) for t in rng.choice(V, size=2, replace=False))
                val = np.uint16(0x4280) if r in tie_rows else np.uint16(BF16_NAN)  # 64.0 / NaN
                base[r, s, t1] = val
                base[r, s, t2] = val
                injected[r].append((s, t1, t2))

    prev = rng.integers(0, V, size=rows, dtype=np.int64)
    if name == "tiny":
        seeds = np.array([1, 2][:rows] + [3] * max(0, rows - 2), dtype=np.int64)
        P = np.array([10, 20][:rows] + [30] * max(0, rows - 2), dtype=np.int64)
    elif name == "single":
        seeds = rng.integers(0, 2 ** 32, size=rows, dtype=np.int64)
        P = np.full(rows, 4096, dtype=np.int64)
    elif name == "small":
        seeds = rng.integers(0, 32768, size=rows, dtype=np.int64)
        P = rng.integers(0, 32768, size=rows, dtype=np.int64)
    else:
        seeds = rng.integers(0, 2 ** 63, size=rows, dtype=np.int64)
        P = rng.integers(0, 32768, size=rows, dtype=np.int64)
    positions = P[:, None] + np.arange(k, dtype=np.int64)[None, :]

    if name == "tiny" or name == "small":
        temperature = np.full(rows, 1.0, dtype=np.float32)
    elif name == "single":
        temperature = np.full(rows, 0.8, dtype=np.float32)
    elif name == "large":
        temperature = np.full(rows, 0.7, dtype=np.float32)
    else:
        temperature = np.where(np.arange(rows) % 2 == 0, 0.0, 1.0).astype(np.float32)

    mult, softcap = (1.0, 30.0) if name == "large" else (1.0, 0.0)
    return Workload(name=name, V=V, R=R, rows=rows, k=k, w1=w1, w2=w2, base=base, prev=prev,
                    seeds=seeds, positions=np.ascontiguousarray(positions),
                    temperature=temperature, mult=mult, softcap=softcap,
                    tie_rows=sorted(tie_rows), nan_rows=sorted(nan_rows), injected=injected)


def to_device(w: Workload, device="cuda") -> dict:
    """The workload's arrays as device tensors (bf16 bit patterns become
    torch.bfloat16), plus empty outputs and a zeroed workspace."""
    import torch

    from . import new_workspace

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)

    def plain(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return dict(
        base=bf(w.base), w1=bf(w.w1), w2=bf(w.w2), prev=plain(w.prev), seeds=plain(w.seeds),
        positions=plain(w.positions), temperature=plain(w.temperature),
        cache=torch.empty((w.rows, w.k, w.V), dtype=torch.bfloat16, device=device),
        tokens=torch.empty((w.rows, w.k), dtype=torch.int64, device=device),
        workspace=new_workspace(w.rows, w.V, w.R, w.k, device=device, mult=w.mult, softcap=w.softcap),
    )


def run(w: Workload, d: dict, stream=None, exact: bool = False, step: int | None = None,
        fallback: bool = False):
    """One k-step loop of workload `w` on the device tensors `d` (or its one
    step `step`)."""
    from . import sample_sequential

    sample_sequential(d["base"], d["w1"], d["w2"], d["prev"], d["seeds"], d["positions"],
                      d["temperature"], d["cache"], d["tokens"], d["workspace"], w.mult,
                      w.softcap, stream=stream, exact=exact, step=step, fallback=fallback)


def fetch(d: dict):
    """(cache uint16 [rows, k, V], tokens int64 [rows, k]) back on the host."""
    import torch

    cache = d["cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    return cache, d["tokens"].cpu().numpy()


# -- verification of a drafted block ---------------------------------------------
# Synthetic target and draft distributions shaped like the large workload's
# drafting (64 rows, k = 5 proposals, V = 163840): target logits N(0, 3)
# per (row, position); draft logits the target's plus N(0, 1) noise, so the
# draft is close to but not the target; probabilities are their softmax in
# binary64 stored as binary32. Greedy drafts are the target's argmax with
# probability 0.8 per position, else a uniform id; sampled drafts are drawn
# from the draft distribution (Gumbel-max with numpy's generator). A quarter
# of the rows propose fewer than P tokens. Uniforms are uniform in [0, 1).


@dataclass
class VerifyWorkload:
    name: str
    B: int
    P: int
    V: int
    logits: np.ndarray        # uint16 bf16 [B, P+1, V]: the target's logits (greedy verifier)
    target: np.ndarray        # float32 [B, P+1, V]
    draftp: np.ndarray        # float32 [B, P, V]
    draft_greedy: np.ndarray  # int64 [B, P]
    draft_sampled: np.ndarray  # int64 [B, P]
    lengths: np.ndarray       # int32 [B]
    uniforms: np.ndarray      # float32 [B, 2P+1]


def make_verify(B: int = 64, P: int = 5, V: int = 163840, data_seed: int = 5,
                name: str = "verify") -> VerifyWorkload:
    rng = np.random.default_rng(data_seed)
    x = rng.standard_normal(size=(B, P + 1, V), dtype=np.float32) * np.float32(3.0)
    logits = to_bf16_bits(x)
    lf = bf16_bits_to_f32(logits).astype(np.float64)

    def softmax(z):
        z = z - z.max(axis=-1, keepdims=True)
        e = np.exp(z)
        return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)

    target = np.empty((B, P + 1, V), dtype=np.float32)
    draftp = np.empty((B, P, V), dtype=np.float32)
    draft_sampled = np.empty((B, P), dtype=np.int64)
    for b in range(B):
        target[b] = softmax(lf[b])
        dz = lf[b, :P] + rng.standard_normal(size=(P, V))
        draftp[b] = softmax(dz)
        g = -np.log(-np.log(rng.random(size=(P, V))))
        draft_sampled[b] = np.argmax(np.log(np.maximum(draftp[b], 1e-45)) + g, axis=1)
    am = np.argmax(bf16_bits_to_f32(logits[:, :P]), axis=2)
    draft_greedy = np.where(rng.random((B, P)) < 0.8, am, rng.integers(0, V, size=(B, P))).astype(np.int64)
    lengths = np.full(B, P, dtype=np.int32)
    short = rng.random(B) < 0.25
    lengths[short] = rng.integers(0, max(P, 1), size=int(short.sum()))
    uniforms = rng.random((B, 2 * P + 1)).astype(np.float32)
    return VerifyWorkload(name=name, B=B, P=P, V=V, logits=logits, target=target, draftp=draftp,
                          draft_greedy=draft_greedy, draft_sampled=draft_sampled,
                          lengths=lengths, uniforms=uniforms)
