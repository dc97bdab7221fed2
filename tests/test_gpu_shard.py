"""One GPU's share of the vocabulary-parallel step, on one GPU.

The vocabulary is cut into G slabs; each step runs markov_shard_step on
every slab (global ids in the noise and the packets, w1 whole), then
markov_pick combines the G packets into the tokens that feed the next step.
Because every element's arithmetic is the same as in the full-vocabulary
kernel, the sharded loop must give the full loop's tokens and cache bit for
bit, and so the oracle's (vLLM muse_spark cutedsl draft Markov page: module
docstring on tensor-parallel drafting, the packet of the last block,
`_PickKernel`). Nothing here uses a second GPU.
"""

import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import markov_draft_sampling_step_amd as m  # noqa: E402
from markov_draft_sampling_step_amd import workloads  # noqa: E402
from oracle import parity  # noqa: E402
from tests.cases import custom  # noqa: E402

THREADS = min(16, os.cpu_count() or 4)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()
    return torch.device("cuda:0")


def run_sharded(w, d, G):
    """The loop of w over G slabs; returns (cache [rows, k, V] u16, tokens)."""
    rows, k, V, R = w.rows, w.k, w.V, w.R
    assert V % (8 * G) == 0
    Vs = V // G
    dev = d["base"].device
    slabs = []
    for g in range(G):
        sl = slice(g * Vs, (g + 1) * Vs)
        slabs.append(dict(base=d["base"][:, :, sl].contiguous(), w2=d["w2"][sl].contiguous(),
                          cache=torch.zeros((rows, k, Vs), dtype=torch.bfloat16, device=dev),
                          ws=m.new_workspace(rows, Vs, R, k, device=dev, mult=w.mult,
                                             softcap=w.softcap)))
    packets = torch.zeros((G, rows), dtype=torch.int64, device=dev)
    tokens = torch.full((rows, k), -1, dtype=torch.int64, device=dev)
    flat = tokens.view(-1)
    for s in range(k):
        feed, stride = (d["prev"], 1) if s == 0 else (flat[s - 1:], k)
        for g, sd in enumerate(slabs):
            m.shard_step(sd["base"], d["w1"], sd["w2"], feed, d["seeds"], d["positions"],
                         d["temperature"], sd["cache"], packets[g], sd["ws"], step=s,
                         vocab_offset=g * Vs, feed_stride=stride, mult=w.mult, softcap=w.softcap)
        m.pick(packets, flat[s:], stride=k)
    torch.cuda.synchronize()
    cache = torch.cat([sd["cache"] for sd in slabs], dim=2)
    for sd in slabs:
        assert not sd["ws"].cpu().numpy()[m.TABLES_BYTES:].any(), "slots left dirty"
    return cache.view(torch.int16).cpu().numpy().view(np.uint16), tokens.cpu().numpy()


def check(w, dev, G, oracle_check=True):
    say(f"shards {G} {w.name} V={w.V} R={w.R} rows={w.rows} k={w.k}")
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    torch.cuda.synchronize()
    c_full, t_full = workloads.fetch(d)
    c_sh, t_sh = run_sharded(w, d, G)
    assert np.array_equal(t_sh, t_full), np.argwhere(t_sh != t_full)[:5]
    assert np.array_equal(c_sh, c_full)
    if oracle_check:
        rep = parity.check_loop(w, c_sh, t_sh, threads=THREADS)
        parity.assert_parity(rep)
    return t_sh


@pytest.mark.parametrize("args,G", [
    (dict(V=4096, R=32, rows=2, k=3, seed=301), 8),
    (dict(V=2048, R=64, rows=33, k=4, seed=302, temps=(1.0, 0.0, 0.7), softcap=30.0), 8),
    (dict(V=2048, R=128, rows=19, k=3, seed=303, temps=(0.0, 1.0, float("nan"))), 4),
    (dict(V=4096, R=256, rows=160, k=2, seed=304, temps=(1.0, 0.0)), 8),
])
def test_sharded_loop_equals_full_vocabulary(dev, args, G):
    check(custom(**args), dev, G)


def test_ties_and_nans_across_shards(dev):
    """Injected ties and NaNs at ids in different slabs: the lower global id
    wins, as in the full vocabulary."""
    w = custom(V=2048, R=32, rows=6, k=3, seed=305, temps=(0.0, 1.0), inject=False)
    for r in range(w.rows):
        for s in range(w.k):
            t1, t2 = 100 + 37 * r + s, 1500 - 11 * r
            w.base[r, s, t1] = w.base[r, s, t2] = 0x4280 if r < 3 else workloads.BF16_NAN
    t = check(w, dev, 8)
    for r in range(w.rows):
        if r >= 3 or w.temperature[r] == 0:
            assert all(t[r, s] == 100 + 37 * r + s for s in range(w.k)), r


def test_large_in_eight_shards(dev):
    """The large workload (V=163840, 64 rows, soft cap) as 8 slabs of 20480:
    tokens and cache equal to the full-vocabulary loop (itself pinned to the
    oracle elsewhere)."""
    check(workloads.make("large"), dev, 8, oracle_check=False)
