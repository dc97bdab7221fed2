"""The greedy loop (every row at temperature 0) on the GPU, through the C ABI.

markov_greedy_sequential runs a kernel specialised for temperature 0 (no
noise, exact in-register argmax with NaN and -inf ranked). Its tokens and
cache are compared teacher-forced with the oracle at temperature 0, its
packed winners with the oracle's packing of the device's own winning logit,
markov_greedy_finalize with the tokens, the cache-less (chain) mode with the
cache-writing one, and the whole loop with markov_sample_sequential at
temperature 0.
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


def greedy_run(w, d, cache=True):
    win = torch.full((w.rows, w.k), -1, dtype=torch.int64, device=d["tokens"].device)
    m.greedy_sequential(d["base"], d["w1"], d["w2"], d["prev"], d["tokens"], d["workspace"],
                        cache=d["cache"] if cache else None, winners=win, mult=w.mult,
                        softcap=w.softcap)
    torch.cuda.synchronize()
    return win


def check_greedy(w, dev, rows=None):
    """Greedy loop of w (temperatures set to 0) against the oracle; returns
    (cache, tokens, winners) of the device."""
    import oracle

    w.temperature = np.zeros(w.rows, dtype=np.float32)
    say(f"greedy {w.name} V={w.V} R={w.R} rows={w.rows} k={w.k} cap={w.softcap}")
    d = workloads.to_device(w, dev)
    win = greedy_run(w, d)
    cg, tg = workloads.fetch(d)
    wg = win.cpu().numpy().view(np.uint64)
    rep = parity.check_loop(w, cg, tg, rows=rows, threads=THREADS)
    say(f"  row-steps {rep['row_steps']} decided {rep['decided']} undecided {rep['undecided']} "
        f"cache differing {rep['cache_differ']} admissible-by-cancellation {rep['cache_cancel']}")
    parity.assert_parity(rep)
    # the packed winners: the device's own winning logit and token
    for r in (range(w.rows) if rows is None else rows):
        for s in range(w.k):
            t = int(tg[r, s])
            lv = float(parity.bf16_to_f32(cg[r, s, t:t + 1])[0])
            assert int(wg[r, s]) == oracle.pack_winner(lv, t), (r, s)
    # finalize gives the tokens back
    toks = torch.empty((w.rows, w.k), dtype=torch.int64, device=dev)
    m.greedy_finalize(win, toks)
    torch.cuda.synchronize()
    assert np.array_equal(toks.cpu().numpy(), tg)
    # chain mode (no cache written): the same tokens and winners
    d["cache"].fill_(0)
    d["tokens"].fill_(-1)
    win2 = greedy_run(w, d, cache=False)
    cg2, tg2 = workloads.fetch(d)
    assert np.array_equal(tg2, tg)
    assert np.array_equal(win2.cpu().numpy(), win.cpu().numpy())
    assert not cg2.any(), "chain mode wrote the cache"
    return cg, tg, wg


@pytest.mark.parametrize("args", [
    dict(V=1000, R=32, rows=19, k=3, seed=101),
    dict(V=264, R=16, rows=3, k=2, seed=102),
    dict(V=8, R=16, rows=1, k=2, seed=103, inject=False),
    dict(V=2056, R=64, rows=33, k=4, seed=104, softcap=30.0),
    dict(V=1032, R=512, rows=5, k=2, seed=105, mult=0.5),
    dict(V=4104, R=128, rows=70, k=2, seed=106),
    dict(V=2056, R=256, rows=160, k=3, seed=107, softcap=30.0),
    dict(V=1016, R=256, rows=256, k=2, seed=108),
])
def test_greedy_cases(dev, args):
    check_greedy(custom(**args), dev)


def test_greedy_nan_and_minus_inf_rows(dev):
    """Rows whose logits are all -inf (token 0), -inf except a few, NaN at
    several ids (the lowest wins), and +inf ties."""
    w = custom(V=1032, R=32, rows=6, k=2, seed=109, inject=False)
    NEG, POS, NAN = 0xFF80, 0x7F80, workloads.BF16_NAN
    w.base[0, :, :] = NEG
    w.base[1, :, :] = NEG
    w.base[1, 0, 700] = 0x3F80
    w.base[1, 1, 5] = 0x3F80
    w.base[2, 0, [40, 41, 900]] = NAN
    w.base[2, 1, [1031, 3]] = NAN
    w.base[3, 0, [10, 20]] = POS
    w.base[3, 1, [1000, 999]] = POS
    cg, tg, _ = check_greedy(w, dev)
    assert tg[0, 0] == 0 and tg[0, 1] == 0
    assert tg[1, 0] == 700 and tg[1, 1] == 5
    assert tg[2, 0] == 40 and tg[2, 1] == 3
    assert tg[3, 0] == 10 and tg[3, 1] == 999


@pytest.mark.parametrize("name", ["large", "stress"])
def test_greedy_full_size(dev, name):
    """The greedy loop on the large (V=163840, 64 rows, soft cap) and stress
    (256 rows, k=8, tie and NaN rows) inputs, every row-step against the
    oracle at temperature 0."""
    w = workloads.make(name)
    cg, tg, _ = check_greedy(w, dev)
    for r in w.nan_rows + w.tie_rows:
        for (s, t1, t2) in w.injected[r]:
            assert tg[r, s] == t1, (r, s)


def test_greedy_equals_sampling_at_temperature_zero(dev):
    """The sampling kernel with every temperature 0 and the greedy kernel give
    the same bits."""
    w = custom(V=4104, R=128, rows=70, k=3, seed=110, softcap=30.0)
    w.temperature = np.zeros(w.rows, dtype=np.float32)
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    torch.cuda.synchronize()
    c1, t1 = workloads.fetch(d)
    d["cache"].fill_(0)
    greedy_run(w, d)
    c2, t2 = workloads.fetch(d)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)


def test_greedy_steps_equal_the_loop(dev):
    w = custom(V=2056, R=64, rows=33, k=3, seed=111)
    d = workloads.to_device(w, dev)
    win = greedy_run(w, d)
    c1, t1 = workloads.fetch(d)
    d["cache"].fill_(0)
    d["tokens"].fill_(-1)
    win2 = torch.full_like(win, -1)
    for s in range(w.k):
        m.greedy_sequential(d["base"], d["w1"], d["w2"], d["prev"], d["tokens"], d["workspace"],
                            cache=d["cache"], winners=win2, step=s)
    torch.cuda.synchronize()
    c2, t2 = workloads.fetch(d)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
    assert torch.equal(win, win2)
    assert not d["workspace"].cpu().numpy()[m.TABLES_BYTES:].any()
