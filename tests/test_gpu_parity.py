"""Parity of the HIP path with the oracle, through the C ABI, on the GPU.

Every case runs the device loop, then recomputes each checked row-step with
the oracle teacher-forced by the device's own previous token. The bar:
cache within one bf16 ulp of the oracle; tokens equal on every decided
row-step (see ``oracle_decided``); undecided row-steps counted and kept
within the near-tie set.
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

THREADS = min(16, os.cpu_count() or 4)   # the GPU machine's CPU share


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    m.lib()
    return torch.device("cuda:0")


def run_and_check(w, dev, rows=None, exact=False, fallback=False):
    say(f"case {w.name} V={w.V} R={w.R} rows={w.rows} k={w.k} exact={exact} fallback={fallback}")
    d = workloads.to_device(w, dev)
    workloads.run(w, d, exact=exact, fallback=fallback)
    torch.cuda.synchronize()
    cg, tg = workloads.fetch(d)
    rep = parity.check_loop(w, cg, tg, rows=rows, threads=THREADS)
    say(f"  row-steps {rep['row_steps']} decided {rep['decided']} (literal {rep['decided_literal']}) "
        f"undecided {rep['undecided']} cache differing {rep['cache_differ']}/{rep['cache_elems']}")
    say(f"COUNTS {w.name} row_steps={rep['row_steps']} decided={rep['decided']} "
        f"decided_literal={rep['decided_literal']} undecided={rep['undecided']} "
        f"cache_differ={rep['cache_differ']} cache_elems={rep['cache_elems']}")
    path = os.environ.get("PARITY_COUNTS_FILE")
    if path and rows is None and not exact and not fallback:
        import json

        with open(path, "a") as f:
            f.write(json.dumps({k: rep[k] for k in ("row_steps", "decided", "decided_literal",
                                                     "undecided", "cache_differ", "cache_cancel",
                                                     "cache_elems")} | {"workload": w.name}) + "\n")
    parity.assert_parity(rep)
    return cg, tg, rep


from tests.cases import custom  # noqa: E402


# -- pieces -------------------------------------------------------------------------

@pytest.mark.parametrize("V,R,rows", [(1000, 32, 19), (264, 16, 3), (2056, 64, 33), (1032, 512, 5),
                                      (4096, 256, 70)])
def test_bias_contraction_matches_oracle(dev, V, R, rows):
    import oracle

    say(f"bias V={V} R={R} rows={rows}")
    rng = np.random.default_rng(V + R + rows)
    w1 = workloads.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.05)
    w2 = workloads.to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.05)
    tok = rng.integers(-3, V + 3, size=rows).astype(np.int64)
    bw1 = torch.from_numpy(w1.view(np.int16)).to(dev).view(torch.bfloat16)
    bw2 = torch.from_numpy(w2.view(np.int16)).to(dev).view(torch.bfloat16)
    ttok = torch.from_numpy(tok).to(dev)
    bias = torch.empty((rows, V), dtype=torch.bfloat16, device=dev)
    m.debug_bias(bw1, bw2, ttok, bias)
    torch.cuda.synchronize()
    bg = bias.view(torch.int16).cpu().numpy().view(np.uint16)
    # oracle: sequential fp32 dot per element
    out = oracle.step(np.zeros((rows, V), np.uint16), w1, w2, tok, np.zeros(rows, np.int64),
                      np.zeros(rows, np.int64), 0, np.zeros(rows, np.float32), want_bias=True,
                      threads=THREADS)
    bo = out["bias"]
    g = parity.bf16_to_f32(bg).astype(np.float64)
    o = parity.bf16_to_f32(bo).astype(np.float64)
    tol = parity.ulp_bf16(np.maximum(np.abs(g), np.abs(o)))
    bad = np.abs(g - o) > tol
    # where cancellation leaves more than an ulp, fall back on the order-free
    # bound: the device value is a bf16 rounding of some sum within gamma_R of
    # the exact one
    if bad.any():
        idx = np.argwhere(bad)
        for r, v in idx[:2000]:
            row = oracle.w1_row(int(tok[r]), V)
            _, s64, sabs = oracle.bias(w1[row], w2[v])
            gam = R * 2.0 ** -24 / (1 - R * 2.0 ** -24)
            lo, hi = s64 - gam * sabs, s64 + gam * sabs
            assert parity.bf16_to_f32(np.array([oracle.bf16_round(lo)]))[0] <= g[r, v] <= \
                parity.bf16_to_f32(np.array([oracle.bf16_round(hi)]))[0], (r, v, g[r, v], o[r, v])
    say(f"  bias elements differing {int((g != o).sum())}/{g.size}, beyond one ulp {int(bad.sum())}")


def test_bf16_conversion_matches_oracle(dev):
    import oracle

    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # exact ties and near-ties in every binade, subnormals, extremes
    e = np.arange(0, 255, dtype=np.uint32)
    for low in (0x8000, 0x7FFF, 0x8001, 0x18000, 0x0000):
        bits = np.concatenate([bits, (e << 23) | np.uint32(low), (e << 23) | np.uint32(low) | np.uint32(1 << 31)])
    bits = np.concatenate([bits, np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F800000, 0xFF800000, 0x7FC00000,
                                           0x00000001, 0x80000001, 0x007FFFFF], dtype=np.uint32)])
    x = bits.view(np.float32)
    xt = torch.from_numpy(x).to(dev)
    out = torch.empty(x.size, dtype=torch.int16, device=dev)
    m.debug_bf16_round(xt, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    idx = np.arange(x.size)[:: max(1, x.size // 200000)]
    for i in idx:
        xi = float(x[i])
        if np.isnan(xi):
            assert (got[i] & 0x7F80) == 0x7F80 and (got[i] & 0x7F) != 0
            continue
        assert got[i] == oracle.bf16_round(xi), (hex(int(bits[i])), hex(int(got[i])))


M32 = (1 << 32) - 1


def _rotl(x, r):
    return ((x << r) | (x >> (32 - r))) & M32


def _rotr(x, r):
    return ((x >> r) | (x << (32 - r))) & M32


def _inv(a):
    return pow(a, -1, 1 << 32)


def _block(h, k):
    k = (k * 0xCC9E2D51) & M32
    k = _rotl(k, 15)
    k = (k * 0x1B873593) & M32
    h ^= k
    h = _rotl(h, 13)
    return (h * 5 + 0xE6546B64) & M32


def id_for_hash(seed, step, position, target):
    """A token id whose noise hash is `target`: MurmurHash3's last block and
    finaliser are bijections of the 32-bit word, so they invert exactly."""
    S = (seed & ((1 << 64) - 1)) ^ ((step & M32) << 32)
    P = (position - 1 + (1 << 30)) & ((1 << 64) - 1)
    h = _block(_block(_block(0, S & M32), S >> 32), P & M32)
    x = target
    x ^= x >> 16
    x = (x * _inv(0xC2B2AE35)) & M32
    x ^= (x >> 13) ^ (x >> 26)
    x = (x * _inv(0x85EBCA6B)) & M32
    x ^= x >> 16
    x ^= 16
    x = ((x - 0xE6546B64) * _inv(5)) & M32
    k = _rotr(x, 13) ^ h
    k = (k * _inv(0x1B873593)) & M32
    k = _rotr(k, 15)
    return (k * _inv(0xCC9E2D51)) & M32


def test_gumbel_exact_key_and_upper_bound(dev):
    """The kernel's exact key equals the oracle's, and its cheap bound is
    above it, at chosen hashes (every bucket start and end of the noise
    table, h = 0, the top 128 hashes where u rounds to 1) and random ones,
    for spread-out logits and several temperatures."""
    import oracle
    from tests.test_noise_bound import bucket_starts

    starts = bucket_starts()
    targets = [0, 1, 2, 3, (1 << 32) - 1, (1 << 32) - 128, (1 << 32) - 129, (1 << 32) - 127]
    for b in range(len(starts) - 1):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi >= lo:
            targets += [lo, hi, min(lo + 1, hi)]
    rng = np.random.default_rng(9)
    targets += [int(x) for x in rng.integers(0, 1 << 32, size=200000)]
    n = len(targets)
    ws = m.new_workspace(1, 4096, 32, 1, device=dev)
    vals = rng.standard_normal(n).astype(np.float32) * 4
    vals[: n // 8] *= 1e3
    vals[n // 8: n // 4] *= 1e-6
    logits = parity.bf16_to_f32(workloads.to_bf16_bits(vals))
    for T, seed, step, pos in ((1.0, 12345, 0, 4096), (0.7, -(2 ** 60) + 3, 3, 17), (0.8, 7, 7, 1),
                               (2.5, 99, 1, 1 << 40), (1e-3, 5, 2, 3)):
        ids = np.array([id_for_hash(seed, step, pos, t) for t in targets], dtype=np.uint64).astype(np.uint32)
        for i in range(0, n, 997):
            assert oracle.noise_hash(seed, step, pos, int(ids[i])) == targets[i]
        lt = torch.from_numpy(logits).to(dev)
        it = torch.from_numpy(ids.view(np.int32)).to(dev)
        kx = torch.empty(n, dtype=torch.float32, device=dev)
        ku = torch.empty_like(kx)
        m.debug_gumbel(lt, it, T, seed, step, pos, ws, kx, ku)
        torch.cuda.synchronize()
        kx, ku = kx.cpu().numpy().astype(np.float64), ku.cpu().numpy().astype(np.float64)
        fin = np.isfinite(ku)
        assert fin.mean() > 0.99
        gap = ku[fin] - kx[fin]
        assert np.all(gap >= 0), (T, float(gap.min()), int(np.argmin(gap)))
        say(f"  T={T}: bound - key: min {gap.min():.3g}, median {np.median(gap):.3g}")
        # exact keys bit-equal to the oracle's (sampled, with every chosen hash)
        sel = list(range(0, n - 200000)) + [int(x) for x in rng.choice(np.arange(n - 200000, n), 5000)]
        mism = 0
        for i in sel:
            ko = oracle.gumbel_key(float(logits[i]), T, targets[i])
            if np.float32(ko).view(np.uint32) != np.float32(kx[i]).view(np.uint32):
                mism += 1
        assert mism <= 2, mism   # only a binary64 log within an ulp of a rounding midpoint may differ


# -- loops ----------------------------------------------------------------------------

def test_tiny(dev):
    run_and_check(workloads.make("tiny"), dev)


@pytest.mark.parametrize("args", [
    dict(V=1000, R=32, rows=19, k=3, seed=1, temps=(1.0, 0.0, 0.7)),
    dict(V=264, R=16, rows=3, k=2, seed=2, temps=(2.0,)),
    dict(V=8, R=16, rows=1, k=2, seed=3, temps=(1.0,), inject=False),
    dict(V=2056, R=64, rows=33, k=4, seed=4, temps=(0.0, 1.0), softcap=30.0),
    dict(V=1032, R=512, rows=5, k=2, seed=5, temps=(1.5, -0.0, 0.5), mult=0.5),
    dict(V=4104, R=128, rows=70, k=2, seed=6, temps=(1.0, float("nan"), 0.0)),
    dict(V=1016, R=256, rows=256, k=2, seed=7, temps=(0.0, 1.0)),
    # two row groups with a soft cap (the kernel's own tanh, constant noise bounds)
    dict(V=2056, R=256, rows=160, k=3, seed=8, temps=(1.0, 0.0, 0.7), softcap=30.0),
    dict(V=1544, R=128, rows=200, k=2, seed=9, temps=(0.6, 1.3), softcap=20.0, mult=0.9),
    # negative and infinite temperatures (a negative T divides; an infinite
    # one leaves the noise alone, and an infinite logit over it a NaN key)
    dict(V=1032, R=64, rows=24, k=3, seed=10, temps=(-0.8, float("inf"), 1.0, -float("inf"), 0.0)),
])
def test_ragged_and_edge_shapes(dev, args):
    w = custom(**args)
    run_and_check(w, dev)


@pytest.mark.parametrize("R", [32, 256, 512])
def test_max_rows(dev, R):
    """The most rows each rank class takes (the LDS budget's limit): 512 at
    R = 32 (one thread per row in the prologue), 272 at R = 256 and 144 at
    R = 512 (the embeddings fill LDS; 16-block and 512-rank plans)."""
    rows = m.max_rows(R)
    assert m.why_not(rows, 2056, R, 2) is None
    run_and_check(custom(V=2056, R=R, rows=rows, k=2, seed=50 + R, temps=(1.0, 0.0, 0.7)), dev)


def test_exact_and_pruned_agree_small(dev):
    w = custom(V=2056, R=64, rows=33, k=4, seed=11, temps=(0.0, 1.0, 0.3))
    cg1, tg1, _ = run_and_check(w, dev)
    cg2, tg2, _ = run_and_check(w, dev, exact=True)
    cg3, tg3, _ = run_and_check(w, dev, fallback=True)
    assert np.array_equal(tg1, tg2) and np.array_equal(tg1, tg3)
    assert np.array_equal(cg1, cg2) and np.array_equal(cg1, cg3)


def test_workspace_reuse_is_deterministic(dev):
    w = custom(V=1000, R=32, rows=19, k=3, seed=12, temps=(1.0, 0.0))
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    c1, t1 = workloads.fetch(d)
    for _ in range(3):
        workloads.run(w, d)
    c2, t2 = workloads.fetch(d)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
    ws = d["workspace"].cpu().numpy()
    table = m.debug_noise_table()
    pairs = ws[: 2050 * 8].view(np.float32).reshape(2050, 2)
    consts = ws[m.TABLE_PAIRS_BYTES: m.TABLE_PAIRS_BYTES + 2050 * 4].view(np.float32)
    assert np.array_equal(pairs, table[:, :2]) and np.array_equal(consts, table[:, 2]), "noise table changed"
    assert not ws[m.TABLES_BYTES:].any(), "slots must be left zeroed"


def test_workspace_shared_across_loops_of_different_k(dev):
    """One workspace serves loops of k = 3, 1 and 2 in turn (its slots and the
    last step's ticket are left zeroed by every loop): each loop gives the
    bits it gives on a fresh workspace of its own."""
    shared = None
    for k, seed in ((3, 41), (1, 42), (2, 43), (3, 44)):
        w = custom(V=2056, R=64, rows=33, k=k, seed=seed, temps=(1.0, 0.0, 0.7), softcap=30.0)
        d = workloads.to_device(w, dev)
        workloads.run(w, d)
        torch.cuda.synchronize()
        c_ref, t_ref = workloads.fetch(d)
        if shared is None:
            shared = m.new_workspace(w.rows, w.V, w.R, w.k, device=dev, mult=w.mult, softcap=w.softcap)
        d["workspace"] = shared
        d["cache"].zero_()
        d["tokens"].fill_(-1)
        workloads.run(w, d)
        torch.cuda.synchronize()
        c, t = workloads.fetch(d)
        assert np.array_equal(t, t_ref), k
        assert np.array_equal(c, c_ref), k
        assert not shared.cpu().numpy()[m.TABLES_BYTES:].any(), k
    say("  shared workspace: k = 3, 1, 2, 3 match fresh workspaces")


@pytest.mark.parametrize("args", [
    dict(V=4104, R=128, rows=70, k=3, seed=31, temps=(1.0, 0.0, 0.6)),
    dict(V=1000, R=32, rows=19, k=4, seed=32, temps=(0.0, 1.0)),
    dict(V=2056, R=256, rows=160, k=3, seed=33, temps=(1.0, 0.0), softcap=30.0),
])
def test_loop_equals_step_by_step_calls(dev, args):
    """markov_sample_sequential and markov_sample_step called for each step
    in turn give the same bits."""
    w = custom(**args)
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    torch.cuda.synchronize()
    c1, t1 = workloads.fetch(d)
    d["cache"].zero_()
    d["tokens"].fill_(-1)
    for s in range(w.k):
        workloads.run(w, d, step=s)
    torch.cuda.synchronize()
    c2, t2 = workloads.fetch(d)
    assert np.array_equal(t1, t2)
    assert np.array_equal(c1, c2)
    assert not d["workspace"].cpu().numpy()[m.TABLES_BYTES:].any()
    say(f"  {w.name}: loop == steps")


@pytest.mark.parametrize("name", ["single", "small", "large"])
def test_full_config(dev, name):
    run_and_check(workloads.make(name), dev)


def test_full_stress(dev):
    """Every row and step of the stress workload against the oracle, and the
    injected rows' tokens: the first of two NaN logits at any temperature,
    the first of two tied maxima at T = 0."""
    w = workloads.make("stress")
    cg, tg, rep = run_and_check(w, dev)
    for r in w.nan_rows:
        for (s, t1, t2) in w.injected[r]:
            assert tg[r, s] == t1, (r, s)
    for r in w.tie_rows:
        if w.temperature[r] == 0:
            for (s, t1, t2) in w.injected[r]:
                assert tg[r, s] == t1, (r, s)


@pytest.mark.parametrize("name", ["large", "stress"])
def test_exact_and_pruned_agree_full(dev, name):
    w = workloads.make(name)
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    c1, t1 = workloads.fetch(d)
    workloads.run(w, d, exact=True)
    c2, t2 = workloads.fetch(d)
    workloads.run(w, d, fallback=True)
    c3, t3 = workloads.fetch(d)
    assert np.array_equal(t1, t2) and np.array_equal(t1, t3)
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)


def test_graph_replay_matches_eager(dev):
    """The loop captured as a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager result."""
    w = custom(V=2056, R=64, rows=33, k=4, seed=21, temps=(0.0, 1.0, 0.7), softcap=30.0)
    d = workloads.to_device(w, dev)
    workloads.run(w, d)
    torch.cuda.synchronize()
    c_ref, t_ref = workloads.fetch(d)
    call = m.prepare(w, d)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        call.on(side)()
    for i in range(4):
        d["cache"].zero_()
        d["tokens"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c, t = workloads.fetch(d)
        assert np.array_equal(t, t_ref), i
        assert np.array_equal(c, c_ref), i
        workloads.run(w, d)          # eager work between replays
        torch.cuda.synchronize()
    assert not d["workspace"].cpu().numpy()[m.TABLES_BYTES:].any()       # slots left zeroed


@pytest.mark.parametrize("mult,softcap,stamped", [(1.0, 30.0, True), (0.75, 30.0, True),
                                                  (1.0, 0.5, True), (1.25, 0.0, True),
                                                  (1.0, 30.0, False), (0.75, 30.0, False)])
def test_transform_exhaustive_over_bf16(dev, mult, softcap, stamped):
    """Every finite bf16 base logit through the kernel with a zero bias: the
    cached value is the oracle's transform of it (multiplier, soft cap,
    rounding) within one bf16 ulp, and the mismatch count is reported. With
    the workspace stamped for this (mult, softcap) the kernel looks the soft
    cap up in the host-built table and must match exactly; with a workspace
    stamped for no cap it evaluates the transform itself."""
    import oracle

    vals = np.array([b for b in range(0x10000) if (b & 0x7F80) != 0x7F80], dtype=np.uint16)
    V = (len(vals) // 8) * 8
    vals = vals[:V]
    R = 16
    w = workloads.make("tiny", V=V, R=R, rows=1, k=1, data_seed=77)
    w.name = "transform"
    w.w1 = np.zeros((V, R), dtype=np.uint16)
    w.w2 = np.zeros((V, R), dtype=np.uint16)
    w.base = vals.reshape(1, 1, V).copy()
    w.temperature = np.zeros(1, dtype=np.float32)
    w.mult, w.softcap = mult, softcap
    d = workloads.to_device(w, dev)
    if not stamped:
        d["workspace"] = m.new_workspace(w.rows, w.V, w.R, w.k, device=dev)
    workloads.run(w, d)
    torch.cuda.synchronize()
    cg, tg = workloads.fetch(d)
    co = np.array([oracle.cache_value(int(b), 0, mult, softcap) for b in vals], dtype=np.uint16)
    beyond, differ = parity.compare_cache(cg[0, 0], co)
    say(f"  transform mult={mult} cap={softcap}: differing {differ}/{V}, beyond one ulp {beyond}")
    bad = np.nonzero(cg[0, 0] != co)[0][:12]
    for i in bad:
        say(f"    base {vals[i]:#06x} ({parity.bf16_to_f32(vals[i:i+1])[0]:.6g}) gpu {cg[0, 0, i]:#06x} oracle {co[i]:#06x}")
    assert beyond == 0
    assert differ <= (0 if (stamped and softcap > 0) else V // 1000)
    assert tg[0, 0] == int(np.argmax(parity.bf16_to_f32(cg[0, 0])))
