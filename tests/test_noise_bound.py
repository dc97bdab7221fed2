"""The step kernel's noise bound tables, on the host, against the oracle.

The kernel does not compute the Gumbel noise -lb of most elements. It bounds
it from above by a table entry for the bucket of the hash h (h = 0, else the
exponent and top 6 mantissa bits of the nearest binary32 to h), and takes
exact keys only where a bound reaches the best exact key. Two tables:
  - per bucket a line (A, B): the bound of h is RN32(fma(B, float(h), A));
  - per bucket a constant C (the largest noise of the bucket plus 1e-5), used
    by the plans short of registers.
These tests pin every entry to the oracle's definition of the noise: in each
bucket, at the hashes where a line is most likely to fall short (the
bucket's ends) and at others across it, the oracle's noise lies below both
bounds by at least the 1e-5 left for rounding the key. No GPU is needed: the
tables are host data.
"""

import numpy as np
import pytest

import markov_draft_sampling_step_amd as m

BASE = 8127
N = 2050


@pytest.fixture(scope="module")
def table():
    if not __import__("os").path.exists(m.LIBRARY):
        from markov_draft_sampling_step_amd import build

        build.build()
    return m.debug_noise_table()          # float32 [N, 3]: A, B, C


def bucket_of(h: np.ndarray) -> np.ndarray:
    bits = np.asarray(h, dtype=np.uint32).astype(np.float32).view(np.uint32)
    return np.maximum(bits >> np.uint32(17), np.uint32(BASE)).astype(np.int64) - BASE


def line_bound(table, b: int, h: int) -> float:
    """The kernel's binary32 evaluation of bucket b's line at h: B * float(h)
    is exact in binary64, so one binary64 addition rounded to binary32 gives
    the fused result (a double rounding could move it by an ulp, far inside
    the margin tested)."""
    A, B = float(table[b, 0]), float(table[b, 1])
    fh = float(np.float32(h))
    return float(np.float32(B * fh + A))


def bucket_starts() -> np.ndarray:
    """starts[b] = the smallest h in bucket b or above (b = 0 .. N-1), found
    by scanning the rounding boundary below each bucket's binary32 value.
    Buckets of fractional values (between small integers) are empty: their
    start is the next bucket's."""
    starts = np.zeros(N + 1, dtype=np.int64)
    for b in range(1, N):
        F = np.array([(b + BASE) << 17], dtype=np.uint32).view(np.float32)[0]
        lo = int(np.floor(np.float64(np.nextafter(F, np.float32(0)))))
        cand = np.arange(max(0, lo - 2), lo + 300, dtype=np.int64)
        cand = cand[cand < 2 ** 32]
        hit = cand[bucket_of(cand) >= b]
        assert hit.size, b
        starts[b] = hit[0]
    starts[N] = 2 ** 32
    return starts


@pytest.fixture(scope="module")
def starts():
    return bucket_starts()


def samples(lo: int, hi: int, rng) -> set:
    hs = {lo, hi, min(lo + 1, hi), max(hi - 1, lo), (lo + hi) // 2}
    if hi > lo:
        hs.update(int(x) for x in rng.integers(lo, hi + 1, size=10))
    return hs


def test_buckets_cover_all_hashes(starts):
    assert starts[0] == 0 and starts[1] == 1
    assert np.all(np.diff(starts) >= 0)
    nonempty = np.diff(starts) > 0
    assert bucket_of(starts[:-1][nonempty]).tolist() == np.nonzero(nonempty)[0].tolist()
    assert nonempty.sum() > 1700                           # 1729: small h leave gaps
    assert bucket_of(np.array([0, 1, 2 ** 24, 2 ** 32 - 129, 2 ** 32 - 128, 2 ** 32 - 1])).tolist() == \
        [0, 1, bucket_of(np.array([2 ** 24]))[0], 2048, 2049, 2049]


def test_tables_bound_the_oracle_noise_in_every_bucket(oracle_lib, table, starts):
    import oracle

    rng = np.random.default_rng(5)
    worst_line = worst_const = np.inf
    for b in range(N):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi < lo:
            continue
        assert table[b, 1] <= 0.0, b                     # the line falls with h
        for h in samples(lo, hi, rng):
            g = oracle.gumbel_key(0.0, 1.0, h)           # = -lb, the definition's noise
            s_line = line_bound(table, b, h) - g
            s_const = float(table[b, 2]) - g
            worst_line = min(worst_line, s_line)
            worst_const = min(worst_const, s_const)
            assert s_line >= 0.9e-5, (b, h, g, s_line)
            assert s_const >= 0.9e-5, (b, h, g, s_const)
    assert worst_line < 1e-4 and worst_const < 1e-4      # tight somewhere


def test_line_is_tight(oracle_lib, table, starts):
    """Not needed for correctness: the line is only worth its cost if it is
    much closer than a constant. The noise is convex in u below 1 - 1/e and
    concave above, and smooth on the scale of a bucket below u = 0.9: there
    the line stays within 1e-4 of it (3e-4 above u = 0.8, where the chord of
    the concave part is lifted by its sag), while the constant, the noise's
    fall across a bucket, reaches about 0.03."""
    import oracle

    rng = np.random.default_rng(6)
    widest_const = 0.0
    for b in range(N):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi < lo or hi >= 0.9 * 2 ** 32:
            continue
        tol = 1e-4 if hi < 0.8 * 2 ** 32 else 3e-4
        for h in samples(lo, hi, rng):
            g = oracle.gumbel_key(0.0, 1.0, h)
            assert line_bound(table, b, h) - g <= tol, (b, h)
            widest_const = max(widest_const, float(table[b, 2]) - g)
    assert widest_const > 0.01                            # the line is worth it


def test_constant_is_the_noise_at_the_bucket_start(oracle_lib, table, starts):
    """The noise falls as h grows, so a bucket's largest noise is at its first
    hash; the constant sits 1e-5 (and a rounding up) above it."""
    import oracle

    for b in range(N):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi < lo:
            continue
        d = float(table[b, 2]) - oracle.gumbel_key(0.0, 1.0, lo)
        assert 0.99e-5 <= d <= 1.3e-5, (b, d)


def test_extreme_entries(table, starts):
    # h = 0: u = 2^-33, the largest noise, a one-hash bucket (flat line); the
    # top bucket: u rounds to 1 and the clamp gives -log(24 ln 2)
    g0 = -np.log(-np.log1p(-2.0 ** -33))
    assert table[0, 1] == 0.0 and 1e-5 <= table[0, 0] - g0 < 3e-5
    gtop = -np.log(24 * np.log(2.0))
    top = line_bound(table, N - 1, 2 ** 32 - 1)
    assert 0.0 < top - gtop < 1e-3
    c = table[:, 2][np.diff(starts) > 0]
    assert np.all(np.diff(c) <= 0)                        # the noise falls as h grows
