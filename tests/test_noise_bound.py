"""The step kernel's noise bound table, on the host, against the oracle.

The kernel does not compute the Gumbel noise -lb of most elements. It reads
an upper bound of it from a table indexed by the bucket of the hash h (h = 0,
else the exponent and top 6 mantissa bits of the nearest binary32 to h), and
takes exact keys only where a bound reaches the best exact key. These tests
pin every table entry to the oracle's definition of the noise: in each
bucket, at the hash where the noise is largest (the bucket's smallest h, as
the noise falls with u) and at others across the bucket, the oracle's noise
lies below the entry by at least 1e-5 (the part of the kernel's margin left
for rounding the key). No GPU is needed: the table is host data.
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
    return m.debug_noise_table().astype(np.float64)


def bucket_of(h: np.ndarray) -> np.ndarray:
    bits = np.asarray(h, dtype=np.uint32).astype(np.float32).view(np.uint32)
    return np.maximum(bits >> np.uint32(17), np.uint32(BASE)).astype(np.int64) - BASE


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


def test_buckets_cover_all_hashes(starts):
    assert starts[0] == 0 and starts[1] == 1
    assert np.all(np.diff(starts) >= 0)
    nonempty = np.diff(starts) > 0
    assert bucket_of(starts[:-1][nonempty]).tolist() == np.nonzero(nonempty)[0].tolist()
    assert nonempty.sum() > 1700                           # 1729: small h leave gaps
    assert bucket_of(np.array([0, 1, 2 ** 24, 2 ** 32 - 129, 2 ** 32 - 128, 2 ** 32 - 1])).tolist() == \
        [0, 1, bucket_of(np.array([2 ** 24]))[0], 2048, 2049, 2049]


def test_table_bounds_the_oracle_noise_in_every_bucket(oracle_lib, table, starts):
    import oracle

    rng = np.random.default_rng(5)
    worst_slack = np.inf
    for b in range(N):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi < lo:
            continue
        hs = {lo, hi, min(lo + 1, hi), (lo + hi) // 2}
        if hi > lo:
            hs.update(int(x) for x in rng.integers(lo, hi + 1, size=8))
        for h in hs:
            g = oracle.gumbel_key(0.0, 1.0, h)           # = -lb, the definition's noise
            slack = table[b] - g
            worst_slack = min(worst_slack, slack)
            assert slack >= 1e-5, (b, h, g, table[b])
    assert worst_slack < 5e-5                              # tight at some bucket start


def test_table_is_tight(oracle_lib, table, starts):
    """Not needed for correctness: the bound is only useful if it is close.
    At each bucket's start the slack is the 3e-5 margin (plus one rounding);
    across a bucket it is the noise's variation over the bucket, below 0.04
    for u < 0.9."""
    import oracle

    for b in range(N):
        lo, hi = int(starts[b]), int(starts[b + 1]) - 1
        if hi < lo:
            continue
        g_lo = oracle.gumbel_key(0.0, 1.0, lo)
        assert table[b] - g_lo <= 3e-5 + 4e-6, b
        if hi < 0.9 * 2 ** 32:
            assert table[b] - oracle.gumbel_key(0.0, 1.0, hi) <= 0.04, b


def test_extreme_entries(table):
    # h = 0: u = 2^-33, the largest noise; the top bucket: u rounds to 1 and
    # the clamp gives -log(24 ln 2)
    assert abs(table[0] - (-np.log(-np.log1p(-2.0 ** -33)) + 3e-5)) < 1e-5
    assert abs(table[N - 1] - (-np.log(24 * np.log(2.0)) + 3e-5)) < 1e-5
    assert np.all(np.diff(table) <= 0)                     # the noise falls as h grows
