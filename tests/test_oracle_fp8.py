"""Pins of the oracle's E4M3 w2 path (TensorRT Edge-LLM "DSpark kernels"
page: `dsparkQuantizeMarkovW2Fp8`, `dsparkMarkovGreedyFusedStepFp8`) to the
formats' definitions and to the brute-force statement (exact rationals)."""

import math
import struct
from fractions import Fraction

import numpy as np
import pytest


def f32(x):
    return float(np.float32(x))


def test_e4m3_decode_every_code(oracle_lib):
    from oracle import brute

    for c in range(256):
        v = brute.e4m3_value(c)
        got = oracle_lib.e4m3_decode(c)
        if v is None:
            assert math.isnan(got), c
        else:
            assert got == float(v), c
    # the format's landmarks: largest finite, smallest normal and subnormal, one
    assert oracle_lib.e4m3_decode(0x7E) == 448.0 and oracle_lib.e4m3_decode(0xFE) == -448.0
    assert oracle_lib.e4m3_decode(0x08) == 2.0 ** -6 and oracle_lib.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle_lib.e4m3_decode(0x38) == 1.0 and oracle_lib.e4m3_decode(0x80) == 0.0
    # every finite E4M3 value is a bf16 value (so the products with bf16 are exact in binary32)
    for c in range(256):
        v = oracle_lib.e4m3_decode(c)
        if not math.isnan(v):
            assert brute.rnbf(Fraction(v)) == v


def _encode_inputs(rng):
    from oracle import brute

    xs = [brute.bf_value(b) for b in range(0x10000)]                     # every bf16
    vals = sorted(float(brute.e4m3_value(c)) for c in range(0x7F))
    for a, b in zip(vals, vals[1:]):                                    # exact ties and near them
        mid = (a + b) / 2
        xs += [mid, -mid, f32(np.nextafter(np.float32(mid), np.float32(0))),
               f32(np.nextafter(np.float32(mid), np.float32(1e9)))]
    xs += [447.0, 448.0, 449.0, 463.9, 464.0, 465.0, 1e30, float("inf"), -float("inf"),
           2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -149, -0.0, 0.0]
    xs += [f32(x) for x in rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000)]
    return [f32(x) if not math.isnan(x) else x for x in xs]


def test_e4m3_encode_nearest_even_saturating(oracle_lib):
    from oracle import brute

    rng = np.random.default_rng(51)
    for x in _encode_inputs(rng):
        got, want = oracle_lib.e4m3_encode(x), brute.e4m3_encode(x)
        if math.isnan(x):
            assert (got & 0x7F) == 0x7F
        else:
            assert got == want, (x, hex(got), hex(want))


def test_fp16_rounding(oracle_lib):
    from oracle import brute

    rng = np.random.default_rng(52)
    xs = [brute.bf_value(b) for b in range(0, 0x10000, 3)]
    xs += [65504.0, 65519.0, 65520.0, 65536.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14,
           1 / 3, 1e-9]
    xs += list(rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000))
    for x in xs:
        if math.isnan(x):
            continue
        got = oracle_lib.fp16_to_f32(oracle_lib.fp16_round(x))
        assert got == (x if math.isinf(x) else brute.fp16_rn(Fraction(x))), x
    for h in range(0x10000):                                             # decode against the closed form
        s, e, m = h >> 15, (h >> 10) & 31, h & 1023
        v = oracle_lib.fp16_to_f32(h)
        if e == 31:
            assert math.isinf(v) if m == 0 else math.isnan(v)
            continue
        want = (m * 2.0 ** -24) if e == 0 else (1 + m / 1024) * 2.0 ** (e - 15)
        assert v == (-want if s else want), hex(h)


def test_row_scale_is_one_rounding_of_absmax_over_448(oracle_lib):
    """The scale of every possible row maximum (each positive bf16) is the
    FP16 value nearest the exact quotient rowAbsMax / 448."""
    from oracle import brute

    for b in range(1, 0x7F80, 7):
        a = brute.bf_value(b)
        row = np.array([b, 0, b ^ 0x8000, 0], dtype=np.uint16)
        q = np.zeros(4, dtype=np.uint8)
        sbits = oracle_lib.lib().oracle_quantize_row_fp8(row.ctypes.data, 4, q.ctypes.data)
        assert oracle_lib.fp16_to_f32(sbits) == brute.fp16_rn(Fraction(a) / 448), hex(b)


def test_quantized_rows_match_brute(oracle_lib):
    from oracle import brute
    from markov_draft_sampling_step_amd.workloads import to_bf16_bits

    rng = np.random.default_rng(53)
    rows = [to_bf16_bits(rng.standard_normal(32).astype(np.float32) * s) for s in (0.02, 1.0, 300.0)]
    rows.append(np.zeros(16, dtype=np.uint16))                            # zero row: scale 0, codes 0
    tiny = to_bf16_bits(np.float32([1e-6, -3e-7, 2e-6, 0.0] * 4))          # scale below FP16 range
    rows.append(tiny)
    one = np.zeros(16, dtype=np.uint16)
    one[5] = to_bf16_bits(np.float32([-7.5]))[0]                          # a single non-zero
    rows.append(one)
    for w in rows:
        codes, scale = brute.quantize_row(list(w))
        q, sbits = oracle_lib.quantize_w2_fp8(w.reshape(1, -1))
        assert oracle_lib.fp16_to_f32(int(sbits[0])) == scale
        assert list(q[0]) == codes
    # the full-range property: the row maximum maps to +-448 (or just below)
    w = rows[1]
    q, _ = oracle_lib.quantize_w2_fp8(w.reshape(1, -1))
    assert max(abs(oracle_lib.e4m3_decode(int(c))) for c in q[0]) >= 416.0


def test_fp8_bias_brute_and_quantization_error(oracle_lib):
    """The E4M3 bias equals the brute-force one (R <= 32), lies within the
    summation-order bound of its exact scaled dot, and within the
    quantization error of the bf16 bias."""
    from oracle import brute
    from markov_draft_sampling_step_amd.workloads import to_bf16_bits

    rng = np.random.default_rng(54)
    for R in (16, 32, 256):
        for _ in range(40):
            e = to_bf16_bits(rng.standard_normal(R).astype(np.float32) * 0.02)
            w = to_bf16_bits(rng.standard_normal(R).astype(np.float32) * 0.02)
            q, sc = oracle_lib.quantize_w2_fp8(w.reshape(1, -1))
            b8, s64, sabs = oracle_lib.bias_fp8(e, q[0], int(sc[0]))
            scale = oracle_lib.fp16_to_f32(int(sc[0]))
            v8 = brute.bf_value(b8)
            if R <= 32:
                assert v8 == brute.bias_fp8(list(e), list(q[0]), scale)
            exact = sum(Fraction(brute.bf_value(int(x))) * brute.e4m3_value(int(c)) for x, c in zip(e, q[0]))
            gam = Fraction(R, 2 ** 24) / (1 - Fraction(R, 2 ** 24))
            lo = Fraction(scale) * (exact - gam * Fraction(sabs))
            hi = Fraction(scale) * (exact + gam * Fraction(sabs))
            assert brute.rnbf(brute.rn32(min(lo, hi))) <= v8 <= brute.rnbf(brute.rn32(max(lo, hi)))
            b16, _, _ = oracle_lib.bias(e, w)
            err = sum(abs(brute.bf_value(int(x))) * (abs(brute.bf_value(int(y))) * 2.0 ** -4 + scale * 2.0 ** -10)
                      for x, y in zip(e, w))
            assert abs(v8 - brute.bf_value(b16)) <= 2 * err + 2 * brute.ulp_bf16(v8) + 1e-30


@pytest.mark.slow
def test_fp8_step_matches_brute_on_tiny_inputs(oracle_lib):
    from oracle import brute
    from markov_draft_sampling_step_amd.workloads import to_bf16_bits

    rng = np.random.default_rng(55)
    for i, (V, R, rows, k) in enumerate(((7, 16, 2, 2), (64, 32, 2, 2), (33, 16, 1, 3))):
        w1 = to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.3)
        w2 = to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * 0.3)
        base = to_bf16_bits(rng.standard_normal((rows, k, V)).astype(np.float32) * 2)
        base[0, 0, 1] = base[0, 0, 4] = 0x7FC0
        q, sc = oracle_lib.quantize_w2_fp8(w2)
        prev = rng.integers(-2, V + 2, size=rows).astype(np.int64)
        seeds = rng.integers(0, 2 ** 40, size=rows).astype(np.int64)
        pos = (rng.integers(0, 5000, size=rows)[:, None] + np.arange(k)[None, :]).astype(np.int64)
        temp = np.array([[0.0, 1.0, 0.7][(r + i) % 3] for r in range(rows)], dtype=np.float32)
        cap = 30.0 if i == 1 else 0.0
        feed = [int(p) for p in prev]
        scales = [oracle_lib.fp16_to_f32(int(x)) for x in sc]
        for s in range(k):
            out = oracle_lib.step(np.ascontiguousarray(base[:, s]), w1, None, np.array(feed),
                                  seeds, np.ascontiguousarray(pos[:, s]), s, temp, 1.0, cap,
                                  w2q=q, w2s=sc)
            for r in range(rows):
                c_b, _, t_b = brute.step_fp8(base[r, s], w1, q, scales, feed[r], int(seeds[r]),
                                             int(pos[r, s]), s, float(temp[r]), 1.0, cap)
                for v in range(V):
                    a, b = int(out["cache"][r, v]), int(c_b[v])
                    assert a == b or ((a & 0x7F80) == 0x7F80 and (a & 0x7F) and (b & 0x7F80) == 0x7F80), (i, r, s, v)
                assert out["tokens"][r] == t_b, (i, r, s)
            feed = [int(t) for t in out["tokens"]]
