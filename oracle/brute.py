"""Brute-force statement of one Markov draft step, for tiny vocabularies.

TEST INFRASTRUCTURE ONLY. A second, independent reading of the definition
the C oracle follows, written for checking by eye rather than speed: every
binary32 / bf16 operation is an exact rational result rounded once by
``rn`` below, logs and tanh come from mpmath at 200 bits and are rounded
once (correctly rounded, not via binary64), MurmurHash3 is restated from its
public definition, and the argmax is a sort under the total order.

Sources: vLLM API pages "vllm.models.kimi_k3.nvidia.specialized_decode.
drafter.markov" (`_gumbel_key`, `_loop_rest`, exactness paragraph) and
"vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.draft.markov"
(`_logit`, `_gumbel`, `_murmur_prefix`, `_combine`, `_w1_row`).
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

import mpmath

mpmath.mp.prec = 200

NAN = float("nan")


# -- exact rounding ------------------------------------------------------------

def rn(q: Fraction, mant_bits: int, emin: int, emax: int) -> float:
    """Round an exact rational to the nearest value of a binary format with
    `mant_bits` significand bits (implicit bit included), normal exponents
    [emin, emax], subnormals below; ties to even; overflow to infinity."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1)
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * quantum
    if val >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(val)


def rn32(q) -> float:
    """Nearest binary32 value (returned as a Python float, exactly)."""
    return rn(Fraction(q), 24, -126, 127)


def rnbf(q) -> float:
    """Nearest bf16 value."""
    return rn(Fraction(q), 8, -126, 127)


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bf_bits(x: float) -> int:
    """bf16 bit pattern of a value that is exactly a bf16 (or NaN)."""
    if math.isnan(x):
        return 0x7FC0
    return f32_bits(x) >> 16


def bf_value(b: int) -> float:
    return bits_f32((b & 0xFFFF) << 16)


def mp_round32(v) -> float:
    """Correctly rounded binary32 of an mpmath value (200-bit)."""
    sign, man, exp, _ = mpmath.mpf(v)._mpf_
    q = Fraction(int(man)) * Fraction(2) ** int(exp)
    return rn32(-q if sign else q)


def log_cr(x: float) -> float:
    return mp_round32(mpmath.log(mpmath.mpf(x)))


def tanh_cr(x: float) -> float:
    return mp_round32(mpmath.tanh(mpmath.mpf(x)))


# -- MurmurHash3_x86_32 from its public definition ------------------------------

def murmur3(data: bytes, seed: int = 0) -> int:
    M = 0xFFFFFFFF

    def rotl(x, r):
        return ((x << r) | (x >> (32 - r))) & M

    h = seed & M
    n4 = len(data) // 4
    for i in range(n4):
        k = int.from_bytes(data[4 * i: 4 * i + 4], "little")
        k = (k * 0xCC9E2D51) & M
        k = rotl(k, 15)
        k = (k * 0x1B873593) & M
        h ^= k
        h = rotl(h, 13)
        h = (h * 5 + 0xE6546B64) & M
    tail = data[4 * n4:]
    if tail:
        k = int.from_bytes(tail, "little")
        k = (k * 0xCC9E2D51) & M
        k = rotl(k, 15)
        k = (k * 0x1B873593) & M
        h ^= k
    h ^= len(data)
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & M
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & M
    h ^= h >> 16
    return h


def noise_hash(seed: int, step: int, position: int, token: int) -> int:
    S = (seed & 0xFFFFFFFFFFFFFFFF) ^ ((step & 0xFFFFFFFF) << 32)
    P = (position - 1 + (1 << 30)) & 0xFFFFFFFF
    msg = struct.pack("<IIII", S & 0xFFFFFFFF, S >> 32, P, token & 0xFFFFFFFF)
    return murmur3(msg, 0)


# -- the step ---------------------------------------------------------------------

def uniform(h: int) -> float:
    return rn32(Fraction(2 * h + 1, 2 ** 33))


def log1m(u: float) -> float:
    if u < 0.25:
        p = rn32(Fraction(1, 8))
        for k in (7, 6, 5, 4, 3, 2, 1):
            p = rn32(Fraction(u) * Fraction(p) + Fraction(rn32(Fraction(1, k))))
        return rn32(Fraction(p) * Fraction(-u))
    om = rn32(Fraction(1) - Fraction(u))
    return log_cr(max(om, 2.0 ** -24))


def key(l: float, T: float, h: int) -> float:
    if T == 0.0 and not math.isnan(T):
        return l
    if math.isnan(l) or math.isnan(T):
        return NAN
    u = uniform(h)
    L = log1m(u)
    lb = log_cr(-L)
    q = rn32(Fraction(l) / Fraction(T))
    return rn32(Fraction(q) - Fraction(lb))


def cache_value(base_bits: int, bias_bits: int, mult: float, softcap: float) -> float:
    a, b = bf_value(base_bits), bf_value(bias_bits)
    if math.isnan(a) or math.isnan(b):
        return NAN
    x = rnbf(Fraction(a) + Fraction(b))            # one rounding of the exact sum
    y = rn32(Fraction(mult) * Fraction(x))
    w = y
    if softcap > 0:
        inv = rn32(Fraction(1) / Fraction(softcap))
        z = rn32(Fraction(y) * Fraction(inv))
        w = rn32(Fraction(softcap) * Fraction(tanh_cr(z)))
    return rnbf(w)


def bias(e_bits, w_bits) -> float:
    acc = 0.0
    for eb, wb in zip(e_bits, w_bits):
        acc = rn32(Fraction(acc) + Fraction(bf_value(int(eb))) * Fraction(bf_value(int(wb))))
    return rnbf(acc)


def order_key(v: float, i: int):
    """Sort key: the first element of a sorted list is the argmax (first
    NaN, else the largest value, ties and -0 == +0 to the lowest id)."""
    if math.isnan(v):
        return (0, 0.0, i)
    return (1, -v, i)


def step(base_row, w1, w2, prev: int, seed: int, position: int, step_index: int,
         T: float, mult: float = 1.0, softcap: float = 0.0):
    """One row, one step. Returns (cache bf16 bits list, keys list, token)."""
    V = len(base_row)
    row = min(prev & 0xFFFFFFFFFFFFFFFF, V - 1)      # unsigned clamp to the last row
    e = [int(x) for x in w1[row]]
    cache, keys = [], []
    for v in range(V):
        b = bias(e, [int(x) for x in w2[v]])
        c = cache_value(int(base_row[v]), bf_bits(b), mult, softcap)
        cache.append(bf_bits(c))
        keys.append(key(c, T, noise_hash(seed, step_index, position, v)))
    token = sorted(range(V), key=lambda v: order_key(keys[v], v))[0]
    return cache, keys, token


# -- spacing of the formats, from the definition ----------------------------------

def _binade(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return e


def ulp32(x: float) -> float:
    """Gap between the binary32 values around |x| in its binade: 2^(e-23)
    for 2^e <= |x| < 2^(e+1), e clamped at the smallest normal exponent -126
    (so 2^-149 across the subnormals and at zero)."""
    a = Fraction(abs(x))
    e = -126 if a == 0 else max(_binade(a), -126)
    return float(Fraction(2) ** (e - 23))


def ulp_bf16(x: float) -> float:
    """The same for bf16 (8 significand bits): 2^(e-7), 2^-133 at the bottom."""
    a = Fraction(abs(x))
    e = -126 if a == 0 else max(_binade(a), -126)
    return float(Fraction(2) ** (e - 7))


# -- FP8 (E4M3) w2 with an FP16 row scale ----------------------------------------
# TensorRT Edge-LLM "DSpark kernels" page: `dsparkQuantizeMarkovW2Fp8`,
# `dsparkMarkovGreedyFusedStepFp8`. Closed forms of the formats, exact
# rationals, a bisection over the sorted code values.

def e4m3_value(c: int):
    """Exact value of an E4M3 code (Fraction), or None for NaN."""
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


_E4M3_POS = [(e4m3_value(c), c) for c in range(0x7F)]        # rising values, codes 0 .. 0x7E


def e4m3_encode(x: float) -> int:
    if math.isnan(x):
        return 0xFF if math.copysign(1.0, x) < 0 else 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x)) if not math.isinf(x) else Fraction(10 ** 6)
    if a >= 448:
        return sign | 0x7E
    import bisect

    vals = [v for v, _ in _E4M3_POS]
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | _E4M3_POS[i][1]
    lo, hi = _E4M3_POS[i - 1], _E4M3_POS[i]
    dl, dh = a - lo[0], hi[0] - a
    pick = lo if dl < dh else hi if dh < dl else (lo if lo[1] % 2 == 0 else hi)
    return sign | pick[1]


def fp16_rn(q) -> float:
    """Nearest binary16 value (11 significand bits, exponents -14 .. 15)."""
    return rn(Fraction(q), 11, -14, 15)


def quantize_row(w_bits):
    """(codes, scale value) of a bf16 row."""
    amax = max(abs(Fraction(bf_value(int(b)))) for b in w_bits)
    scale = fp16_rn(amax / 448)
    if scale == 0:
        return [0] * len(w_bits), 0.0
    return [e4m3_encode(rn32(Fraction(bf_value(int(b))) / Fraction(scale))) for b in w_bits], scale


def bias_fp8(e_bits, codes, scale: float) -> float:
    acc = 0.0
    for eb, c in zip(e_bits, codes):
        acc = rn32(Fraction(acc) + Fraction(bf_value(int(eb))) * e4m3_value(int(c)))
    return rnbf(rn32(Fraction(scale) * Fraction(acc)))


def step_fp8(base_row, w1, codes, scales, prev: int, seed: int, position: int, step_index: int,
             T: float, mult: float = 1.0, softcap: float = 0.0):
    """One row, one step with an E4M3 w2 (codes [V][R], scale values [V])."""
    V = len(base_row)
    row = min(prev & 0xFFFFFFFFFFFFFFFF, V - 1)
    e = [int(x) for x in w1[row]]
    cache, keys = [], []
    for v in range(V):
        b = bias_fp8(e, [int(c) for c in codes[v]], float(scales[v]))
        c = cache_value(int(base_row[v]), bf_bits(b), mult, softcap)
        cache.append(bf_bits(c))
        keys.append(key(c, T, noise_hash(seed, step_index, position, v)))
    token = sorted(range(V), key=lambda v: order_key(keys[v], v))[0]
    return cache, keys, token
