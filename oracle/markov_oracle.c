/*
 * Oracle for the DSpark sequential Markov draft-sampling step.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously-correct CPU
 * statement of what one draft step computes. Only the tests, the smoke check
 * and the CPU-baseline leg of the benchmark may load it. It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * the seeded inputs the tests hand to both.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Contraction is off so every float expression below rounds exactly where it
 * is written; x86-64 evaluates float in SSE (no excess precision).
 *
 * Sources (the pages this follows; sections named, not line-numbered):
 *   [KIMI]  vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.
 *           drafter.markov": module docstring (exactness paragraph),
 *           `_gumbel_key`, `_gumbel_log_arg32`, `_loop_rest`.
 *   [MUSE]  vLLM API page "vllm.models.muse_spark.nvidia.specialized_decode.
 *           cutedsl.draft.markov": module docstring, `_StepKernel.kernel`,
 *           `_logit`, `_gumbel`, `_murmur_prefix`, `_nonzero_f32`,
 *           `_combine`, `_w1_row`.
 *   [DSV41] vLLM API page "vllm.models.deepseek_v41.amd.ops.fused_markov":
 *           module docstring, `_loop_rest`.
 *
 * Readings taken where the pages leave a step open (each repeated at its
 * function):
 *   - the block step of MurmurHash3_x86_32 is not printed; the public
 *     MurmurHash3_x86_32 definition is used (its finaliser constants are the
 *     ones [MUSE] `_gumbel` prints);
 *   - logs and tanh are the correctly rounded binary32 values (the pages'
 *     own libdevice routines are NVIDIA code and are not reproduced);
 *   - the division logit / temperature is IEEE round-to-nearest;
 *   - the bias sum is taken in index order j = 0..R-1 in binary32 (the pages
 *     leave the order free);
 *   - parity with vLLM's own draws is unpinned: no page prints a value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> binary32 is exact: the bf16 pattern is the high half of the float. */
EXPORT float oracle_bf16_to_f32(uint16_t b) { return bits_to_f32((uint32_t)b << 16); }

/*
 * binary32 -> bf16, round to nearest, ties to even, as the pages' conversions
 * do ([MUSE] `_logit`: the cache value is a round-to-nearest bf16 of the
 * transformed logit). Written from the definition: take the two bf16 values
 * that bracket x (truncation toward zero, and one bf16 ulp further from
 * zero), and keep the nearer one; on an exact tie keep the one with an even
 * last bit. Distances are computed in binary64, where they are exact (both
 * operands carry at most 24 significant bits within a factor of 2).
 * Overflow follows IEEE: the value one ulp past the largest finite bf16 is
 * 2^128, and it rounds to infinity. NaN stays NaN (quiet, same sign).
 */
EXPORT uint16_t oracle_bf16_round(float x) {
  uint32_t u = f32_to_bits(x);
  if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
  if (isinf(x)) return (uint16_t)(u >> 16);
  uint16_t lo = (uint16_t)(u >> 16);            /* toward zero */
  uint16_t hi = (uint16_t)(lo + 1u);            /* away from zero */
  double dx = fabs((double)x);
  double dlo = fabs((double)oracle_bf16_to_f32(lo));
  double dhi;
  if ((hi & 0x7fffu) == 0x7f80u)
    dhi = ldexp(1.0, 128);                      /* one ulp past the top */
  else
    dhi = fabs((double)oracle_bf16_to_f32(hi));
  double below = dx - dlo, above = dhi - dx;
  if (below < above) return lo;
  if (above < below) return hi;
  return (lo & 1u) ? hi : lo;
}

/* Unit in the last place of a binary32 magnitude: the spacing of the
 * binary32 values in |x|'s binade (the gap above |x|; at the largest finite
 * value, which has no finite successor, the gap below it, the same binade). */
EXPORT double oracle_ulp32(float x) {
  float a = fabsf(x);
  if (isnan(a) || isinf(a)) return INFINITY;
  float n = nextafterf(a, INFINITY);
  if (isinf(n)) return (double)a - (double)nextafterf(a, 0.0f);
  return (double)n - (double)a;
}

/* Unit in the last place of a bf16 magnitude. */
EXPORT double oracle_ulp_bf16(float x) {
  float a = fabsf(x);
  if (isnan(a) || isinf(a)) return INFINITY;
  uint16_t b = oracle_bf16_round(a);
  float v = oracle_bf16_to_f32(b);
  if (v > a) { b = (uint16_t)(b - 1u); v = oracle_bf16_to_f32(b); }
  uint16_t n = (uint16_t)(b + 1u);
  double vn = ((n & 0x7fffu) == 0x7f80u) ? ldexp(1.0, 128) : (double)oracle_bf16_to_f32(n);
  return vn - (double)v;
}

/*
 * Correctly rounded binary32 log and tanh (see the readings above). The
 * binary64 library value, good to under one binary64 ulp, rounds to the
 * right binary32 unless it lies within a few binary64 ulps of a binary32
 * rounding midpoint; there (two inputs on the step's whole log domain) the
 * 64-bit-significand long double routine decides the rounding.
 */
static int near_midpoint(double y) {
  float f = (float)y;
  if (isnan(f) || isinf(f)) return 0;
  double fd = (double)f;
  double up = (double)nextafterf(f, INFINITY), dn = (double)nextafterf(f, -INFINITY);
  double tol = 8.0 * (nextafter(fabs(y), INFINITY) - fabs(y));
  return fabs(y - 0.5 * (fd + up)) <= tol || fabs(y - 0.5 * (fd + dn)) <= tol;
}
EXPORT float oracle_logf_cr(float x) {
  double y = log((double)x);
  if (near_midpoint(y)) return (float)logl((long double)x);
  return (float)y;
}
EXPORT float oracle_tanhf_cr(float x) {
  double y = tanh((double)x);
  if (near_midpoint(y)) return (float)tanhl((long double)x);
  return (float)y;
}

/* ------------------------------------------------------------------------ */
/* Noise: MurmurHash3 of (seed, step, position, token id)                    */
/* ------------------------------------------------------------------------ */

static uint32_t rotl32(uint32_t x, int r) { return (x << r) | (x >> (32 - r)); }

/*
 * MurmurHash3_x86_32 of `len` bytes, written from its public definition:
 * 4-byte little-endian blocks, each scrambled (x c1, rotl 15, x c2), xored
 * into the state, which is rotated left 13 and advanced as h*5 + 0xe6546b64;
 * then the 1-3 tail bytes; then h ^= len and the fmix32 finaliser (the two
 * finaliser multipliers 0x85ebca6b and 0xc2b2ae35 are the ones [MUSE]
 * `_gumbel` prints as signed decimals).
 */
EXPORT uint32_t oracle_murmur3_x86_32(const uint8_t* data, uint64_t len, uint32_t seed) {
  const uint32_t c1 = 0xcc9e2d51u, c2 = 0x1b873593u;
  uint32_t h = seed;
  uint64_t nblocks = len / 4;
  for (uint64_t i = 0; i < nblocks; ++i) {
    const uint8_t* p = data + 4 * i;
    uint32_t k = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                 ((uint32_t)p[3] << 24);
    k *= c1;
    k = rotl32(k, 15);
    k *= c2;
    h ^= k;
    h = rotl32(h, 13);
    h = h * 5u + 0xe6546b64u;
  }
  const uint8_t* tail = data + 4 * nblocks;
  uint32_t k = 0;
  switch (len & 3u) {
    case 3: k ^= (uint32_t)tail[2] << 16; /* fall through */
    case 2: k ^= (uint32_t)tail[1] << 8;  /* fall through */
    case 1:
      k ^= (uint32_t)tail[0];
      k *= c1;
      k = rotl32(k, 15);
      k *= c2;
      h ^= k;
  }
  h ^= (uint32_t)len;
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

/*
 * The hash behind one token's noise ([MUSE] `_StepKernel.kernel` and
 * `_murmur_prefix`; [KIMI] exactness paragraph): four little-endian words,
 *   lo32(S), hi32(S), lo32(P), token id,   hashed with seed 0, where
 *   S = seed XOR (step << 32)        (the step seed, step = 0-based draft step)
 *   P = (position - 1) + 2^30        (the position before the sampled token
 *                                     plus the draft salt)
 * `position` is the sample position of this row at this step.
 */
EXPORT uint32_t oracle_noise_hash(int64_t seed, int32_t step, int64_t position, uint32_t token) {
  uint64_t S = (uint64_t)seed ^ ((uint64_t)(uint32_t)step << 32);
  int64_t P = (position - 1) + ((int64_t)1 << 30);
  uint32_t words[4] = {(uint32_t)(S & 0xffffffffu), (uint32_t)(S >> 32),
                       (uint32_t)((uint64_t)P & 0xffffffffu), token};
  uint8_t bytes[16];
  for (int w = 0; w < 4; ++w)
    for (int b = 0; b < 4; ++b) bytes[4 * w + b] = (uint8_t)(words[w] >> (8 * b));
  return oracle_murmur3_x86_32(bytes, 16, 0u);
}

/*
 * The hash's uniform ([MUSE] `_gumbel`): u = RN32((h + 1/2) * 2^-32), one
 * rounding. (h + 1/2) * 2^-32 is exact in binary64, so the only rounding is
 * the conversion to binary32. h = 0 gives 2^-33; the top 128 hash values give
 * exactly 1.0.
 */
EXPORT float oracle_uniform(uint32_t h) { return (float)(((double)h + 0.5) * 0x1p-32); }

/*
 * L = log(1 - u), the stable form the pages use ([MUSE] `_gumbel`; [KIMI]
 * `_gumbel_key` calls it `_log1p_neg_stable`). For u < 1/4 (strict): the
 * Taylor series -(u + u^2/2 + ... + u^8/8), evaluated in binary32 as a Horner
 * chain of fused multiply-adds over the coefficients RN32(1/k), k = 8..1,
 * then one multiply by -u. Otherwise log(max(RN32(1 - u), 2^-24)).
 */
EXPORT float oracle_log1m(float u) {
  if (u < 0.25f) {
    const float coef[7] = {(float)(1.0 / 7.0), (float)(1.0 / 6.0), (float)(1.0 / 5.0), 0.25f,
                           (float)(1.0 / 3.0), 0.5f, 1.0f};
    float p = 0.125f;
    for (int i = 0; i < 7; ++i) p = fmaf(u, p, coef[i]);
    return p * (-u);
  }
  float om = 1.0f - u;
  float x = om > 0x1p-24f ? om : 0x1p-24f;
  return oracle_logf_cr(x);
}

/*
 * Whether a row's temperature makes it noisy: T != 0 by an ordered compare
 * ([MUSE] `_nonzero_f32`). NaN is noisy; -0.0 is not.
 */
EXPORT int oracle_noisy(float T) { return !(T == 0.0f); }

/*
 * The sampling key of a cached logit l ([KIMI] `_gumbel_key`, [MUSE]
 * `_gumbel`): at a noisy temperature, RN32(RN32(l / T) - log(-L)) where
 * L = log1m(u(h)); at T = 0 the plain logit. The noise -log(-L) is never
 * rounded separately: the subtraction of the rounded log is the one step
 * ([KIMI] `_gumbel_log_arg32` explains why a stored noise would differ).
 * `lb_out` / `L_out` (optional) receive the two log values.
 */
EXPORT float oracle_gumbel_key(float l, float T, uint32_t h, float* lb_out, float* L_out) {
  if (!oracle_noisy(T)) {
    if (lb_out) *lb_out = 0.0f;
    if (L_out) *L_out = 0.0f;
    return l;
  }
  float u = oracle_uniform(h);
  float L = oracle_log1m(u);
  float lb = oracle_logf_cr(-L);
  float q = l / T;
  if (lb_out) *lb_out = lb;
  if (L_out) *L_out = L;
  return q - lb;
}

/* ------------------------------------------------------------------------ */
/* Logits                                                                    */
/* ------------------------------------------------------------------------ */

/*
 * The Markov bias of one (row, token): the binary32 dot product of the
 * row's embedding and the token's w2 row, rounded once to bf16 ([KIMI]
 * exactness paragraph; [DSV41] module docstring). Products of two bf16 are
 * exact in binary32; the sum runs j = 0..R-1. `s64` (optional) gets the sum
 * in binary64 and `sabs` the sum of |products|, for the order-free bound.
 */
EXPORT uint16_t oracle_bias(const uint16_t* e, const uint16_t* w, int32_t R, double* s64,
                            double* sabs) {
  float acc = 0.0f;
  double d = 0.0, a = 0.0;
  for (int32_t j = 0; j < R; ++j) {
    float p = oracle_bf16_to_f32(e[j]) * oracle_bf16_to_f32(w[j]);
    acc = acc + p;
    d += (double)p;
    a += fabs((double)p);
  }
  if (s64) *s64 = d;
  if (sabs) *sabs = a;
  return oracle_bf16_round(acc);
}

/*
 * The cached logit ([MUSE] `_logit`, module docstring): the bf16 add of base
 * and bias (one binary32 add rounded to bf16, [KIMI] exactness paragraph),
 * times the multiplier, then with a soft cap cap * tanh(y * RN32(1/cap)),
 * rounded to bf16. softcap <= 0 means no cap.
 */
EXPORT uint16_t oracle_cache_value(uint16_t base, uint16_t bias, float mult, float softcap) {
  float x = oracle_bf16_to_f32(oracle_bf16_round(oracle_bf16_to_f32(base) + oracle_bf16_to_f32(bias)));
  float y = mult * x;
  float w = y;
  if (softcap > 0.0f) {
    float inv_cap = 1.0f / softcap;
    float z = y * inv_cap;
    w = softcap * oracle_tanhf_cr(z);
  }
  return oracle_bf16_round(w);
}

/* The bf16 value next to b toward +infinity (up) or -infinity (down). */
static uint16_t bf16_step(uint16_t b, int up) {
  float v = oracle_bf16_to_f32(b);
  if (v == 0.0f) return up ? (uint16_t)0x0001u : (uint16_t)0x8001u;
  int away = (v > 0.0f) == (up != 0);       /* moving away from zero */
  return (uint16_t)(away ? b + 1u : b - 1u);
}

/*
 * Whether a device's cached value c_dev of one element is one the
 * definition admits. The pages leave only the bias's summation order open
 * ([KIMI] exactness paragraph, [DSV41] module docstring: the last bf16 bit of
 * the bias may differ), so the admissible biases b' span from the lower to
 * the upper of: the oracle's bias one bf16 step down / up, and the bf16
 * roundings of the ends of [S - gamma_R sum|p|, S + gamma_R sum|p|] (S the
 * exact sum; any order of R binary32 additions stays that close, gamma_R =
 * R u / (1 - R u), u = 2^-24), one step further out for the rounding of the
 * ends. The cached value is monotone in the bias (bf16 add, a multiplier, a
 * rising tanh, roundings), so the admissible cache values are those between
 * the cache values at the two extreme biases. Where base and bias nearly
 * cancel, a one-ulp bias difference moves the cache by many of its own
 * ulps: this is the rule such elements are held to.
 */
EXPORT int oracle_cache_admissible(uint16_t base, const uint16_t* e, const uint16_t* w, int32_t R,
                                   float mult, float softcap, uint16_t c_dev) {
  double s64 = 0.0, sabs = 0.0;
  uint16_t b_o = oracle_bias(e, w, R, &s64, &sabs);
  const double u = ldexp(1.0, -24), gamma = R * u / (1.0 - R * u);
  uint16_t lo = bf16_step(oracle_bf16_round((float)(s64 - gamma * sabs)), 0);
  uint16_t hi = bf16_step(oracle_bf16_round((float)(s64 + gamma * sabs)), 1);
  uint16_t dn = bf16_step(b_o, 0), up = bf16_step(b_o, 1);
  if (oracle_bf16_to_f32(dn) < oracle_bf16_to_f32(lo)) lo = dn;
  if (oracle_bf16_to_f32(up) > oracle_bf16_to_f32(hi)) hi = up;
  const float c1 = oracle_bf16_to_f32(oracle_cache_value(base, lo, mult, softcap));
  const float c2 = oracle_bf16_to_f32(oracle_cache_value(base, hi, mult, softcap));
  const float cd = oracle_bf16_to_f32(c_dev);
  if (isnan(c1) || isnan(c2) || isnan(cd)) return isnan(c1) && isnan(c2) && isnan(cd);
  return (c1 <= cd && cd <= c2) || (c2 <= cd && cd <= c1);
}

/* ------------------------------------------------------------------------ */
/* FP8 (E4M3) w2 with a per-row FP16 scale                                   */
/* ------------------------------------------------------------------------ */
/*
 * [EDGE] TensorRT Edge-LLM "DSpark kernels" page: `dsparkQuantizeMarkovW2Fp8`
 * (w2 [V, R] to E4M3 bytes of w / rowScale, one FP16 scale per row,
 * rowScale = rowAbsMax / 448 so each row spans the E4M3 range; R % 16 == 0)
 * and `dsparkMarkovGreedyFusedStepFp8` (the step with that w2). Readings:
 *   - the source w2 is the bf16 w2 of the other pages;
 *   - rowScale = the FP16 value nearest rowAbsMax / 448 (ties to even);
 *   - code = E4M3 of the binary32 quotient w / float(rowScale), nearest, ties
 *     to even, saturating at +-448 (E4M3 has no infinities); a zero scale (a
 *     zero row, or a scale below FP16's range) gives zero codes;
 *   - the bias is bf16(RN32(float(rowScale) * sum_j e_j q_j)) with q_j the
 *     code's value: the dot as for bf16 w2 (every E4M3 value is a bf16, so
 *     the products are exact in binary32), then the scale, then one bf16
 *     rounding.
 */

/* The value of an E4M3 code: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent 0 holds the subnormals m 2^-9; S.1111.111 is NaN. */
EXPORT float oracle_e4m3_decode(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (float)(sgn ? -v : v);
}

/* E4M3 nearest to x, ties to the even code, saturating at +-448; NaN gives
 * the NaN code of x's sign. Found by search over the 127 non-negative finite
 * codes (their values rise with the code). */
EXPORT uint8_t oracle_e4m3_encode(float x) {
  uint8_t sgn = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sgn | 0x7F);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sgn | 0x7E);
  uint8_t best = 0;
  for (int c = 1; c <= 0x7E; ++c) {
    double dc = fabs((double)oracle_e4m3_decode((uint8_t)c) - a);
    double db = fabs((double)oracle_e4m3_decode(best) - a);
    if (dc < db || (dc == db && (c & 1) == 0)) best = (uint8_t)c;
  }
  return (uint8_t)(sgn | best);
}

/* IEEE binary16: the value of a pattern, and the pattern nearest to x (ties
 * to even, overflow to infinity, NaN kept). */
EXPORT float oracle_fp16_to_f32(uint16_t h) {
  int sgn = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp(1.0 + m / 1024.0, e - 15);
  return (float)(sgn ? -v : v);
}

EXPORT uint16_t oracle_fp16_round(double x) {
  uint16_t sgn = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(sgn | 0x7E00);
  double a = fabs(x);
  /* the two neighbours among the non-negative patterns 0 .. 0x7C00 (inf) */
  uint16_t lo = 0, hi = 0x7C00;
  while (hi - lo > 1) {                  /* values rise with the pattern */
    uint16_t mid = (uint16_t)((lo + hi) / 2);
    if ((double)oracle_fp16_to_f32(mid) <= a) lo = mid; else hi = mid;
  }
  double vl = (double)oracle_fp16_to_f32(lo);
  if (vl == a) return (uint16_t)(sgn | lo);
  /* one ulp past the largest finite (65504) counts as 65536 for the tie */
  double vh = hi == 0x7C00 ? 65536.0 : (double)oracle_fp16_to_f32(hi);
  if (a >= vh) return (uint16_t)(sgn | hi);
  double dl = a - vl, dh = vh - a;
  uint16_t r = dl < dh ? lo : dh < dl ? hi : ((lo & 1) ? hi : lo);
  return (uint16_t)(sgn | r);
}

/* One w2 row to E4M3 codes q[R] and its FP16 scale (the bits). */
EXPORT uint16_t oracle_quantize_row_fp8(const uint16_t* w, int32_t R, uint8_t* q) {
  float amax = 0.0f;
  for (int32_t j = 0; j < R; ++j) {
    float a = fabsf(oracle_bf16_to_f32(w[j]));
    if (a > amax) amax = a;               /* a NaN weight is skipped */
  }
  uint16_t sbits = oracle_fp16_round((double)amax / 448.0);
  float scale = oracle_fp16_to_f32(sbits);
  for (int32_t j = 0; j < R; ++j)
    q[j] = scale == 0.0f ? (uint8_t)0 : oracle_e4m3_encode(oracle_bf16_to_f32(w[j]) / scale);
  return sbits;
}

EXPORT void oracle_quantize_w2_fp8(int32_t V, int32_t R, const uint16_t* w2, uint8_t* q,
                                   uint16_t* scales) {
  for (int32_t v = 0; v < V; ++v)
    scales[v] = oracle_quantize_row_fp8(w2 + (size_t)v * R, R, q + (size_t)v * R);
}

/* The bias against an E4M3 w2 row: the binary32 dot of e and the codes'
 * values in index order, times the scale in binary32, rounded to bf16.
 * s64 / sabs (optional) get the unscaled dot in binary64 and its sum of
 * |products|. */
EXPORT uint16_t oracle_bias_fp8(const uint16_t* e, const uint8_t* q, uint16_t scale_bits, int32_t R,
                                double* s64, double* sabs) {
  float acc = 0.0f;
  double d = 0.0, a = 0.0;
  for (int32_t j = 0; j < R; ++j) {
    float p = oracle_bf16_to_f32(e[j]) * oracle_e4m3_decode(q[j]);
    acc = acc + p;
    d += (double)p;
    a += fabs((double)p);
  }
  if (s64) *s64 = d;
  if (sabs) *sabs = a;
  float scaled = oracle_fp16_to_f32(scale_bits) * acc;
  return oracle_bf16_round(scaled);
}

/* oracle_cache_admissible for an E4M3 w2 row: the admissible unscaled dots
 * are those within gamma_R sum|p| of the exact one (any summation order),
 * then scaled and rounded as the definition does; the oracle's bias one
 * bf16 step either way also counts. */
EXPORT int oracle_cache_admissible_fp8(uint16_t base, const uint16_t* e, const uint8_t* q,
                                       uint16_t scale_bits, int32_t R, float mult, float softcap,
                                       uint16_t c_dev) {
  double s64 = 0.0, sabs = 0.0;
  uint16_t b_o = oracle_bias_fp8(e, q, scale_bits, R, &s64, &sabs);
  const double u = ldexp(1.0, -24), gamma = R * u / (1.0 - R * u);
  const float sc = oracle_fp16_to_f32(scale_bits);
  float x1 = sc * (float)(s64 - gamma * sabs), x2 = sc * (float)(s64 + gamma * sabs);
  if (x1 > x2) { float t = x1; x1 = x2; x2 = t; }
  uint16_t lo = bf16_step(oracle_bf16_round(x1), 0), hi = bf16_step(oracle_bf16_round(x2), 1);
  uint16_t dn = bf16_step(b_o, 0), up = bf16_step(b_o, 1);
  if (oracle_bf16_to_f32(dn) < oracle_bf16_to_f32(lo)) lo = dn;
  if (oracle_bf16_to_f32(up) > oracle_bf16_to_f32(hi)) hi = up;
  const float c1 = oracle_bf16_to_f32(oracle_cache_value(base, lo, mult, softcap));
  const float c2 = oracle_bf16_to_f32(oracle_cache_value(base, hi, mult, softcap));
  const float cd = oracle_bf16_to_f32(c_dev);
  if (isnan(c1) || isnan(c2) || isnan(cd)) return isnan(c1) && isnan(c2) && isnan(cd);
  return (c1 <= cd && cd <= c2) || (c2 <= cd && cd <= c1);
}

/* ------------------------------------------------------------------------ */
/* Argmax under the total order                                              */
/* ------------------------------------------------------------------------ */

/*
 * Whether (v1, i1) comes before (v2, i2) in the order every argmax of the
 * method uses ([MUSE] module docstring and `_combine`): a NaN value beats
 * every non-NaN value; among NaNs the lower id wins; otherwise the larger
 * value wins, and equal values (IEEE ==, so -0 == +0) go to the lower id.
 */
EXPORT int oracle_before(float v1, int64_t i1, float v2, int64_t i2) {
  int n1 = isnan(v1), n2 = isnan(v2);
  if (n1 || n2) {
    if (n1 && n2) return i1 < i2;
    return n1;
  }
  if (v1 > v2) return 1;
  if (v1 < v2) return 0;
  return i1 < i2;
}

/*
 * The packed 64-bit image of a winner (v, id) in the greedy slot format
 * (TensorRT Edge-LLM "DSpark kernels" page, `dsparkMarkovGreedyFusedStep`:
 * an orderable float key, ties to the lowest vocabulary index): unsigned
 * comparison of two images agrees with oracle_before. High word: every NaN
 * maps to 0xffffffff; otherwise -0 counts as +0, a non-negative value maps to
 * its bits with the top bit set, a negative one to its bits inverted (larger
 * magnitude, smaller image). Low word: the complement of the 32-bit id.
 */
EXPORT uint64_t oracle_pack_winner(float v, int64_t id) {
  uint32_t hi;
  if (isnan(v)) {
    hi = 0xffffffffu;
  } else {
    uint32_t b = f32_to_bits(v == 0.0f ? 0.0f : v);
    hi = (b >> 31) ? ~b : (b | 0x80000000u);
  }
  return ((uint64_t)hi << 32) | (uint64_t)(uint32_t)~(uint32_t)id;
}

/* Argmax of keys[0..n) under that order, scanning ids upward. */
EXPORT int64_t oracle_argmax(const float* keys, int64_t n) {
  int64_t best = 0;
  for (int64_t v = 1; v < n; ++v)
    if (oracle_before(keys[v], v, keys[best], best)) best = v;
  return best;
}

/* ------------------------------------------------------------------------ */
/* One draft step and the k-step loop                                        */
/* ------------------------------------------------------------------------ */

/* The w1 row of a token: clamped to V-1 as an unsigned value ([MUSE] `_w1_row`). */
EXPORT int64_t oracle_w1_row(int64_t token, int32_t V) {
  uint64_t t = (uint64_t)token, last = (uint64_t)(V - 1);
  return (int64_t)(t < last ? t : last);
}

/* One step for every row with either a bf16 w2 (w2 != NULL) or an E4M3 w2
 * (q, scales); otherwise as oracle_step below. */
static void step_any(int32_t rows, int32_t V, int32_t R, const uint16_t* base, int64_t base_rs,
                     const uint16_t* w1, const uint16_t* w2, const uint8_t* q,
                     const uint16_t* scales, const int64_t* prev, const int64_t* seeds,
                     const int64_t* positions, int64_t pos_rs, int32_t step,
                     const float* temperature, float mult, float softcap, uint16_t* cache,
                     int64_t cache_rs, float* keys, int64_t keys_rs, uint16_t* bias,
                     int64_t bias_rs, int64_t* tokens, int32_t threads) {
#ifdef _OPENMP
  int nt = threads > 0 ? threads : 1;
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
#endif
  for (int32_t r = 0; r < rows; ++r) {
    const uint16_t* e = w1 + (size_t)oracle_w1_row(prev[r], V) * (size_t)R;
    float T = temperature[r];
    int64_t position = positions[(int64_t)r * pos_rs];
    int64_t best = -1;
    float best_key = 0.0f;
    for (int32_t v = 0; v < V; ++v) {
      uint16_t b = w2 ? oracle_bias(e, w2 + (size_t)v * (size_t)R, R, NULL, NULL)
                      : oracle_bias_fp8(e, q + (size_t)v * (size_t)R, scales[v], R, NULL, NULL);
      uint16_t c = oracle_cache_value(base[(int64_t)r * base_rs + v], b, mult, softcap);
      cache[(int64_t)r * cache_rs + v] = c;
      if (bias) bias[(int64_t)r * bias_rs + v] = b;
      float l = oracle_bf16_to_f32(c);
      uint32_t h = oracle_noisy(T) ? oracle_noise_hash(seeds[r], step, position, (uint32_t)v) : 0u;
      float key = oracle_gumbel_key(l, T, h, NULL, NULL);
      if (keys) keys[(int64_t)r * keys_rs + v] = key;
      if (best < 0 || oracle_before(key, v, best_key, best)) {
        best = v;
        best_key = key;
      }
    }
    tokens[r] = best;
  }
}

/*
 * One draft step for every row, teacher-forced from `prev` (the token that
 * feeds this step). Follows one iteration of the eager loop ([KIMI] and
 * [DSV41] `_loop_rest`): embed the previous token, form the bias over the
 * whole vocabulary, add the base logits, transform and cache, then sample.
 *   base       bf16, row r of this step at base + r*base_rs, V entries
 *   w1, w2     bf16 [V, R] row-major
 *   prev       [rows] token feeding this step
 *   seeds      [rows]; positions: row r's sample position at positions[r*pos_rs]
 *   temperature[rows] binary32
 *   cache      out, bf16, row r at cache + r*cache_rs
 *   keys       out (may be NULL), binary32 [rows, V] at keys + r*keys_rs
 *   bias       out (may be NULL), bf16 [rows, V] at bias + r*bias_rs
 *   tokens     out [rows]
 * threads > 1 runs rows in parallel (rows are independent).
 */
EXPORT void oracle_step(int32_t rows, int32_t V, int32_t R, const uint16_t* base, int64_t base_rs,
                        const uint16_t* w1, const uint16_t* w2, const int64_t* prev,
                        const int64_t* seeds, const int64_t* positions, int64_t pos_rs,
                        int32_t step, const float* temperature, float mult, float softcap,
                        uint16_t* cache, int64_t cache_rs, float* keys, int64_t keys_rs,
                        uint16_t* bias, int64_t bias_rs, int64_t* tokens, int32_t threads) {
  step_any(rows, V, R, base, base_rs, w1, w2, NULL, NULL, prev, seeds, positions, pos_rs, step,
           temperature, mult, softcap, cache, cache_rs, keys, keys_rs, bias, bias_rs, tokens,
           threads);
}

/* oracle_step with the E4M3 w2 (q [V, R] codes, scales [V] FP16 bits) in
 * place of w2 ([EDGE] `dsparkMarkovGreedyFusedStepFp8`). */
EXPORT void oracle_step_fp8(int32_t rows, int32_t V, int32_t R, const uint16_t* base,
                            int64_t base_rs, const uint16_t* w1, const uint8_t* q,
                            const uint16_t* scales, const int64_t* prev, const int64_t* seeds,
                            const int64_t* positions, int64_t pos_rs, int32_t step,
                            const float* temperature, float mult, float softcap, uint16_t* cache,
                            int64_t cache_rs, float* keys, int64_t keys_rs, uint16_t* bias,
                            int64_t bias_rs, int64_t* tokens, int32_t threads) {
  step_any(rows, V, R, base, base_rs, w1, NULL, q, scales, prev, seeds, positions, pos_rs, step,
           temperature, mult, softcap, cache, cache_rs, keys, keys_rs, bias, bias_rs, tokens,
           threads);
}

/*
 * The k-step loop ([KIMI] `_loop_rest`): step s feeds on prev (s = 0) or on
 * the token step s-1 sampled. Layouts as the library's entry point:
 *   base, cache  bf16 [rows, k, V] contiguous
 *   positions    [rows, k];  tokens out [rows, k]
 */
EXPORT void oracle_sample_sequential(int32_t rows, int32_t V, int32_t R, int32_t k,
                                     const uint16_t* base, const uint16_t* w1,
                                     const uint16_t* w2, const int64_t* prev,
                                     const int64_t* seeds, const int64_t* positions,
                                     const float* temperature, float mult, float softcap,
                                     uint16_t* cache, int64_t* tokens, int32_t threads) {
  int64_t* feed = (int64_t*)malloc(sizeof(int64_t) * (size_t)(rows > 0 ? rows : 1));
  int64_t* out = (int64_t*)malloc(sizeof(int64_t) * (size_t)(rows > 0 ? rows : 1));
  for (int32_t r = 0; r < rows; ++r) feed[r] = prev[r];
  int64_t row_stride = (int64_t)k * V;
  for (int32_t s = 0; s < k; ++s) {
    oracle_step(rows, V, R, base + (int64_t)s * V, row_stride, w1, w2, feed, seeds, positions + s,
                k, s, temperature, mult, softcap, cache + (int64_t)s * V, row_stride, NULL, 0,
                NULL, 0, out, threads);
    for (int32_t r = 0; r < rows; ++r) {
      tokens[(int64_t)r * k + s] = out[r];
      feed[r] = out[r];
    }
  }
  free(feed);
  free(out);
}

/* ------------------------------------------------------------------------ */
/* The tolerance: which row-steps the definition decides                     */
/* ------------------------------------------------------------------------ */

/*
 * Whether one row-step's token is decided despite the differences the
 * definition admits, and its winner. The only freedoms are the bias
 * summation order ([KIMI] and [DSV41]: the last bf16 bit of a bias may
 * differ) and the last ulp of the two logs. A token v competes with the
 * winner w through its key K(v); its key may move by
 *   d(v) = dc(v) / |T| + eps(v)    (T noisy),   d(v) = dc(v)   (T = 0)
 * where dc(v) is the cache difference allowed at v, and
 *   eps(v) = 2 ulp32(K(v)) + 2 ulp32(lb(v)) + 2 |ulp32(L(v)) / L(v)|
 * bounds a one-ulp change of either log and of the rounded quotient.
 * `literal` != 0 takes dc(v) = one bf16 ulp of the oracle's cache value at
 * every v; otherwise dc(v) = |cache_g(v) - cache_o(v)| (the realized
 * difference; 0 where the two agree).
 * Equal cache values (infinities included) differ by 0; an infinite key has
 * no rounding band (its quotient is infinite, the noise finite), and at
 * an infinite cached value the literal band is 0.
 * Decided: for every v != w, K(w) - K(v) > d(w) + d(v), or K(w) == K(v) with
 * d(w) = d(v) = 0 and w < v. A NaN winner is decided when its NaN comes from
 * the cache on both sides and no lower id has a NaN cache value on either
 * side, or when T itself is NaN (then every key is NaN).
 * Any v where exactly one of the two caches is NaN makes the step undecided.
 * Returns 1 (decided) or 0; *winner gets the oracle's token.
 */
/* The keys K(v) and perturbation bands d(v) of one row-step (see
 * oracle_decided); returns 0 where exactly one of the two caches is NaN at
 * some v, else 1. */
static int keys_and_bands(int32_t V, const uint16_t* cache_o, const uint16_t* cache_g, float T,
                          int64_t seed, int32_t step, int64_t position, int32_t literal, float* K,
                          double* d) {
  int ok = 1;
  int noisy = oracle_noisy(T);
  for (int32_t v = 0; v < V; ++v) {
    float lo = oracle_bf16_to_f32(cache_o[v]);
    float lg = oracle_bf16_to_f32(cache_g[v]);
    if (isnan(lo) != isnan(lg)) ok = 0;
    double dc;
    if (literal)
      dc = isinf(lo) ? 0.0 : oracle_ulp_bf16(lo);   /* infinities are exact */
    else
      dc = ((isnan(lo) && isnan(lg)) || lo == lg) ? 0.0 : fabs((double)lg - (double)lo);
    float lb = 0.0f, L = 0.0f;
    uint32_t h = noisy ? oracle_noise_hash(seed, step, position, (uint32_t)v) : 0u;
    K[v] = oracle_gumbel_key(lo, T, h, &lb, &L);
    if (noisy) {
      /* an infinite key is exact: the quotient is infinite and the finite
       * noise cannot move it */
      double eps = isinf(K[v]) ? 0.0
                               : 2.0 * oracle_ulp32(K[v]) + 2.0 * oracle_ulp32(lb) +
                                     2.0 * fabs(oracle_ulp32(L) / (double)L);
      d[v] = dc / fabs((double)T) + eps;
    } else {
      d[v] = dc;
    }
  }
  return ok;
}

EXPORT int oracle_decided(int32_t V, const uint16_t* cache_o, const uint16_t* cache_g, float T,
                          int64_t seed, int32_t step, int64_t position, int32_t literal,
                          int64_t* winner) {
  float* K = (float*)malloc(sizeof(float) * (size_t)V);
  double* d = (double*)malloc(sizeof(double) * (size_t)V);
  int ok = keys_and_bands(V, cache_o, cache_g, T, seed, step, position, literal, K, d);
  int64_t w = oracle_argmax(K, V);
  *winner = w;
  if (ok && isnan(K[w])) {
    if (isnan(T)) {
      ok = 1;
    } else {
      int structural = isnan(oracle_bf16_to_f32(cache_o[w])) && isnan(oracle_bf16_to_f32(cache_g[w]));
      for (int64_t v = 0; v < w && structural; ++v)
        if (isnan(oracle_bf16_to_f32(cache_o[v])) || isnan(oracle_bf16_to_f32(cache_g[v])))
          structural = 0;
      ok = structural;
    }
  } else if (ok) {
    for (int32_t v = 0; v < V && ok; ++v) {
      if (v == w) continue;
      if (isnan(K[v])) { ok = 0; break; }
      double gap = (double)K[w] - (double)K[v];
      if (gap > d[w] + d[v]) continue;
      if (K[w] == K[v] && d[w] == 0.0 && d[v] == 0.0 && w < v) continue;
      ok = 0;
    }
  }
  free(K);
  free(d);
  return ok;
}

/*
 * Whether token `cand` lies in the near-tie set of an undecided row-step:
 * it is the oracle's winner w, or its key is NaN while some key may be, or
 * the bands of the two overlap, K(w) - K(cand) <= d(w) + d(cand), with the
 * same K and d as oracle_decided. A device token outside this set is wrong
 * whatever the row's margin. cand outside [0, V) is never in the set.
 */
EXPORT int oracle_near_tie(int32_t V, const uint16_t* cache_o, const uint16_t* cache_g, float T,
                           int64_t seed, int32_t step, int64_t position, int32_t literal,
                           int64_t cand) {
  if (cand < 0 || cand >= V) return 0;
  float* K = (float*)malloc(sizeof(float) * (size_t)V);
  double* d = (double*)malloc(sizeof(double) * (size_t)V);
  int one_side_nan = !keys_and_bands(V, cache_o, cache_g, T, seed, step, position, literal, K, d);
  int64_t w = oracle_argmax(K, V);
  int in;
  if (cand == w)
    in = 1;
  else if (isnan(K[w]) || isnan(K[cand]))
    in = one_side_nan || isnan(T);   /* a NaN on one side only can move the winner anywhere */
  else
    in = ((double)K[w] - (double)K[cand]) <= d[w] + d[cand];
  free(K);
  free(d);
  return in;
}

/* ------------------------------------------------------------------------ */
/* Self-check support                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Scan every binary32 x in [lo, hi] and list those where the binary64 log
 * lies within `ulps` binary64 ulps of a binary32 rounding midpoint: only
 * there can RN32(log64(x)) differ from the correctly rounded log, given a
 * binary64 log accurate to under one ulp. Returns the count (the first
 * `cap` are written to out).
 */
EXPORT int64_t oracle_log_hard_cases(float lo, float hi, double ulps, float* out, int64_t cap) {
  /* the raw binary64 log, before the long double fallback */
  int64_t n = 0;
  for (uint32_t b = f32_to_bits(lo); b <= f32_to_bits(hi); ++b) {
    float x = bits_to_f32(b);
    double y = log((double)x);
    float f = (float)y;
    /* the two binary32 midpoints around f */
    double fd = (double)f;
    double up = (double)nextafterf(f, INFINITY), dn = (double)nextafterf(f, -INFINITY);
    double m1 = 0.5 * (fd + up), m2 = 0.5 * (fd + dn);
    double tol = ulps * (nextafter(fabs(y), INFINITY) - fabs(y));
    if (fabs(y - m1) <= tol || fabs(y - m2) <= tol) {
      if (n < cap) out[n] = x;
      ++n;
    }
    if (b == 0xffffffffu) break;
  }
  return n;
}

/*
 * The Gumbel noise -lb(h) = log(-log1m(u(h))) negated, for the n hashes
 * h0, h0+1, ... (wrapping at 2^32), into out[n]: the key of a zero logit at
 * temperature 1. For checks that sweep every hash.
 */
EXPORT void oracle_noise_many(uint32_t h0, int64_t n, float* out, int32_t threads) {
#ifdef _OPENMP
  int nt = threads > 0 ? threads : 1;
#pragma omp parallel for num_threads(nt) schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_gumbel_key(0.0f, 1.0f, (uint32_t)(h0 + (uint64_t)i), NULL, NULL);
}

/* ------------------------------------------------------------------------ */
/* Verification of a drafted block                                           */
/* ------------------------------------------------------------------------ */
/*
 * [EDGE] TensorRT Edge-LLM "DSpark kernels" page: `dsparkGreedyAccept` (a
 * draft token is accepted while it equals the base argmax at the previous
 * verify position, then the base bonus token is appended) and
 * `dsparkProbabilisticAccept` (the rejection-sampling verifier with a
 * residual: acceptUniforms [B, 2P+1], the first P driving accept / reject,
 * the next P the residual sample of a rejection at the matching step, the
 * last the bonus sample when the whole proposal is accepted). The rule is
 * the speculative-sampling rule: accept draft token d at step j with
 * probability min(1, p_j(d) / q_j(d)); on the first rejection sample from
 * max(0, p_j - q_j) normalised; if all L proposals pass, sample the bonus
 * from p_L. Readings:
 *   - draft token j sits at verify position j + 1, so it is checked against
 *     the target at position j (the "previous verify position");
 *   - accept iff u_j q_j(d) < p_j(d), both products exact in binary64;
 *   - the residual is r(x) = max(0, RN32(p(x) - q(x))); a sample with
 *     uniform u from weights w is the smallest x with C(x) > u S, C the
 *     prefix sums of w in index order in binary64, S = C(V-1), u S one
 *     binary64 product; with S = 0 the residual is replaced by p itself,
 *     and with that 0 too the token is 0;
 *   - a proposal length above P counts as P, below 0 as 0; accepted slots
 *     after the emitted tokens are set to -1; a draft token outside [0, V)
 *     is never accepted (its p and q are taken as 0).
 */

/* Sample from weights w[0..V) with uniform u (see above); *margin gets the
 * distance of u S to the nearer of C(x-1) and C(x) (for the decided rule). */
static int64_t cdf_sample(const double* w, int64_t V, double u, double* margin) {
  double S = 0.0;
  for (int64_t x = 0; x < V; ++x) S += w[x];
  if (!(S > 0.0)) {
    if (margin) *margin = INFINITY;
    return -1;                              /* no mass */
  }
  const double t = u * S;
  double C = 0.0;
  for (int64_t x = 0; x < V; ++x) {
    const double prev = C;
    C += w[x];
    if (C > t) {
      if (margin) *margin = fmin(C - t, t - prev);
      return x;
    }
  }
  if (margin) *margin = 0.0;                /* rounding left u S at or above the total */
  return V - 1;
}

/*
 * The greedy verifier for one row b: argmax under the total order of each
 * bf16 row logits[j][0..V) for j = 0..P, then acceptance. Returns the number
 * of tokens written to accepted[0..P] (the accepted drafts and the bonus).
 */
EXPORT int32_t oracle_greedy_accept_row(const uint16_t* logits, int64_t V, int32_t P,
                                        const int64_t* draft, int32_t L, int64_t* accepted) {
  if (L > P) L = P;
  if (L < 0) L = 0;
  float* row = (float*)malloc(sizeof(float) * (size_t)V);
  int32_t n = 0;
  int64_t bonus = 0;
  for (int32_t j = 0; j <= L; ++j) {
    for (int64_t v = 0; v < V; ++v) row[v] = oracle_bf16_to_f32(logits[(size_t)j * V + v]);
    const int64_t a = oracle_argmax(row, V);
    if (j < L && draft[j] == a) {
      accepted[n++] = draft[j];
      continue;
    }
    bonus = a;
    break;
  }
  accepted[n++] = bonus;
  for (int32_t i = n; i <= P; ++i) accepted[i] = -1;
  free(row);
  return n;
}

/*
 * The probabilistic verifier for one row b: target [P+1][V] and draft [P][V]
 * binary32 probabilities, draft tokens [P], L, uniforms [2P+1]. Writes
 * accepted[0..P], returns the count; *margin_out (optional) gets the
 * sampled token's CDF margin relative to the mass S (the decided rule:
 * any summation order keeps C within (V + 2) 2^-52 S of the index-order
 * one, so a margin above that leaves the token unique).
 */
EXPORT int32_t oracle_prob_accept_row(const float* target, const float* draftp, int64_t V, int32_t P,
                                      const int64_t* draft, int32_t L, const float* uniforms,
                                      int64_t* accepted, double* margin_out, double* mass_out) {
  if (L > P) L = P;
  if (L < 0) L = 0;
  int32_t n = 0;
  int32_t j = 0;
  for (; j < L; ++j) {
    const int64_t d = draft[j];
    const double p = (d >= 0 && d < V) ? (double)target[(size_t)j * V + d] : 0.0;
    const double q = (d >= 0 && d < V) ? (double)draftp[(size_t)j * V + d] : 0.0;
    if ((double)uniforms[j] * q < p) {
      accepted[n++] = d;
      continue;
    }
    break;
  }
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  double u;
  const float* prow = target + (size_t)j * V;
  if (j < L) {                              /* rejected at j: the residual */
    for (int64_t x = 0; x < V; ++x) {
      const float r = prow[x] - draftp[(size_t)j * V + x];
      w[x] = r > 0.0f ? (double)r : 0.0;
    }
    u = (double)uniforms[P + j];
  } else {                                  /* all accepted: the bonus from p_L */
    for (int64_t x = 0; x < V; ++x) w[x] = (double)prow[x];
    u = (double)uniforms[2 * P];
  }
  double margin = 0.0, S = 0.0;
  int64_t x = cdf_sample(w, V, u, &margin);
  if (x < 0) {                              /* no residual mass: sample p itself */
    for (int64_t y = 0; y < V; ++y) w[y] = (double)prow[y];
    x = cdf_sample(w, V, u, &margin);
    if (x < 0) { x = 0; margin = INFINITY; }
  }
  for (int64_t y = 0; y < V; ++y) S += w[y];
  accepted[n++] = x;
  for (int32_t i = n; i <= P; ++i) accepted[i] = -1;
  if (margin_out) *margin_out = margin;
  if (mass_out) *mass_out = S;
  free(w);
  return n;
}
