/*
 * Sweeps over all 2^32 hashes, for the CPU tests (built by the test that
 * uses it, with gcc -O2 -fopenmp; not part of the library or the oracle).
 *
 * check_uniform_all: the oracle's uniform u(h) against the exact rounding of
 *   (h + 1/2) 2^-32 to binary32 computed here with integer arithmetic only
 *   (round to nearest, ties to even, on the odd integer 2h + 1 scaled by
 *   2^-33): the oracle forms it with one binary64 product and a conversion.
 *
 * check_noise_tables_all: the step kernel's two noise bound tables (per hash
 *   bucket a line A + B float(h), and a constant C) against the oracle's
 *   noise -lb(h) at every h. The bucket of h is the kernel's: the exponent
 *   and top 6 mantissa bits of the nearest binary32 to h, less 8127,
 *   saturated at 0. The kernel rounds the fused line A + B float(h) once to
 *   binary32; rounding is monotone and the noise is a binary32, so the line
 *   bounds the noise exactly when its exact value does. B float(h) is exact
 *   in binary64 and the binary64 sum errs by at most 2^-53 of its size, so a
 *   line counts as holding where that sum exceeds the noise by 2^-52 of its
 *   size. The minimum slack over all h of each table is reported.
 *
 * Both take the oracle's function by pointer (the test passes the address of
 * the oracle library's export), so no code is shared with it.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef float (*uniform_fn)(uint32_t h);
typedef float (*key_fn)(float l, float T, uint32_t h, float* lb, float* L);

static float exact_uniform(uint32_t h) {
  const uint64_t N = 2 * (uint64_t)h + 1; /* the value is N 2^-33, N odd */
  const int n = 64 - __builtin_clzll(N);
  if (n <= 24) return ldexpf((float)N, -33);
  const int shift = n - 24;
  uint64_t m = N >> shift;
  const uint64_t rem = N - (m << shift), half = (uint64_t)1 << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) ++m;
  return ldexpf((float)m, shift - 33); /* m <= 2^24: exact */
}

int64_t check_uniform_all(uniform_fn uni, int threads, uint32_t* first_bad) {
  int64_t bad = 0;
  uint32_t first = 0xffffffffu;
#pragma omp parallel for num_threads(threads) schedule(static) reduction(+ : bad)
  for (int64_t i = 0; i < ((int64_t)1 << 32); ++i) {
    const uint32_t h = (uint32_t)i;
    const float a = uni(h), b = exact_uniform(h);
    uint32_t ab, bb;
    memcpy(&ab, &a, 4);
    memcpy(&bb, &b, 4);
    if (ab != bb) {
      ++bad;
#pragma omp critical
      if (h < first) first = h;
    }
  }
  *first_bad = first;
  return bad;
}

int64_t check_noise_tables_all(key_fn key, const float* A, const float* B, const float* C, int nb,
                               int threads, double* min_line, uint32_t* arg_line,
                               double* min_const, uint32_t* arg_const) {
  int64_t bad = 0;
  double ml = INFINITY, mc = INFINITY;
  uint32_t al = 0, ac = 0;
#pragma omp parallel num_threads(threads)
  {
    double tl = INFINITY, tc = INFINITY;
    uint32_t tal = 0, tac = 0;
    int64_t tb = 0;
#pragma omp for schedule(static)
    for (int64_t i = 0; i < ((int64_t)1 << 32); ++i) {
      const uint32_t h = (uint32_t)i;
      const float noise = key(0.0f, 1.0f, h, NULL, NULL); /* 0 / 1 - lb = -lb */
      const float fh = (float)h;
      uint32_t fb;
      memcpy(&fb, &fh, 4);
      uint32_t b = fb >> 17;
      b = b > 8127u ? b - 8127u : 0u;
      if ((int)b >= nb) {
        ++tb;
        continue;
      }
      const double line = (double)B[b] * (double)fh + (double)A[b];
      const double sl = line - (double)noise;
      if (!(sl >= ldexp(fabs(line), -52))) ++tb;
      if (sl < tl) {
        tl = sl;
        tal = h;
      }
      const double sc = (double)C[b] - (double)noise;
      if (!(sc >= 0.0)) ++tb;
      if (sc < tc) {
        tc = sc;
        tac = h;
      }
    }
#pragma omp critical
    {
      bad += tb;
      if (tl < ml) {
        ml = tl;
        al = tal;
      }
      if (tc < mc) {
        mc = tc;
        ac = tac;
      }
    }
  }
  *min_line = ml;
  *arg_line = al;
  *min_const = mc;
  *arg_const = ac;
  return bad;
}
