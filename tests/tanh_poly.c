/*
 * Error sweep of the step kernel's binary32 tanh polynomial (for the CPU
 * tests; built by the test with gcc -O2 -fopenmp, not part of the library or
 * the oracle). The test passes the kernel's six coefficients, so the sweep
 * evaluates exactly what the kernel does: t = z z, p by Horner with fused
 * multiply-adds, then fma(t z, p, z), every operation in binary32. Each
 * value is compared with tanh in binary64 (whose own error, under a binary64
 * ulp, is below 2^-28 of a binary32 ulp), in binary32 ulps of the rounded
 * reference. The polynomial is odd in binary32 as well (t and p are even,
 * t z odd), so z >= 0 covers the interval.
 *
 * sweep_tanh_poly(c, zmax, z_dense, stride, &worst_u32): every binary32 z in
 * [z_dense, zmax] and every stride-th one in [0, z_dense); returns the
 * largest error in ulps and the z where it occurs.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float f_of(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t u_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static double ulp32(float y) {
  int e;
  frexpf(fabsf(y), &e);
  double u = ldexp(1.0, e - 24);
  return u < ldexp(1.0, -149) ? ldexp(1.0, -149) : u;
}

static double err_at(const float* c, float z) {
  const float t = z * z;
  float p = c[0];
  for (int i = 1; i < 6; ++i) p = fmaf(p, t, c[i]);
  const float y = fmaf(t * z, p, z);
  const double ref = tanh((double)z);
  return fabs((double)y - ref) / ulp32((float)ref);
}

double sweep_tanh_poly(const float* c, float zmax, float z_dense, int stride, uint32_t* worst_at) {
  const int64_t hi = u_of(zmax), mid = u_of(z_dense);
  double worst = 0.0;
  uint32_t wu = 0;
#pragma omp parallel
  {
    double lw = 0.0;
    uint32_t lu = 0;
#pragma omp for schedule(static)
    for (int64_t u = 0; u <= hi; ++u) {
      if (u < mid && u % stride) continue;
      const double e = err_at(c, f_of((uint32_t)u));
      if (e > lw) {
        lw = e;
        lu = (uint32_t)u;
      }
    }
#pragma omp critical
    if (lw > worst) {
      worst = lw;
      wu = lu;
    }
  }
  *worst_at = wu;
  return worst;
}
