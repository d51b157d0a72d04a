/*
 * Plain C reference of the W4A8 block-32 linear layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg may load this library; the GPU library never calls it and shares no
 * code with it.
 *
 * What it computes (ML Drift explainer on tech.dede.sh, section "Stage-aware
 * optimization for large language models": 4-bit weights in blocks of 32,
 * activations quantised by the kernel itself), in the scheme this project
 * pins:
 *   per token row m and block b of 32 consecutive inputs
 *     amax = max |x|  (fp16 widened to fp32, exact)
 *     sx   = fp32(amax / 127)            (IEEE division, round to nearest even)
 *     qx   = clamp(rint(fp32(x / sx)), -127, 127), half to even; amax = 0 -> sx = 0, qx = 0
 *   I[m][n][b] = sum_{j<32} qx[m][32b+j] * qw[n][32b+j]     (exact integer)
 *   out[m][n]  = sum_b fp64(I) * fp64(sw[n][b]) * fp64(sx[m][b])   (blocks in ascending order)
 * Build with a plain C compiler, no fast-math, -ffp-contract=off, so every
 * operation above is one IEEE operation in the stated precision; each output
 * is formed by one thread in a fixed order, so the result does not depend on
 * the thread count.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define BLOCK 32

/* fp16 bits -> fp32 (exact widening: normals, subnormals, signed zeros). */
static float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h >> 15) << 31;
  const uint32_t exp = (h >> 10) & 0x1F;
  uint32_t mant = h & 0x3FF;
  uint32_t bits;
  if (exp == 0) {
    if (mant == 0) {
      bits = sign;
    } else { /* subnormal: value = mant * 2^-24 */
      int e = -1;
      do {
        mant <<= 1;
        ++e;
      } while ((mant & 0x400) == 0);
      mant &= 0x3FF;
      bits = sign | (uint32_t)(127 - 15 - e) << 23 | mant << 13;
    }
  } else if (exp == 0x1F) {
    bits = sign | 0x7F800000u | mant << 13;
  } else {
    bits = sign | (exp - 15 + 127) << 23 | mant << 13;
  }
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* Quantise rows of fp16 activations: qx int8 [M][K], sx fp32 [M][K/32]. */
void w4a8_ref_quantize(const uint16_t* x16, int64_t M, int64_t K, int8_t* qx, float* sx) {
  fesetround(FE_TONEAREST);
  const int64_t nb = K / BLOCK;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* xb = x16 + m * K + b * BLOCK;
      float v[BLOCK];
      float amax = 0.0f;
      for (int j = 0; j < BLOCK; ++j) {
        v[j] = half_to_float(xb[j]);
        const float a = fabsf(v[j]);
        if (a > amax) amax = a;
      }
      int8_t* qb = qx + m * K + b * BLOCK;
      if (amax == 0.0f) {
        sx[m * nb + b] = 0.0f;
        for (int j = 0; j < BLOCK; ++j) qb[j] = 0;
        continue;
      }
      const float s = amax / 127.0f;
      sx[m * nb + b] = s;
      for (int j = 0; j < BLOCK; ++j) {
        const float ratio = v[j] / s;
        float q = rintf(ratio);
        if (q > 127.0f) q = 127.0f;
        if (q < -127.0f) q = -127.0f;
        qb[j] = (int8_t)q;
      }
    }
  }
}

static int32_t block_dot(const int8_t* a, const int8_t* w) {
  int32_t s = 0;
  for (int j = 0; j < BLOCK; ++j) s += (int32_t)a[j] * (int32_t)w[j];
  return s;
}

/* Integer block sums I[m][n][b] (int32 [M][N][K/32]) of quantised activations and weights qw [N][K]. */
void w4a8_ref_block_sums(const int8_t* qx, const int8_t* qw, int64_t M, int64_t K, int64_t N, int32_t* sums,
                         int threads) {
  const int64_t nb = K / BLOCK;
#ifdef _OPENMP
#pragma omp parallel for num_threads(threads > 0 ? threads : 1) schedule(static)
#else
  (void)threads;
#endif
  for (int64_t n = 0; n < N; ++n)
    for (int64_t m = 0; m < M; ++m)
      for (int64_t b = 0; b < nb; ++b)
        sums[(m * N + n) * nb + b] = block_dot(qx + m * K + b * BLOCK, qw + n * K + b * BLOCK);
}

/* out fp64 [M][N] from quantised activations (qx, sx), weights qw int8 [N][K] in [-8, 7] and
 * scales sw16 fp16 [N][K/32]; columns split over `threads` OpenMP threads. */
void w4a8_ref_scaled(const int8_t* qx, const float* sx, const int8_t* qw, const uint16_t* sw16, int64_t M, int64_t K,
                     int64_t N, double* out, int threads) {
  const int64_t nb = K / BLOCK;
#ifdef _OPENMP
#pragma omp parallel for num_threads(threads > 0 ? threads : 1) schedule(static)
#else
  (void)threads;
#endif
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        const int32_t I = block_dot(qx + m * K + b * BLOCK, qw + n * K + b * BLOCK);
        double t = (double)I * (double)half_to_float(sw16[n * nb + b]);
        t = t * (double)sx[m * nb + b];
        acc = acc + t;
      }
      out[m * N + n] = acc;
    }
  }
}

/* The whole linear: quantise x16 [M][K] into the caller's scratch (qx [M][K], sx [M][K/32]),
 * then the scaled block sums. */
void w4a8_ref_linear(const uint16_t* x16, const int8_t* qw, const uint16_t* sw16, int64_t M, int64_t K, int64_t N,
                     int8_t* qx, float* sx, double* out, int threads) {
  w4a8_ref_quantize(x16, M, K, qx, sx);
  w4a8_ref_scaled(qx, sx, qw, sw16, M, K, N, out, threads);
}

/* Threads an OpenMP build uses by default (1 without OpenMP). */
int w4a8_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
