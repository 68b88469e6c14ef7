/*
 * Reference (oracle) implementation of the tensorwise-scaled Float8Linear
 * element-wise steps: amax, scale, fp8 cast (+ transposed copy), delayed-scaling
 * history.  TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load this library.  Nothing on the
 * product path links it, and it shares no code with the HIP kernels.
 *
 * Written to be slow and obviously correct: plain C99, no intrinsics, fp64 or
 * IEEE binary32 arithmetic as each step states, OpenMP only over independent
 * elements or rows.  Built with -O2 -ffp-contract=off (no FMA contraction, no
 * fast-math), so every float operation below is one correctly rounded IEEE op.
 *
 * Sources.
 *  - The method: tensorwise *dynamic* scaling (one scale per tensor from the
 *    tensor's current amax; pytorch/torchtitan PR #778 "Integrate
 *    float8nocompile", Summary) and *delayed* scaling of input, weight and
 *    grad_output from an amax history that is synced after backward
 *    (pytorch/ao issue #1297 "FP8 GPT 1.5B Delayed Scaling 2x Slower than
 *    BF16", repro script: Float8LinearConfig with ScalingType.DELAYED and
 *    sync_float8_amax_and_scale_history after loss.backward()).
 *  - The pages never spell out the arithmetic.  The formats are the OCP 8-bit
 *    floating point formats E4M3 and E5M2 (OCP "OFP8" specification, the
 *    exponent-parameter and value-encoding tables).  The readings taken where
 *    the pages are silent: scale = fmax / max(amax, eps) in fp32 with
 *    eps = 1e-12; cast = fp32 multiply x*scale, then saturate to +-fmax, then
 *    round to nearest, ties to even, onto the fp8 grid; NaN stays NaN; the
 *    sign of zero is kept; subnormals are produced, never flushed.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define FMT_E4M3 0
#define FMT_E5M2 1
#define HIST_LEN 16

/* OCP OFP8 parameters: mantissa bits, exponent bias, largest finite value. */
static int fmt_mbits(int fmt) { return fmt == FMT_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == FMT_E4M3 ? 7 : 15; }
static double fmt_max(int fmt) { return fmt == FMT_E4M3 ? 448.0 : 57344.0; }

/* bfloat16 is the upper half of an IEEE binary32: widening is exact. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

float oracle_bf16_to_f32(uint16_t b) { return bf16_to_f32(b); }

/* ---- fp8 decode: the value an 8-bit code stands for (OCP OFP8 encoding). ----
 * E4M3: exponent field 0 is subnormal, S.1111.111 is NaN, there is no
 * infinity (so S.1111.110 = 448 is the largest finite value).
 * E5M2: IEEE-like; exponent field 31 is +-Inf (mantissa 0) or NaN. */
double oracle_fp8_decode(uint8_t code, int fmt) {
  const int m = fmt_mbits(fmt), bias = fmt_bias(fmt);
  const int ebits = 7 - m;
  const int sign = code >> 7;
  const int E = (code >> m) & ((1 << ebits) - 1);
  const int M = code & ((1 << m) - 1);
  double mag;
  if (fmt == FMT_E4M3 && E == 15 && M == 7) return NAN;
  if (fmt == FMT_E5M2 && E == 31) {
    if (M != 0) return NAN;
    return sign ? -INFINITY : INFINITY;
  }
  if (E == 0)
    mag = ldexp((double)M, 1 - bias - m);             /* subnormal: 0.M * 2^(1-bias) */
  else
    mag = ldexp((double)((1 << m) + M), E - bias - m); /* normal: 1.M * 2^(E-bias) */
  return sign ? -mag : mag;
}

/* ---- fp8 encode with saturation and round-to-nearest-even. ----
 * Steps, in order:
 *   1. NaN -> sign | 0x7F (a NaN code in both formats).
 *   2. |v| is clamped to fmax (this also maps +-Inf to +-fmax).
 *   3. The spacing of the fp8 grid around |v| is q = 2^(max(e, emin) - m),
 *      where 2^e <= |v| < 2^(e+1) and emin = 1 - bias is the smallest normal
 *      exponent (below it the grid is the uniform subnormal grid).
 *   4. n = |v| / q is exact (q is a power of two); it is rounded to the
 *      nearest integer, an exact half going to the even integer.  An even n
 *      is an fp8 value whose mantissa LSB is 0, so this is ties-to-even.
 *   5. The rounded value n*q (<= fmax, since fmax is on the grid) is
 *      re-encoded from its exponent and mantissa.  A carry out of the
 *      mantissa (n = 2^(m+1)) lands in the next binade automatically.
 *   6. The sign bit is copied from v, so -0 encodes as 0x80. */
uint8_t oracle_fp8_encode(float v, int fmt) {
  const int m = fmt_mbits(fmt), bias = fmt_bias(fmt);
  const int emin = 1 - bias;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a, q, n, fl, rem, val;
  int e;
  if (isnan(v)) return (uint8_t)(sign | 0x7F);
  a = fabs((double)v);
  if (a > fmt_max(fmt)) a = fmt_max(fmt);
  if (a == 0.0) return sign;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  e -= 1;       /* now 2^e <= a < 2^(e+1) */
  if (e < emin) e = emin;
  q = ldexp(1.0, e - m);
  n = a / q;
  fl = floor(n);
  rem = n - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  val = fl * q;
  if (val == 0.0) return sign;
  if (val < ldexp(1.0, emin)) { /* subnormal: code mantissa = val / 2^(emin-m) */
    return (uint8_t)(sign | (uint8_t)(val / ldexp(1.0, emin - m)));
  }
  frexp(val, &e);
  e -= 1;
  {
    const int mant = (int)(val / ldexp(1.0, e - m)) - (1 << m);
    return (uint8_t)(sign | ((e + bias) << m) | mant);
  }
}

/* ---- amax = max_i |x_i| over a bf16 tensor (exact: it is one of the inputs'
 * magnitudes).  An empty tensor has amax 0; any NaN makes the result NaN. */
float oracle_amax(const uint16_t *x, int64_t n) {
  float best = 0.0f;
  int saw_nan = 0;
  int64_t i;
#pragma omp parallel for reduction(max : best) reduction(| : saw_nan) schedule(static)
  for (i = 0; i < n; ++i) {
    const float f = fabsf(bf16_to_f32(x[i]));
    if (isnan(f))
      saw_nan = 1;
    else if (f > best)
      best = f;
  }
  return saw_nan ? NAN : best;
}

/* ---- scale = fmax / max(amax, eps) and its inverse, both IEEE binary32
 * divisions (correctly rounded).  eps = 1e-12 (a reading: the pages give no
 * value).  NaN amax gives NaN scales. */
void oracle_scale(float amax, int fmt, float *scale, float *inv_scale) {
  const float eps = 1e-12f;
  const float fmax = (float)fmt_max(fmt);
  float d;
  if (isnan(amax))
    d = amax;
  else
    d = amax > eps ? amax : eps;
  *scale = fmax / d;
  *inv_scale = 1.0f / *scale;
}

/* ---- cast of a bf16 (rows, cols) row-major tensor with a given scale:
 * q[i][j] = encode(fl32(x[i][j] * scale)); optional transposed copy
 * qt[j][i] = q[i][j].  Returns how many products had |x*scale| > fmax (the
 * saturated elements; NaN products are not counted). */
int64_t oracle_cast(const uint16_t *x, int64_t rows, int64_t cols, int fmt, float scale, uint8_t *q,
                    uint8_t *qt) {
  const float fmax = (float)fmt_max(fmt);
  int64_t saturated = 0;
  int64_t i;
#pragma omp parallel for reduction(+ : saturated) schedule(static)
  for (i = 0; i < rows; ++i) {
    int64_t j;
    for (j = 0; j < cols; ++j) {
      const float v = bf16_to_f32(x[i * cols + j]) * scale; /* one binary32 multiply */
      const uint8_t c = oracle_fp8_encode(v, fmt);
      if (fabsf(v) > fmax) ++saturated;
      q[i * cols + j] = c;
    }
  }
  if (qt) {
#pragma omp parallel for schedule(static)
    for (i = 0; i < rows; ++i) {
      int64_t j;
      for (j = 0; j < cols; ++j) qt[j * rows + i] = q[i * cols + j];
    }
  }
  return saturated;
}

/* ---- element-wise encode of fp32 values (scale 1): the conversion alone. */
void oracle_encode_f32(const float *v, int64_t n, int fmt, uint8_t *q) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; ++i) q[i] = oracle_fp8_encode(v[i], fmt);
}

/* Encode the `count` consecutive fp32 bit patterns starting at `lo` (read as
 * uint32), for sweeps over the whole binary32 domain in chunks. */
void oracle_encode_bits_range(uint32_t lo, uint32_t count, int fmt, uint8_t *q) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < (int64_t)count; ++i) {
    const uint32_t u = lo + (uint32_t)i;
    float f;
    memcpy(&f, &u, sizeof f);
    q[i] = oracle_fp8_encode(f, fmt);
  }
}

/* ---- delayed scaling: the amax history of one tensor role. ----
 * The scale for a step comes from the largest amax recorded in the history,
 * which holds past steps only (the history is updated after the step, as the
 * sync call after backward does).  Unused slots hold 0 and cannot raise a max
 * of non-negative values. */
float oracle_history_amax(const float *hist) {
  float best = 0.0f;
  int i;
  for (i = 0; i < HIST_LEN; ++i) {
    if (isnan(hist[i])) return NAN;
    if (hist[i] > best) best = hist[i];
  }
  return best;
}

/* After the step: record this step's amax at `pos`, advance the ring, and
 * count how many slots are filled (saturating at the history length). */
void oracle_history_push(float *hist, int32_t *count, int32_t *pos, float amax_now) {
  hist[*pos] = amax_now;
  *pos = (*pos + 1) % HIST_LEN;
  if (*count < HIST_LEN) *count += 1;
}
