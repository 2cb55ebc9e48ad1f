/*
 * Plain C forms of four oracle steps, for full-size checks where the numpy
 * forms are too slow (TEST INFRASTRUCTURE ONLY: loaded by oracle/native.py,
 * which only the tests, the smoke check and the bench's CPU baseline use).
 * Each function restates the numpy oracle's definition step for step, with
 * no blocking or reordering beyond a loop over independent outputs; the CPU
 * tests hold them to the numpy oracle bit for bit.
 *
 * [KANANA-FP8] / [DSV3-FP8] ("Kakao Kanana-2 pre-training deep dive", FP8
 * paragraph; "DeepSeek-V3 technical report summary", section 2.2):
 * 128x128-block weight quantisation and block-scaled FP8 GEMMs with
 * higher-precision accumulation.
 *
 * Built with -O2 -ffp-contract=off (no fused multiply-add, no fast-math):
 * every float operation below is one IEEE binary32 or binary64 operation.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* OCP E4M3FN encoding (RNE, sign kept) of a finite value with |v| <= 448:
 * the spacing of representable values in the binade [2^e, 2^(e+1)) is
 * 2^(e-3) for e >= -6 and 2^-9 below (subnormals); divide by it (exact, a
 * power of two), round half to even, multiply back, read the fields. */
static uint8_t e4m3_encode(double v) {
  const int neg = signbit(v) ? 1 : 0;
  const double a = fabs(v);
  int ex = 0;
  (void)frexp(a, &ex); /* a = f 2^ex, f in [0.5, 1) */
  int e = ex - 1;
  if (e < -6) e = -6;
  const double spacing = ldexp(1.0, e - 3);
  const double q = nearbyint(a / spacing) * spacing; /* round-to-nearest-even mode */
  uint8_t code;
  if (q == 0.0) {
    code = 0;
  } else if (q < 0x1p-6) {
    code = (uint8_t)(q / 0x1p-9); /* exponent field 0: m * 2^-9 */
  } else {
    int qe = 0;
    (void)frexp(q, &qe);
    qe -= 1;
    const int m = (int)((q / ldexp(1.0, qe) - 1.0) * 8.0);
    code = (uint8_t)(((qe + 7) << 3) | m);
  }
  return (uint8_t)(code | (neg << 7));
}

/* Value of an E4M3FN code (NaN for 0x7F / 0xFF). */
static double e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? m * 0x1p-9 : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -mag : mag;
}

void orc_e4m3_encode_many(const double* v, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(v[i]);
}

/* 128x128-block quantisation of w [G, rows, cols] (binary32 values):
 * amax = max |x| over the block; s = fl32(amax / 448) (1 if amax == 0);
 * code = encode(clamp(fl32(x / s), -448, 448)). */
void orc_quant_weight_128x128(const float* w, int64_t G, int32_t rows, int32_t cols, uint8_t* q, float* s) {
  const int64_t br = rows / 128, bc = cols / 128;
  const int64_t nblk = G * br * bc;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t b = 0; b < nblk; ++b) {
    const int64_t g = b / (br * bc), i = (b / bc) % br, j = b % bc;
    const float* blk = w + (g * rows + i * 128) * (int64_t)cols + j * 128;
    uint8_t* qb = q + (g * rows + i * 128) * (int64_t)cols + j * 128;
    float amax = 0.0f;
    for (int r = 0; r < 128; ++r)
      for (int c = 0; c < 128; ++c) {
        const float a = fabsf(blk[(int64_t)r * cols + c]);
        if (a > amax) amax = a;
      }
    const float sc = amax == 0.0f ? 1.0f : amax / 448.0f;
    s[b] = sc;
    for (int r = 0; r < 128; ++r)
      for (int c = 0; c < 128; ++c) {
        float y = blk[(int64_t)r * cols + c] / sc;
        if (y > 448.0f) y = 448.0f;
        if (y < -448.0f) y = -448.0f;
        qb[(int64_t)r * cols + c] = e4m3_encode((double)y);
      }
  }
}

/* Rows of a block-scaled FP8 GEMM against one weight matrix, C = A . B^T:
 *   C[m, n]   = sum_kb P_kb[m, n] * (sa[m, kb] * sb[n / 128, kb])
 *   Mag[m, n] = sum_kb |P|_kb[m, n] * |sa[m, kb] * sb[n / 128, kb]|
 * with P_kb the float64 sum of the decoded products over the 128-wide chunk
 * kb (exact: products are multiples of 2^-18 below 2^18, 128 of them need
 * at most 43 bits), the scale product of two binary32 numbers exact in
 * float64, and the chunks added in order.
 *  aq [m, K] codes, as [m, K/128]; bq [N, K] codes, bs [N/128, K/128];
 *  C, Mag [m, N] (Mag may be NULL). */
void orc_gemm_rows(const uint8_t* aq, const float* as, int64_t m, const uint8_t* bq, const float* bs, int32_t N,
                   int32_t K, double* C, double* Mag) {
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = e4m3_decode((uint8_t)c);
  const int KB = K / 128;
#pragma omp parallel for schedule(static)
  for (int32_t n = 0; n < N; ++n) {
    double brow[128];
    double babs[128];
    for (int64_t i = 0; i < m; ++i) {
      C[i * N + n] = 0.0;
      if (Mag) Mag[i * N + n] = 0.0;
    }
    for (int kb = 0; kb < KB; ++kb) {
      const uint8_t* b = bq + (int64_t)n * K + (int64_t)kb * 128;
      for (int k = 0; k < 128; ++k) {
        brow[k] = lut[b[k]];
        babs[k] = fabs(brow[k]);
      }
      const double sbv = (double)bs[(int64_t)(n / 128) * KB + kb];
      for (int64_t i = 0; i < m; ++i) {
        const uint8_t* a = aq + i * K + (int64_t)kb * 128;
        double p = 0.0, pm = 0.0;
        for (int k = 0; k < 128; ++k) {
          const double av = lut[a[k]];
          p += av * brow[k];
          pm += fabs(av) * babs[k];
        }
        const double sc = (double)as[i * KB + kb] * sbv;
        C[i * N + n] += p * sc;
        if (Mag) Mag[i * N + n] += pm * fabs(sc);
      }
    }
  }
}

/* The binary32 sigmoid specification of oracle/specmath.py, step for step
 * (each line one correctly rounded binary32 operation, no fused
 * multiply-add):
 *   E(y): y = min(max(y, -80), 80); n = rint(y * LOG2E);
 *         r = (y - n LN2_HI) - n LN2_LO  (Cody & Waite);
 *         p = Horner of fl32(1/k!), k = 7..0, at r;  E = p * 2^n
 *   sigmoid(x) = 1 / (1 + E(-x))
 * The constants are passed in from specmath.py (so both forms use the same
 * binary32 values), as ln2hi, ln2lo, log2e and taylor[0..7]. */
static float spec_sigmoid(float x, float log2e, float ln2hi, float ln2lo, const float* taylor) {
  float y = -x;
  y = fminf(fmaxf(y, -80.0f), 80.0f);
  const float n = rintf(y * log2e);
  const float r = (y - n * ln2hi) - n * ln2lo;
  float p = taylor[7];
  for (int k = 6; k >= 0; --k) p = p * r + taylor[k];
  uint32_t tb = (uint32_t)((int32_t)n + 127) << 23;
  float two_n;
  memcpy(&two_n, &tb, 4);
  const float e = p * two_n;
  return 1.0f / (1.0f + e);
}

/* sigmoid of the n binary32 values whose bit patterns are start, start + 1,
 * ... (wrapping modulo 2^32); NaN patterns give NaN. */
void orc_spec_sigmoid_bits(uint32_t start, int64_t n, float log2e, float ln2hi, float ln2lo,
                           const float* taylor, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t b = start + (uint32_t)i;
    float x;
    memcpy(&x, &b, 4);
    out[i] = isnan(x) ? NAN : spec_sigmoid(x, log2e, ln2hi, ln2lo, taylor);
  }
}

void orc_spec_sigmoid(const float* x, int64_t n, float log2e, float ln2hi, float ln2lo, const float* taylor,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = isnan(x[i]) ? NAN : spec_sigmoid(x[i], log2e, ln2hi, ln2lo, taylor);
}
