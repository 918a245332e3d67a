/* Plain C twin of two oracle steps, for parity checks at full workload sizes.

   TEST INFRASTRUCTURE ONLY, like the rest of this folder: only the tests,
   the smoke check and the CPU-baseline leg of the benchmark may load it. It
   shares no code with the HIP library and includes no header of it.

   The numpy oracle (moe_oracle.py) is the definition; these loops compute the
   same two results with C's own arithmetic, much faster, and the CPU tests
   check them against the numpy oracle bit for bit (exhaustively for the FP8
   codes) and against exact rational arithmetic:

   oc_quantize_fp8  per token and 128-column block (DeepEP article, "Support
                    FP8 et MXFP8": FP8 payloads; reading R6): a = max |x|,
                    scale = fp32(a / 448), inv = fp32(448 / a), code =
                    e4m3fn(fp32(x * inv)) rounded to nearest even with
                    saturation at +-448; a zero input keeps its signed zero.
   oc_combine       out[t] = bf16( fp32 chain over the live slots j in order
                    of acc = fmaf(w[t,j], y[dst_row[t,j]], acc), acc = +0 )
                    (glossary "Expert Parallelism", "Le pattern de
                    communication all-to-all", Phase 2; reading R14). C's
                    fmaf rounds a*b + c once, as the reading requires.
   Both loop over tokens in order, one element at a time. */

#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Nearest bf16 (ties to even) of a finite or infinite fp32 value: add half of
   the dropped quantum, minus one when the kept part is even, and cut. */
static uint16_t bf16_round(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) return 0x7FC0; /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* OCP e4m3fn code of an fp32 value: 1 sign bit, 4 exponent bits (bias 7),
   3 mantissa bits, subnormals m * 2^-9, no infinities, largest 448. */
static uint8_t e4m3_code(float v) {
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double a = fabs((double)v);
  if (!(a < 448.0)) return sign | 0x7E;          /* saturate (also +-inf) */
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);                                  /* a = m * 2^ex, m in [0.5, 1) */
  int e = ex - 1;                                 /* floor(log2 a) */
  if (e < -6) e = -6;                             /* subnormal spacing 2^-9 */
  const double q = ldexp(1.0, e - 3);
  const double r = nearbyint(a / q) * q;          /* ties to even */
  if (r >= 448.0) return sign | 0x7E;
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));   /* subnormal */
  frexp(r, &ex);
  const int er = ex - 1;
  const int m = (int)(r / ldexp(1.0, er) * 8.0) - 8;
  return sign | (uint8_t)(((er + 7) << 3) | m);
}

void oc_quantize_fp8(int64_t tokens, int64_t hidden, const uint16_t* x, uint8_t* codes,
                     float* scales) {
  const int64_t nb = hidden / 128;
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint16_t* xb = x + t * hidden + b * 128;
      float amax = 0.0f;
      for (int i = 0; i < 128; ++i) {
        const float a = fabsf(bf16_value(xb[i]));
        if (a > amax) amax = a;
      }
      const float scale = amax / 448.0f;
      const float inv = 448.0f / amax;            /* +inf when amax = 0 */
      scales[t * nb + b] = scale;
      for (int i = 0; i < 128; ++i) {
        const float xv = bf16_value(xb[i]);
        const float p = xv == 0.0f ? xv : xv * inv;
        codes[t * hidden + b * 128 + i] = e4m3_code(p);
      }
    }
  }
}

/* weights may be NULL: every weight is then 1 (the gradient of dispatch).
   dst_row values < 0 or >= num_rows add nothing. acc is a caller-provided
   fp32 row of `hidden` values. */
void oc_combine(int64_t tokens, int64_t hidden, int64_t top_k, int64_t num_rows,
                const uint16_t* y, const int32_t* dst_row, const float* weights,
                uint16_t* out, float* acc) {
  for (int64_t t = 0; t < tokens; ++t) {
    for (int64_t h = 0; h < hidden; ++h) acc[h] = 0.0f;
    for (int64_t j = 0; j < top_k; ++j) {
      const int64_t d = dst_row[t * top_k + j];
      if (d < 0 || d >= num_rows) continue;
      const float w = weights ? weights[t * top_k + j] : 1.0f;
      const uint16_t* row = y + d * hidden;
      for (int64_t h = 0; h < hidden; ++h) acc[h] = fmaf(w, bf16_value(row[h]), acc[h]);
    }
    for (int64_t h = 0; h < hidden; ++h) out[t * hidden + h] = bf16_round(acc[h]);
  }
}
