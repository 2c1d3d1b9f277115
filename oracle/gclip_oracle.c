/*
 * gclip_oracle.c -- plain, slow, obviously correct CPU oracle for global
 * L2-norm gradient clipping.  TEST INFRASTRUCTURE ONLY: it exists so that the
 * GPU library can be checked against it.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg load it; the product path never does.
 *
 * What it computes (all in IEEE binary64, one element at a time, in list order):
 *
 *   "Gradient clipping" glossary page (paweldubiel.com), section "Mechanism and
 *   details": for a threshold c > 0, the clipped gradient is g itself when
 *   ||g||_2 <= c and c * g / ||g||_2 otherwise.
 *
 *   "Grad clip" lesson page (unhomeschool.com, ru), section "Math": the norm is
 *   the square root of the sum of g^2 over every element of every parameter
 *   tensor (the whole list is one vector, section "Two variants: Per-Tensor or
 *   Global"), and the factor applied when clipping is max_norm / norm.
 *
 *   "Backprop" lesson page (unhomeschool.com, vi), section "Accumulation across
 *   microbatches": after summing microbatch gradients the buffer is averaged by
 *   1/n_microbatches before the optimizer step; the glossary page, section
 *   "Order changes the result", puts clipping after the whole effective batch
 *   has been collected.  So the norm is that of the averaged gradient a*g and
 *   the factor written back is a * coef.
 *
 *   Glossary page, section "Mechanism and details", last paragraph: a NaN or
 *   infinite value calls for diagnosis, and an error-if-nonfinite switch lets
 *   the caller stop that update.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - the tie norm == c leaves the gradient unchanged (both pages write "<=");
 *   - no epsilon is added to the norm before dividing;
 *   - "non-finite" is tested on the elements (any NaN or +-Inf);
 *   - with the stop switch on and a non-finite element, nothing is written;
 *   - with the switch off, plain IEEE arithmetic decides (NaN > c is false);
 *   - outputs are rounded once, to nearest-even, into the storage format,
 *     keeping subnormals and overflowing to +-Inf.
 *
 * Storage formats are decoded and encoded from their bit layouts (IEEE 754
 * binary32 and binary16; bfloat16 is the top half of binary32), not through
 * any GPU code.  Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

/* exponent bits / stored mantissa bits / bytes per element of each format */
static int fmt_ebits(int dt) { return dt == OR_F16 ? 5 : 8; }
static int fmt_mbits(int dt) { return dt == OR_F32 ? 23 : (dt == OR_F16 ? 10 : 7); }
static int fmt_bytes(int dt) { return dt == OR_F32 ? 4 : 2; }

static uint32_t load_bits(const void* base, int64_t i, int dt) {
  if (fmt_bytes(dt) == 4) {
    uint32_t b;
    memcpy(&b, (const unsigned char*)base + 4 * i, 4);
    return b;
  }
  uint16_t h;
  memcpy(&h, (const unsigned char*)base + 2 * i, 2);
  return h;
}

static void store_bits(void* base, int64_t i, int dt, uint32_t b) {
  if (fmt_bytes(dt) == 4) {
    memcpy((unsigned char*)base + 4 * i, &b, 4);
  } else {
    uint16_t h = (uint16_t)b;
    memcpy((unsigned char*)base + 2 * i, &h, 2);
  }
}

/* Value of a bit pattern: (-1)^s * 1.m * 2^(e-bias) for normal numbers,
 * (-1)^s * 0.m * 2^(1-bias) for subnormals, Inf/NaN when e is all ones. */
double oracle_decode_bits(uint32_t bits, int32_t dt) {
  const int eb = fmt_ebits(dt), mb = fmt_mbits(dt);
  const int bias = (1 << (eb - 1)) - 1;
  const uint32_t sign = (bits >> (eb + mb)) & 1u;
  const uint32_t e = (bits >> mb) & ((1u << eb) - 1u);
  const uint32_t m = bits & ((1u << mb) - 1u);
  double v;
  if (e == (1u << eb) - 1u) {
    v = (m == 0) ? INFINITY : NAN;
  } else if (e == 0) {
    v = ldexp((double)m, 1 - bias - mb);
  } else {
    v = ldexp((double)((1u << mb) + m), (int)e - bias - mb);
  }
  return sign ? -v : v;
}

/* Round a binary64 value once, to nearest with ties to even, into the format
 * and return its bit pattern.  Subnormal results are kept; a result whose
 * rounded magnitude exceeds the largest finite value becomes +-Inf. */
uint32_t oracle_encode(double x, int32_t dt) {
  const int eb = fmt_ebits(dt), mb = fmt_mbits(dt);
  const int bias = (1 << (eb - 1)) - 1;
  const int emin = 1 - bias, emax = bias;
  const uint32_t sign = signbit(x) ? (1u << (eb + mb)) : 0u;
  const uint32_t exp_all = ((1u << eb) - 1u) << mb;
  if (isnan(x)) return sign | exp_all | (1u << (mb - 1));
  if (isinf(x)) return sign | exp_all;
  if (x == 0.0) return sign;
  double a = fabs(x);
  int e2;
  (void)frexp(a, &e2);
  int E = e2 - 1;                       /* 2^E <= a < 2^(E+1) */
  if (E > emax) return sign | exp_all;  /* already beyond the top binade */
  if (E < emin) E = emin;               /* subnormal range: fixed quantum */
  const double q = ldexp(a, mb - E);    /* a / quantum, exact (power of two) */
  double r = nearbyint(q);              /* default rounding: nearest, ties even */
  const double one = ldexp(1.0, mb);    /* 2^mb: the implicit leading bit */
  if (r >= 2.0 * one) {                 /* rounded up into the next binade */
    r = one;
    E += 1;
    if (E > emax) return sign | exp_all;
  }
  if (r >= one) {
    return sign | ((uint32_t)(E + bias) << mb) | (uint32_t)(r - one);
  }
  return sign | (uint32_t)r; /* subnormal or zero: biased exponent 0 */
}

double oracle_decode(const void* base, int64_t i, int32_t dt) {
  return oracle_decode_bits(load_bits(base, i, dt), dt);
}

static int dtype_ok(int32_t dt) { return dt == OR_F32 || dt == OR_F16 || dt == OR_BF16; }

/* Sum over every element of every tensor, in list order, of (a*g)^2; also
 * whether any element is NaN or +-Inf.  Returns 0, or -1 on a bad argument. */
int oracle_sumsq(const void* const* ptrs, const int64_t* numels, int32_t n, int32_t dt, double avg,
                 double* sumsq, int32_t* nonfinite) {
  if (n < 0 || !dtype_ok(dt) || !sumsq || !nonfinite) return -1;
  double total = 0.0;
  int32_t nf = 0;
  for (int32_t t = 0; t < n; ++t) {
    if (numels[t] < 0) return -1;
    for (int64_t i = 0; i < numels[t]; ++i) {
      const double g = oracle_decode(ptrs[t], i, dt);
      if (!isfinite(g)) nf = 1;
      const double u = avg * g;
      total += u * u;
    }
  }
  *sumsq = total;
  *nonfinite = nf;
  return 0;
}

/* Sum of (a*g)^2 of each tensor on its own (per-tensor diagnostics). */
int oracle_tensor_sumsq(const void* const* ptrs, const int64_t* numels, int32_t n, int32_t dt, double avg,
                        double* out) {
  if (n < 0 || !dtype_ok(dt) || !out) return -1;
  for (int32_t t = 0; t < n; ++t) {
    if (numels[t] < 0) return -1;
    double s = 0.0;
    for (int64_t i = 0; i < numels[t]; ++i) {
      const double u = avg * oracle_decode(ptrs[t], i, dt);
      s += u * u;
    }
    out[t] = s;
  }
  return 0;
}

/* The decision.  coef = c / norm when norm > c (strictly), else 1; the factor
 * written back is a * coef.  skip = 1 when a non-finite element was seen and
 * the caller asked to stop such an update: then nothing is written. */
int oracle_decide(double norm, int32_t nonfinite, double max_norm, double avg, int32_t error_if_nonfinite,
                  double* scale, int32_t* clipped, int32_t* skip) {
  if (!scale || !clipped || !skip) return -1;
  const int32_t clip = (norm > max_norm) ? 1 : 0;
  const double coef = clip ? max_norm / norm : 1.0;
  *clipped = clip;
  *skip = (nonfinite && error_if_nonfinite) ? 1 : 0;
  *scale = avg * coef;
  return 0;
}

/* In place: g <- round(g * s) for every element, unless s == 1 (nothing to
 * do: the gradient passes unchanged, so no byte is rewritten). */
int oracle_scale(void* const* ptrs, const int64_t* numels, int32_t n, int32_t dt, double s) {
  if (n < 0 || !dtype_ok(dt)) return -1;
  if (s == 1.0) return 0;
  for (int32_t t = 0; t < n; ++t) {
    if (numels[t] < 0) return -1;
    for (int64_t i = 0; i < numels[t]; ++i) {
      const double g = oracle_decode(ptrs[t], i, dt);
      store_bits(ptrs[t], i, dt, oracle_encode(g * s, dt));
    }
  }
  return 0;
}

/* The whole path: norm of the averaged gradient, decision, scale in place.
 * out[0] = sumsq, out[1] = norm, out[2] = applied factor; flags[0] =
 * nonfinite, flags[1] = clipped, flags[2] = skipped (nothing written). */
int oracle_clip(void* const* ptrs, const int64_t* numels, int32_t n, int32_t dt, double max_norm, double avg,
                int32_t error_if_nonfinite, double* out, int32_t* flags) {
  if (!out || !flags) return -1;
  double sumsq;
  int32_t nonfinite;
  if (oracle_sumsq((const void* const*)ptrs, numels, n, dt, avg, &sumsq, &nonfinite) != 0) return -1;
  const double norm = sqrt(sumsq);
  double s;
  int32_t clipped, skip;
  oracle_decide(norm, nonfinite, max_norm, avg, error_if_nonfinite, &s, &clipped, &skip);
  out[0] = sumsq;
  out[1] = norm;
  out[2] = skip ? 1.0 : s;
  flags[0] = nonfinite;
  flags[1] = clipped;
  flags[2] = skip;
  if (skip) return 0;
  return oracle_scale(ptrs, numels, n, dt, s);
}

/* Accumulation across microbatches (backprop lesson, section "Accumulation
 * across microbatches"): the backward pass of every microbatch adds its
 * gradient into the gradient buffer (+=, not =), and the clip runs once the
 * last one is in (glossary page, section "Order changes the result").  One
 * such +=: acc[i] <- acc[i] + g[i] for every element, rounded once to the
 * storage format.  The sum is formed in binary64 and then rounded to the
 * format; binary64 carries at least 2p + 2 bits for every format here (p =
 * 24, 11 and 8), so that pair of roundings gives the correctly rounded sum in
 * the format, the IEEE addition of the format itself.  acc and g hold n
 * tensors of numels[t] elements of format dt; g is only read. */
int oracle_accumulate(void* const* acc, const void* const* g, const int64_t* numels, int32_t n, int32_t dt) {
  if (n < 0 || !dtype_ok(dt) || (n > 0 && (!acc || !g || !numels))) return -1;
  for (int32_t t = 0; t < n; ++t) {
    if (numels[t] < 0) return -1;
    for (int64_t i = 0; i < numels[t]; ++i) {
      const double s = oracle_decode(acc[t], i, dt) + oracle_decode(g[t], i, dt);
      store_bits(acc[t], i, dt, oracle_encode(s, dt));
    }
  }
  return 0;
}

/* Per-tensor clipping (grad clip lesson, section "Two variants: Per-Tensor
 * or Global"): every tensor is clipped on its own, by its own norm -- the
 * case split of the global clip with one tensor in place of the whole list.
 * Readings where the pages are silent: the averaging factor a multiplies
 * every tensor before its norm is taken, as in the global clip; the stop
 * switch stops the whole update, so one NaN/Inf anywhere in the list and no
 * tensor is written.
 * Per tensor t: tout[3t] = sumsq, tout[3t+1] = norm, tout[3t+2] = the factor
 * written (1 when nothing is written); tflags[2t] = nonfinite, tflags[2t+1] =
 * clipped.  For the list: out[0] = sumsq, out[1] = norm; flags[0] = any
 * nonfinite, flags[1] = any tensor clipped, flags[2] = skipped. */
int oracle_clip_per_tensor(void* const* ptrs, const int64_t* numels, int32_t n, int32_t dt, double max_norm,
                           double avg, int32_t error_if_nonfinite, double* tout, int32_t* tflags, double* out,
                           int32_t* flags) {
  if (n < 0 || !out || !flags || (n > 0 && (!tout || !tflags))) return -1;
  double list_sumsq;
  int32_t list_nf;
  if (oracle_sumsq((const void* const*)ptrs, numels, n, dt, avg, &list_sumsq, &list_nf) != 0) return -1;
  const int32_t skip = (list_nf && error_if_nonfinite) ? 1 : 0;
  int32_t any_clipped = 0;
  for (int32_t t = 0; t < n; ++t) {
    double s_t;
    int32_t nf_t, clipped_t, unused;
    oracle_sumsq((const void* const*)&ptrs[t], &numels[t], 1, dt, avg, &tout[3 * t], &nf_t);
    tout[3 * t + 1] = sqrt(tout[3 * t]);
    oracle_decide(tout[3 * t + 1], nf_t, max_norm, avg, error_if_nonfinite, &s_t, &clipped_t, &unused);
    tout[3 * t + 2] = skip ? 1.0 : s_t;
    tflags[2 * t] = nf_t;
    tflags[2 * t + 1] = clipped_t;
    any_clipped |= clipped_t;
    if (!skip) oracle_scale(&ptrs[t], &numels[t], 1, dt, s_t);
  }
  out[0] = list_sumsq;
  out[1] = sqrt(list_sumsq);
  flags[0] = list_nf;
  flags[1] = any_clipped;
  flags[2] = skip;
  return 0;
}

/* One AdamW step on one tensor, after the clip.  Grad clip lesson, section
 * "Order matters: Pre-Adam": the clip runs before AdamW's moments m, v and
 * the weights are updated, so the moments only ever see the clipped
 * gradient; backprop lesson, section "Optimizer state": AdamW keeps the two
 * moments per weight, in binary32 beside binary32 weights (section "Signals
 * & checkpoints").  The update itself is not printed on the pages; it is
 * AdamW as published (Loshchilov and Hutter, "Decoupled weight decay
 * regularization", with the bias-corrected moments of Kingma and Ba's Adam),
 * in binary64, element by element:
 *   g    = s * grad                        (s: the factor the clip decided)
 *   m'   = b1 * m + (1 - b1) * g
 *   v'   = b2 * v + (1 - b2) * g * g
 *   mhat = m' / (1 - b1^step),  vhat = v' / (1 - b2^step)
 *   p'   = p - lr * (mhat / (sqrt(vhat) + eps) + wd * p)
 * step >= 1 counts the optimizer steps taken, this one included.  Inputs are
 * the binary32 weights and moments and the gradient in format dt; results
 * are binary64. */
int oracle_adamw(const float* p, const void* grad, const float* m, const float* v, int64_t n, int32_t dt,
                 double s, double lr, double b1, double b2, double eps, double wd, int64_t step,
                 double* p_out, double* m_out, double* v_out) {
  if (n < 0 || !dtype_ok(dt) || step < 1 || !p_out || !m_out || !v_out) return -1;
  const double bc1 = 1.0 - pow(b1, (double)step);
  const double bc2 = 1.0 - pow(b2, (double)step);
  for (int64_t i = 0; i < n; ++i) {
    const double g = s * oracle_decode(grad, i, dt);
    const double mi = b1 * (double)m[i] + (1.0 - b1) * g;
    const double vi = b2 * (double)v[i] + (1.0 - b2) * g * g;
    const double mhat = mi / bc1;
    const double vhat = vi / bc2;
    const double pi = (double)p[i];
    p_out[i] = pi - lr * (mhat / (sqrt(vhat) + eps) + wd * pi);
    m_out[i] = mi;
    v_out[i] = vi;
  }
  return 0;
}

/* Loss scaling (glossary page, introduction and section "Order changes the
 * result"): with loss scaling the gradients are unscaled first, so that the
 * threshold applies to their true size.  The averaging factor of a step is
 * then a = 1 / (n_microbatches * S) for the binary32 loss scale S, and the
 * norm, the decision and the written factor follow from it as above. */
double oracle_amp_avg(double n_microbatches, float scale) {
  return 1.0 / (n_microbatches * (double)scale);
}

/* The loss scale after a step.  The pages do not give the rule; it is
 * dynamic loss scaling as published (Micikevicius et al., "Mixed precision
 * training"): after a step whose gradients held a NaN or Inf the scale is
 * multiplied by backoff and the count of clean steps restarts from 0;
 * otherwise the count grows by one, and when it reaches interval the scale
 * is multiplied by growth -- unless that product is not finite in binary32
 * -- and the count restarts.  Products are formed in binary64 and rounded
 * once to the binary32 scale. */
int oracle_amp_update(float* scale, int32_t* tracker, int32_t found_inf, double growth, double backoff,
                      int32_t interval) {
  if (!scale || !tracker || interval < 1) return -1;
  if (found_inf) {
    *scale = (float)((double)*scale * backoff);
    *tracker = 0;
    return 0;
  }
  const int32_t clean = *tracker + 1;
  if (clean == interval) {
    const float grown = (float)((double)*scale * growth);
    if (isfinite(grown)) *scale = grown;
    *tracker = 0;
  } else {
    *tracker = clean;
  }
  return 0;
}
