/*
 * hqq_oracle.c -- plain, slow, fp64 CPU oracle for group-wise HQQ quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path (the
 * HIP library) never calls, links or includes anything from this directory, and
 * this file includes nothing from the product path.
 *
 * Source of the method: the web page "Half-Quadratic Quantization of Large
 * Machine Learning Models" (Dropbox tech blog, in the csdn translation):
 *   - section 2: objective argmin_{z,s} phi(W - Q^-1(Q(W))), the affine
 *     quantizer Q(W) = round(W/s + z) and its inverse Q^-1(W_q) = s(W_q - z),
 *     the half-quadratic split with s fixed (only z is optimized), and the
 *     alternating updates sp1 (W_e), sp2 (z), beta <- kappa*beta;
 *   - section 2.1: generalized lp soft-threshold
 *       shrink(x, beta) = sign(x) * relu(|x| - |x|^(p-1) / beta);
 *   - section 2.2: closed-form z update, the mean over the group axis of
 *       W_q - (W - W_e)/s, implemented with the inverse scale 1/s;
 *   - section 4.1: p = 0.7, beta = 1, kappa = 1.01, 20 iterations, early
 *     exit once the error stops improving, group-wise buffers.
 *
 * Readings where the page is silent (each listed in the design notes):
 *   init     min-max: s = (max-min)/qmax, inv_s = qmax/(max-min), z = -min*inv_s
 *            (real-valued z); a constant group takes s = inv_s = 1.
 *   round    round half to even.  At the initial zero-point z0 = -min/s the value
 *            w/s + z0 = (w - min) qmax / (max - min) is a ratio of binary16
 *            differences, and its code is decided exactly (integer-valued fp64
 *            comparisons, no rounding); at later steps z is the oracle's fp64
 *            iterate and the code is nearbyint of the fp64 value w (1/s) + z.
 *   clamp    codes clamped to [0, qmax] after rounding.
 *   shrink   exactly the section-2.1 operator; 0 at x = 0 (where |x|^(p-1)
 *            is undefined for p < 1).
 *   error    e = sum_k |r_k|^err_pow over the group with r = W - Q^-1(Q(W)),
 *            |0|^anything := 0; err_pow = p is the reading used everywhere
 *            (phi of the section-2 objective); 1 and 2 exist only as a
 *            sensitivity switch.
 *   stop     per group; an evaluation is accepted only if its error is
 *            strictly below the best so far, otherwise the solver stops and
 *            keeps the best (last accepted) z.  With T iterations there are at
 *            most T+1 evaluations and T z-updates.
 *   storage  codes packed as an LSB-first little-endian bitstream over the
 *            row-major element order; s and z stored as IEEE binary16 (RNE
 *            from fp64, no intermediate fp32 rounding).
 *   meta     section 4.1 quantizes the zero-points to 8 bits without grouping
 *            or optimization, and its table note the scales to 8 bits in groups
 *            of 128: affine min-max round-to-nearest (no solver) over the stored
 *            binary16 values, one group per array for the zero-points, runs of
 *            128 consecutive values (row-major group order, shorter last run) for
 *            the scales; the group min and max map to codes 0 and 255, the code
 *            is the exact half-even rounding of (v - min) 255 / (max - min); a
 *            constant group takes scale 1, codes 0; the meta scale and offset are
 *            stored as binary16, a zero offset as +0.
 *
 * Arithmetic: fp64, one thread, scalar loops, sums in index order.  The binary16
 * conversions are written out from the IEEE 754 definition (no compiler
 * half-precision type is used).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "hqq_oracle.h"

/* ------------------------------------------------------------------------- */
/* IEEE 754 binary16 <-> binary64, by definition.                            */
/* ------------------------------------------------------------------------- */

double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

uint16_t oracle_f64_to_f16(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isnan(v)) return 0x7e00;
  /* 65520 is the midpoint between 65504 (largest finite, odd significand) and
   * 2^16; RNE sends it and everything above to infinity. */
  if (a >= 65520.0) return sign | 0x7c00;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: quantum 2^-24; n in [0, 1024], n == 1024 encodes the
     * smallest normal, which the continuous encoding below gives for free. */
    double n = nearbyint(ldexp(a, 24));
    return sign | (uint16_t)n;
  }
  int E;
  (void)frexp(a, &E); /* a = f * 2^E, f in [0.5, 1) */
  int e = E - 1;      /* a in [2^e, 2^(e+1)) */
  double n = nearbyint(ldexp(a, 10 - e)); /* significand in [1024, 2048] */
  /* n == 2048 rolls over into the next binade through the encoding itself */
  uint32_t bits = ((uint32_t)(e + 15) << 10) + (uint32_t)(n - 1024.0);
  if (bits >= 0x7c00) return sign | 0x7c00;
  return sign | (uint16_t)bits;
}

void oracle_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_to_f16_array(const double* v, int64_t n, uint16_t* out) {
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(v[i]);
}

/* ------------------------------------------------------------------------- */
/* The steps of the method.                                                  */
/* ------------------------------------------------------------------------- */

/* Generalized lp soft-threshold of section 2.1, as printed; 0 at x = 0. */
double oracle_shrink_lp(double x, double beta, double p) {
  if (x == 0.0) return 0.0;
  double ax = fabs(x);
  double v = ax - pow(ax, p - 1.0) / beta;
  if (v < 0.0) v = 0.0; /* relu */
  return x > 0.0 ? v : -v;
}

/* Q_{z,s}(W) of section 2 with the inverse scale: clamp(round(w*inv_s + z)),
 * the pre-round value formed in fp64 and rounded half to even (nearbyint under
 * FE_TONEAREST).  Used at every step after the first, where z is the oracle's
 * own fp64 iterate. */
double oracle_quantize_value(double w, double inv_s, double z, int qmax) {
  double x = w * inv_s + z;
  double q = nearbyint(x);
  if (q < 0.0) q = 0.0;
  if (q > (double)qmax) q = (double)qmax;
  return q;
}

/* Half-even rounding of the exact ratio num/den (den > 0, num >= 0), for num and den
 * that are multiples of 2^-24 below 2^25 and 2^17 and ratios below 256: every
 * product k*den and difference below is then an exact fp64 value (at most 50
 * significant bits), so the decision involves no rounding at all.  Returns the
 * integer nearest num/den; at an exact midpoint the even one. */
double oracle_round_ratio(double num, double den) {
  double k = floor(num / den); /* a guess within one of the floor */
  while (k * den > num) k -= 1.0;
  while ((k + 1.0) * den <= num) k += 1.0;
  /* now k*den <= num < (k+1)*den exactly; compare the remainder with den/2 */
  const double rem2 = 2.0 * (num - k * den);
  if (rem2 < den) return k;
  if (rem2 > den) return k + 1.0;
  return fmod(k, 2.0) == 0.0 ? k : k + 1.0; /* exact midpoint: half to even */
}

/* The code of w at the initial zero-point z0 = -mn/s with s = (mx - mn)/qmax: the
 * value w/s + z0 is exactly (w - mn) qmax / (mx - mn).  For binary16 w, mn, mx the
 * difference w - mn and the product with qmax are exact in fp64, so the code is the
 * exact half-even rounding of that ratio (a constant group, mx = mn, has s = 1 and
 * code 0).  fp64 evaluation of w*(1/s) + z0 would instead move exact midpoints,
 * such as the mid-range element with odd qmax, by rounding noise. */
double oracle_quantize_init_value(double w, double mn, double mx, int qmax) {
  if (!(mx > mn)) return 0.0;
  double q = oracle_round_ratio((w - mn) * (double)qmax, mx - mn);
  if (q < 0.0) q = 0.0;
  if (q > (double)qmax) q = (double)qmax;
  return q;
}

/* Min-max initialisation (reading: the group min and max map to 0 and qmax). */
void oracle_minmax_init(const double* w, int g, int qmax, double* s, double* inv_s, double* z) {
  double mn = w[0], mx = w[0];
  for (int k = 1; k < g; ++k) {
    if (w[k] < mn) mn = w[k];
    if (w[k] > mx) mx = w[k];
  }
  if (mx > mn) {
    *s = (mx - mn) / (double)qmax;
    *inv_s = (double)qmax / (mx - mn);
  } else {
    *s = 1.0;
    *inv_s = 1.0;
  }
  *z = -mn * (*inv_s);
}

/* sum_k |r_k|^err_pow with |0|^anything := 0 (phi of the section-2 objective). */
double oracle_group_error(const double* r, int g, double err_pow) {
  double e = 0.0;
  for (int k = 0; k < g; ++k) {
    if (r[k] != 0.0) e += pow(fabs(r[k]), err_pow);
  }
  return e;
}

/* sp2 of section 2.2: z = mean over the group of (W_q - (W - W_e) * inv_s). */
double oracle_z_update(const double* q, const double* w, const double* we, double inv_s, int g) {
  double acc = 0.0;
  for (int k = 0; k < g; ++k) acc += q[k] - (w[k] - we[k]) * inv_s;
  return acc / (double)g;
}

/* One group through the whole solver.  `trace` (may be NULL) receives every
 * evaluated error e_0, e_1, ... in order and `z_trace` (may be NULL) the z of
 * each evaluation; *n_trace their count.
 *
 * Tie replay (test infrastructure): `n_flip` pairs (flip_eval[i], flip_elem[i])
 * name evaluations at which one element's code is moved to the other neighbour
 * of its pre-round value (clamped to [0, qmax]); the `n_invert` evaluations in
 * invert_eval[] have their stop decision inverted.  With no flips and no
 * inversions this is the solver as written; the tests use them only to show
 * that a device result which left the oracle's trajectory did so at a rounding
 * tie or at a stop test between errors equal to rounding noise. */
int oracle_hqq_group_replay(const double* w, int g, int nbits, double p, double beta0,
                            double kappa, int iters, int early_stop, double err_pow,
                            uint8_t* codes_out, oracle_group_result_t* res, double* trace,
                            double* z_trace, int* n_trace, int n_flip, const int* flip_eval,
                            const int* flip_elem, int n_invert, const int* invert_eval) {
  if (g <= 0 || g > ORACLE_MAX_GROUP || nbits < 1 || nbits > 8 || iters < 0) return -1;
  int qmax = (1 << nbits) - 1;
  double q[ORACLE_MAX_GROUP], r[ORACLE_MAX_GROUP], we[ORACLE_MAX_GROUP], best_q[ORACLE_MAX_GROUP];
  double s, inv_s, z;
  oracle_minmax_init(w, g, qmax, &s, &inv_s, &z);
  double mn = w[0], mx = w[0]; /* the range again, for the exact first decision */
  for (int k = 1; k < g; ++k) {
    if (w[k] < mn) mn = w[k];
    if (w[k] > mx) mx = w[k];
  }

  double beta = beta0;
  double best_e = INFINITY, best_z = z, e0 = NAN;
  int t_star = 0, n_eval = 0;
  for (int t = 0; t <= iters; ++t) {
    /* W_q = Q(W) at the current z; residual r = W - Q^-1(W_q).  At t = 0 the value
     * w/s + z0 is an exact ratio and its code is decided exactly. */
    for (int k = 0; k < g; ++k)
      q[k] = t == 0 ? oracle_quantize_init_value(w[k], mn, mx, qmax)
                    : oracle_quantize_value(w[k], inv_s, z, qmax);
    for (int f = 0; f < n_flip; ++f) {
      if (flip_eval[f] != n_eval || flip_elem[f] < 0 || flip_elem[f] >= g) continue;
      int k = flip_elem[f];
      double x = w[k] * inv_s + z;
      double other = x > q[k] ? q[k] + 1.0 : q[k] - 1.0;
      if (other >= 0.0 && other <= (double)qmax) q[k] = other;
    }
    for (int k = 0; k < g; ++k) r[k] = w[k] - s * (q[k] - z);
    if (err_pow == 0.0) {
      /* The l0 error counts non-zero residuals.  Whether w/s + z equals its code is
       * decided like the code: exactly at t = 0 ((w - mn) qmax = q (mx - mn), both
       * sides exact in fp64), on the fp64 value afterwards.  The fp64 residual
       * itself would count the rounding noise of, e.g., the max element, whose
       * residual at t = 0 is exactly 0. */
      for (int k = 0; k < g; ++k) {
        const int zero_res = t == 0 ? (mx > mn ? (w[k] - mn) * (double)qmax == q[k] * (mx - mn)
                                               : 1)
                                    : w[k] * inv_s + z == q[k];
        if (zero_res) r[k] = 0.0;
      }
    }
    double e = oracle_group_error(r, g, err_pow);
    if (trace) trace[n_eval] = e;
    if (z_trace) z_trace[n_eval] = z;
    ++n_eval;
    if (t == 0) e0 = e;
    int improves = e < best_e;
    for (int f = 0; f < n_invert; ++f)
      if (invert_eval[f] == n_eval - 1 && n_eval > 1) improves = !improves;
    if (early_stop && !improves) break; /* error no longer improves */
    best_e = e;
    best_z = z;
    t_star = t;
    for (int k = 0; k < g; ++k) best_q[k] = q[k];
    if (t == iters) break;
    /* sp1: W_e = shrink(W - Q^-1(Q(W)), beta) */
    for (int k = 0; k < g; ++k) we[k] = oracle_shrink_lp(r[k], beta, p);
    /* sp2: closed-form mean */
    z = oracle_z_update(q, w, we, inv_s, g);
    beta = kappa * beta;
  }
  for (int k = 0; k < g; ++k) codes_out[k] = (uint8_t)best_q[k];
  res->scale = s;
  res->inv_scale = inv_s;
  res->zero = best_z;
  res->stop_step = t_star;
  res->err_init = e0;
  res->err_best = best_e;
  res->n_eval = n_eval;
  if (n_trace) *n_trace = n_eval;
  return 0;
}

int oracle_hqq_group(const double* w, int g, int nbits, double p, double beta0, double kappa,
                     int iters, int early_stop, double err_pow, uint8_t* codes_out,
                     oracle_group_result_t* res, double* trace, int* n_trace) {
  return oracle_hqq_group_replay(w, g, nbits, p, beta0, kappa, iters, early_stop, err_pow,
                                 codes_out, res, trace, NULL, n_trace, 0, NULL, NULL, 0, NULL);
}

/* ------------------------------------------------------------------------- */
/* Packed storage: LSB-first little-endian bitstream, element n occupies      */
/* bits [n*nbits, (n+1)*nbits) of the stream, bit i of a byte is 2^i.        */
/* ------------------------------------------------------------------------- */

int64_t oracle_packed_bytes(int64_t n, int nbits) { return (n * nbits + 7) / 8; }

void oracle_pack_codes(const uint8_t* codes, int64_t n, int nbits, uint8_t* out) {
  int64_t nbytes = oracle_packed_bytes(n, nbits);
  memset(out, 0, (size_t)nbytes);
  for (int64_t i = 0; i < n; ++i) {
    for (int b = 0; b < nbits; ++b) {
      if ((codes[i] >> b) & 1) {
        int64_t bit = i * nbits + b;
        out[bit >> 3] |= (uint8_t)(1u << (bit & 7));
      }
    }
  }
}

void oracle_unpack_codes(const uint8_t* packed, int64_t n, int nbits, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) {
    unsigned c = 0;
    for (int b = 0; b < nbits; ++b) {
      int64_t bit = i * nbits + b;
      c |= (unsigned)((packed[bit >> 3] >> (bit & 7)) & 1) << b;
    }
    codes[i] = (uint8_t)c;
  }
}

/* ------------------------------------------------------------------------- */
/* Whole matrix.                                                             */
/* ------------------------------------------------------------------------- */

int oracle_hqq_quantize(const uint16_t* W_f16, int64_t rows, int64_t cols, int nbits,
                        int group_size, double p, double beta, double kappa, int iters,
                        int early_stop, double err_pow, uint8_t* packed, uint16_t* scale_f16,
                        uint16_t* zero_f16, double* scale_f64, double* zero_f64,
                        uint8_t* stop_step, double* err_init, double* err_best,
                        uint8_t* codes_out) {
  if (rows < 0 || cols < 0 || group_size <= 0 || group_size > ORACLE_MAX_GROUP) return -1;
  if (cols % group_size != 0) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  int64_t n = rows * cols;
  int64_t ngroups = n / group_size;
  double w[ORACLE_MAX_GROUP];
  uint8_t gc[ORACLE_MAX_GROUP];
  uint8_t* codes = codes_out;
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    /* groups are contiguous along the row (input dimension); a row holds
     * cols/group_size of them, so the flat group index is row-major. */
    const uint16_t* src = W_f16 + gi * group_size;
    for (int k = 0; k < group_size; ++k) w[k] = oracle_f16_to_f64(src[k]);
    oracle_group_result_t res;
    if (oracle_hqq_group(w, group_size, nbits, p, beta, kappa, iters, early_stop, err_pow, gc,
                         &res, NULL, NULL) != 0)
      return -1;
    if (scale_f16) scale_f16[gi] = oracle_f64_to_f16(res.scale);
    if (zero_f16) zero_f16[gi] = oracle_f64_to_f16(res.zero);
    if (scale_f64) scale_f64[gi] = res.scale;
    if (zero_f64) zero_f64[gi] = res.zero;
    if (stop_step) stop_step[gi] = (uint8_t)res.stop_step;
    if (err_init) err_init[gi] = res.err_init;
    if (err_best) err_best[gi] = res.err_best;
    if (codes) memcpy(codes + gi * group_size, gc, (size_t)group_size);
    if (packed) {
      /* group_size * nbits is a multiple of 8 for every group size >= 8, so each
       * group owns whole bytes of the stream. */
      if ((group_size * nbits) % 8 == 0) {
        oracle_pack_codes(gc, group_size, nbits, packed + gi * group_size * nbits / 8);
      } else {
        return -1;
      }
    }
  }
  return 0;
}

/* Dequantization Q^-1(W_q) = s (W_q - z) from the stored binary16 s and z,
 * evaluated in fp64 (exact for binary16 operands and codes < 256) and rounded
 * once to binary16. */
int oracle_hqq_dequantize(const uint8_t* packed, const uint16_t* scale_f16,
                          const uint16_t* zero_f16, int64_t rows, int64_t cols, int nbits,
                          int group_size, uint16_t* W_out_f16) {
  if (rows < 0 || cols < 0 || group_size <= 0 || cols % group_size != 0) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  int64_t n = rows * cols;
  for (int64_t i = 0; i < n; ++i) {
    unsigned c = 0;
    for (int b = 0; b < nbits; ++b) {
      int64_t bit = i * nbits + b;
      c |= (unsigned)((packed[bit >> 3] >> (bit & 7)) & 1) << b;
    }
    int64_t gi = i / group_size;
    double s = oracle_f16_to_f64(scale_f16[gi]);
    double z = oracle_f16_to_f64(zero_f16[gi]);
    W_out_f16[i] = oracle_f64_to_f16(s * ((double)c - z));
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Meta quantization of the per-group s or z (section 4.1 and its table note): */
/* 8-bit affine min-max round-to-nearest, no solver.                          */
/* ------------------------------------------------------------------------- */

/* Groups of `group` consecutive values (group = 0: one group of all n; the last
 * group may be shorter).  Per group: mn, mx over the binary16 values; d = mx - mn;
 * if d > 0 the code of v is the half-even rounding of the exact ratio
 * ((v - mn) * 255) / d (v - mn and the product are exact in fp64, and
 * oracle_round_ratio decides without rounding) and the meta scale is d / 255; a
 * constant group has codes 0 and meta scale 1.  The meta scale is stored as binary16
 * (RNE from fp64), the offset mn exactly.  Returns the number of groups, or -1 for
 * invalid arguments. */
int64_t oracle_meta_quantize(const uint16_t* values, int64_t n, int64_t group, uint8_t* codes,
                             uint16_t* scale16, uint16_t* offset16) {
  if (n < 0 || group < 0) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  const int64_t gs = group == 0 ? n : group;
  int64_t ng = 0;
  for (int64_t g0 = 0; g0 < n; g0 += gs, ++ng) {
    const int64_t g1 = g0 + gs < n ? g0 + gs : n;
    double mn = oracle_f16_to_f64(values[g0]), mx = mn;
    for (int64_t i = g0 + 1; i < g1; ++i) {
      const double v = oracle_f16_to_f64(values[i]);
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    if (mn == 0.0) mn = 0.0;  /* a zero minimum is stored as +0 (the order of +-0 is not a min) */
    const double d = mx - mn;
    for (int64_t i = g0; i < g1; ++i) {
      double c = 0.0;
      if (d > 0.0) {
        c = oracle_round_ratio((oracle_f16_to_f64(values[i]) - mn) * 255.0, d);
        if (c < 0.0) c = 0.0;
        if (c > 255.0) c = 255.0;
      }
      codes[i] = (uint8_t)c;
    }
    scale16[ng] = oracle_f64_to_f16(d > 0.0 ? d / 255.0 : 1.0);
    offset16[ng] = oracle_f64_to_f16(mn);
  }
  return ng;
}

/* value = offset + scale * code from the stored binary16 meta scale and offset,
 * exact in fp64 (an 11-bit significand times an 8-bit integer, plus a binary16),
 * rounded once to binary16. */
int oracle_meta_dequantize(const uint8_t* codes, const uint16_t* scale16,
                           const uint16_t* offset16, int64_t n, int64_t group, uint16_t* out16) {
  if (n < 0 || group < 0) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  const int64_t gs = group == 0 ? (n > 0 ? n : 1) : group;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t gi = i / gs;
    out16[i] = oracle_f64_to_f16(oracle_f16_to_f64(offset16[gi]) +
                                 oracle_f16_to_f64(scale16[gi]) * (double)codes[i]);
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Whole-tensor early stop: the reading alternative to the per-group stop of   */
/* section 4.1 (the page says only that the solver exits once "the error" no   */
/* longer improves).                                                           */
/* ------------------------------------------------------------------------- */

/* All groups of the matrix step together.  E_t = sum over the groups (index
 * order) of e_{g,t}, the group's lp error (err_pow) at step t; the tensor continues
 * while E_t is strictly below the best total so far, and every group returns its z
 * of the last accepted step t*.  A stop decision never changes an update, so each
 * group's trajectory is that of the solver without early stop and the outputs are
 * those of oracle_hqq_quantize with early_stop = 0 and iters = t*.  E (may be NULL)
 * receives E_0 .. E_iters.  Returns t*, or -1 for invalid arguments. */
int oracle_hqq_quantize_tensor_stop(const uint16_t* W_f16, int64_t rows, int64_t cols, int nbits,
                                    int group_size, double p, double beta, double kappa,
                                    int iters, double err_pow, double* E, uint8_t* packed,
                                    uint16_t* scale_f16, uint16_t* zero_f16, double* scale_f64,
                                    double* zero_f64, uint8_t* stop_step, double* err_init,
                                    double* err_best, uint8_t* codes_out) {
  if (rows < 0 || cols < 0 || group_size <= 0 || group_size > ORACLE_MAX_GROUP) return -1;
  if (cols % group_size != 0 || iters < 0 || iters > 255) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  const int64_t ngroups = rows * cols / group_size;
  double total[256];
  for (int t = 0; t <= iters; ++t) total[t] = 0.0;
  double w[ORACLE_MAX_GROUP];
  uint8_t gc[ORACLE_MAX_GROUP];
  double trace[256];
  for (int64_t gi = 0; gi < ngroups; ++gi) {
    const uint16_t* src = W_f16 + gi * group_size;
    for (int k = 0; k < group_size; ++k) w[k] = oracle_f16_to_f64(src[k]);
    oracle_group_result_t res;
    int n_trace = 0;
    if (oracle_hqq_group(w, group_size, nbits, p, beta, kappa, iters, 0, err_pow, gc, &res,
                         trace, &n_trace) != 0 || n_trace != iters + 1)
      return -1;
    for (int t = 0; t <= iters; ++t) total[t] += trace[t];
  }
  int t_star = 0;
  double best = total[0];
  for (int t = 1; t <= iters; ++t) {
    if (!(total[t] < best)) break;
    best = total[t];
    t_star = t;
  }
  if (E)
    for (int t = 0; t <= iters; ++t) E[t] = total[t];
  if (oracle_hqq_quantize(W_f16, rows, cols, nbits, group_size, p, beta, kappa, t_star, 0, err_pow,
                          packed, scale_f16, zero_f16, scale_f64, zero_f64, stop_step, err_init,
                          err_best, codes_out) != 0)
    return -1;
  return t_star;
}

/* ------------------------------------------------------------------------- */
/* Product with the quantized weight, the consumer of the stored format:       */
/* y = x Q^-1(W_q)^T with the inverse quantizer Q^-1(W_q) = s (W_q - z) of     */
/* section 2, applied to the stored codes and binary16 s and z.               */
/* ------------------------------------------------------------------------- */

/* X: M x K binary16 activations, row-major.  The weight is N x K (row n holds the
 * weights of output n, grouped along K) as oracle_hqq_quantize stores it: packed
 * codes, binary16 s and z per group.  Y (M x N, fp64):
 *   Y[m][n] = sum over k of x[m][k] * s[n][k/g] * (q[n][k] - z[n][k/g]),
 * each term computed as (x*s) * (q - z) (x*s and q - z are exact in fp64, the
 * product is rounded once) and summed in index order.  Returns 0, or -1 for
 * invalid arguments. */
int oracle_hqq_matmul(const uint16_t* X_f16, int64_t M, int64_t K, const uint8_t* packed,
                      const uint16_t* scale_f16, const uint16_t* zero_f16, int64_t N, int nbits,
                      int group_size, double* Y) {
  if (M < 0 || K < 0 || N < 0 || group_size <= 0 || K % group_size != 0) return -1;
  if (nbits < 1 || nbits > 8) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  const int64_t gpr = K / group_size; /* groups per weight row */
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t elem = n * K + k; /* row-major element index of the weight */
        unsigned c = 0;
        for (int b = 0; b < nbits; ++b) {
          const int64_t bit = elem * nbits + b;
          c |= (unsigned)((packed[bit >> 3] >> (bit & 7)) & 1) << b;
        }
        const int64_t gi = n * gpr + k / group_size;
        const double x = oracle_f16_to_f64(X_f16[m * K + k]);
        const double s = oracle_f16_to_f64(scale_f16[gi]);
        const double z = oracle_f16_to_f64(zero_f16[gi]);
        acc += (x * s) * ((double)c - z);
      }
      Y[m * N + n] = acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------- */
/* The quantization error Delta W = W - Q^-1(W_q) that a low-rank correction   */
/* compensates (the plain SVD compensation on the EoRA page, section 1: the    */
/* LoRA factors B = U Sigma, A = V^T of the truncated SVD of Delta W).          */
/* ------------------------------------------------------------------------- */

/* dW[i] = w[i] - s (q[i] - z) in fp64 for the rows x cols binary16 weight W and its
 * stored codes and binary16 s, z (s (q - z) is exact in fp64, the difference is rounded
 * once).  Returns 0, or -1 for invalid arguments. */
int oracle_hqq_residual(const uint16_t* W_f16, const uint8_t* packed, const uint16_t* scale_f16,
                        const uint16_t* zero_f16, int64_t rows, int64_t cols, int nbits,
                        int group_size, double* dW) {
  if (rows < 0 || cols < 0 || group_size <= 0 || cols % group_size != 0) return -1;
  if (nbits < 1 || nbits > 8) return -1;
  if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
  const int64_t n = rows * cols;
  for (int64_t i = 0; i < n; ++i) {
    unsigned c = 0;
    for (int b = 0; b < nbits; ++b) {
      const int64_t bit = i * nbits + b;
      c |= (unsigned)((packed[bit >> 3] >> (bit & 7)) & 1) << b;
    }
    const int64_t gi = i / group_size;
    const double s = oracle_f16_to_f64(scale_f16[gi]);
    const double z = oracle_f16_to_f64(zero_f16[gi]);
    dW[i] = oracle_f16_to_f64(W_f16[i]) - s * ((double)c - z);
  }
  return 0;
}
