/*
 * spectre_oracle.c -- reference (oracle) implementation of the SPECTRE
 * spectral mix, in plain C and double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * definition that the GPU library is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * library never links, calls or includes anything from here, and this file
 * includes nothing from the product.
 *
 * What it computes (SPECTRE FFT-attention article, hotelren.com/news/5925787,
 * section 2.2 "frequency-domain kernel replaces the attention matrix", its
 * pseudocode, and section 2.3 "frequency truncation"):
 *
 *   for every column (b, h, d) of q, k, v laid out [B, L, H, D]:
 *     Q[f] = sum_n q[n] exp(-2 pi i f n / L)          (same for K, V)
 *     O[f] = (G[h][f] / L) * Q[f] * conj(K[f]) * V[f]  for f < keep_bins, else 0
 *     y    = inverse real FFT of O (length L, 1/L normalisation)
 *   out[b, t, :] = LayerNorm over the H*D channels of (x[b, t, :] + y[b, t, :])
 *
 * Readings taken where the article is silent (each also listed in the design
 * notes): the transform runs along the sequence axis and is real-to-complex
 * (section 2.2 speaks of a real FFT, section 3.3 of irfft); forward unscaled,
 * inverse scaled by 1/L, plus the explicit 1/L of the mix; the gate is a real
 * multiplier per (head, bin); truncation keeps bins f < keep_bins of the
 * half spectrum f = 0 .. floor(L/2); the imaginary parts of the DC and (for
 * even L) Nyquist bins are dropped, as an inverse real FFT does; the norm is
 * a LayerNorm over H*D with biased variance and eps = 1e-5 applied after the
 * residual add (section 2.2's ordering).
 *
 * Algorithm: for each column, the three forward transforms and the inverse
 * are computed with this file's own recursive mixed-radix decimation-in-time
 * FFT (radix 4, 2 and 3 butterflies, plus a direct O(p^2) DFT step for any
 * other prime factor p), so every length L >= 1 is supported.  Twiddles are
 * cos/sin of 2*pi*j/N with the integer exponent reduced modulo N first.
 * Columns are spread over POSIX threads; each column is independent until the
 * LayerNorm, which then runs per token.
 *
 * Storage types: dtype 0 = IEEE binary32, dtype 1 = bfloat16 (the upper 16
 * bits of a binary32; decoded exactly by shifting left 16).  All arithmetic
 * is double.
 *
 * Variants (the *_ex entry points; the plain ones are gate kind 0, post-norm):
 *  - gate kind 0: G[h][f] is the real multiplier itself;
 *    gate kind 1: G[h][f] is a logit and the multiplier is the logistic
 *    sigmoid 1 / (1 + exp(-G)) (section 3.1 recommends a sigmoid gate);
 *    gate kind 2: the gate array is [H][L/2 + 1][2], the real and imaginary
 *    parts of a complex multiplier (section 2.4 carries relative position as
 *    a frequency-dependent rotation inside G(f)).  The bins above L/2 take
 *    the conjugate through the Hermitian extension, and an inverse real FFT
 *    ignores the imaginary part of bins 0 and L/2, so only the real part of
 *    the gate acts there.
 *  - norm order 0 (post-norm, section 2.2's pseudocode): out = LN(x + y);
 *    norm order 1 (pre-norm, the order section 3.3 settles on): out =
 *    x + LN(y), the same LayerNorm applied to y alone.  Adding 2 to either
 *    order uses an RMSNorm instead (section 3.3 names "RMSNorm or
 *    LayerNorm"): z / sqrt(mean(z^2) + eps) * gamma + beta over the H*D
 *    channels -- no mean is subtracted; beta = 0 gives the textbook form.
 *
 * Chunked mix (oracle_spectre_mix_chunked; section 3.2's fft_len below L:
 * an FFT inside 4096-token blocks, then one more low-frequency interaction
 * between blocks, whose form the article leaves open).  Reading: the
 * sequence is cut into nb = L / F blocks of F tokens and each block is mixed
 * on its own (gate [H][F/2 + 1], keep_bins); then the block means of q, k, v
 * (per column, nb values each) are mixed by the same operation over the
 * block axis (gate_blocks [H][nb/2 + 1], keep_blocks), and that result is
 * added to every token of its block; then the residual and the LayerNorm.
 *
 * Local branch (oracle_local_attention, oracle_spectre_mix_local; section
 * 3.2's use_local_branch and section 4.3: a sliding-window attention branch
 * beside the FFT branch, window 128 to 256, the two outputs added).
 * Reading: for token t of head h, the keys j with t - win_left <= j <= t +
 * win_right and 0 <= j < L; scores (q_t . k_j) / sqrt(D); softmax over those
 * keys; y_loc[t] = sum_j p_j v_j.  out = LN(x + y + y_loc);
 * oracle_spectre_mix_local_ex takes the gate kinds and norm orders above
 * (pre-norm: out = x + LN(y + y_loc)).  Section 4.3 has the two branches
 * "summed or gated"; oracle_spectre_mix_local_gated reads the gated form as
 * a per-channel weight g in [0, 1] given by the caller (the sigmoid that
 * would produce it is upstream, as for the gate): the branch sum becomes
 * g * y + (1 - g) * y_loc, channel by channel, before the residual and the
 * norm (g = 1: the FFT branch alone; g = 0: the local branch alone).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-3)
#define ORACLE_EIMAG (-5) /* inverse transform left a large imaginary part */

typedef struct {
  double re, im;
} cpx;

static inline cpx cmul(cpx a, cpx b) {
  cpx r = {a.re * b.re - a.im * b.im, a.re * b.im + a.im * b.re};
  return r;
}
static inline cpx cadd(cpx a, cpx b) {
  cpx r = {a.re + b.re, a.im + b.im};
  return r;
}
static inline cpx csub(cpx a, cpx b) {
  cpx r = {a.re - b.re, a.im - b.im};
  return r;
}
static inline cpx cscale(cpx a, double s) {
  cpx r = {a.re * s, a.im * s};
  return r;
}
static inline cpx cconj(cpx a) {
  cpx r = {a.re, -a.im};
  return r;
}

/* ------------------------------------------------------------------------ */
/* Mixed-radix complex FFT                                                   */
/* ------------------------------------------------------------------------ */

/* Twiddle table for one top-level length N: w[j] = exp(-2 pi i j / N). */
typedef struct {
  int64_t n;
  cpx *w;
} fft_table;

static int table_init(fft_table *t, int64_t n) {
  t->n = n;
  t->w = (cpx *)malloc(sizeof(cpx) * (size_t)(n > 0 ? n : 1));
  if (!t->w) return ORACLE_ENOMEM;
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t j = 0; j < n; ++j) {
    double a = two_pi * (double)j / (double)n;
    t->w[j].re = cos(a);
    t->w[j].im = -sin(a);
  }
  return ORACLE_OK;
}

static void table_free(fft_table *t) {
  free(t->w);
  t->w = NULL;
}

/* exp(sign * 2 pi i e / n) for a sub-transform of length n dividing t->n. */
static inline cpx twiddle(const fft_table *t, int64_t n, int64_t e, int sign) {
  int64_t j = (e % n) * (t->n / n);
  cpx w = t->w[j];
  return sign > 0 ? cconj(w) : w;
}

static int64_t smallest_factor(int64_t n) {
  if (n % 4 == 0) return 4;
  if (n % 2 == 0) return 2;
  if (n % 3 == 0) return 3;
  for (int64_t p = 5; p * p <= n; p += 2)
    if (n % p == 0) return p;
  return n;
}

/*
 * Decimation in time: the n inputs in[0], in[is], in[2 is], ... split into p
 * interleaved subsequences (r = 0 .. p-1, stride p*is); each gets an
 * (n/p)-point transform written to out[r*m .. r*m + m); then for every k the
 * p partial results are combined:
 *   X[k + s*m] = sum_r exp(sign 2 pi i r (k + s m) / n) * Y_r[k].
 * `scratch` holds at least 2*p complex values per recursion level.
 */
static void fft_rec(const fft_table *t, const cpx *in, int64_t is, cpx *out,
                    int64_t n, int sign, cpx *scratch) {
  if (n == 1) {
    out[0] = in[0];
    return;
  }
  int64_t p = smallest_factor(n);
  int64_t m = n / p;
  for (int64_t r = 0; r < p; ++r)
    fft_rec(t, in + r * is, is * p, out + r * m, m, sign, scratch + 2 * p);

  cpx *y = scratch; /* p twiddled partial results for one k */
  for (int64_t k = 0; k < m; ++k) {
    for (int64_t r = 0; r < p; ++r)
      y[r] = r == 0 ? out[k] : cmul(out[r * m + k], twiddle(t, n, r * k, sign));
    if (p == 2) {
      out[k] = cadd(y[0], y[1]);
      out[k + m] = csub(y[0], y[1]);
    } else if (p == 4) {
      /* 4-point DFT: outputs s = 0..3 of sum_r y[r] exp(sign 2 pi i r s / 4) */
      cpx a0 = cadd(y[0], y[2]), a1 = csub(y[0], y[2]);
      cpx b0 = cadd(y[1], y[3]), b1 = csub(y[1], y[3]);
      /* multiply b1 by exp(sign * i pi / 2) = sign * i */
      cpx jb1 = sign > 0 ? (cpx){-b1.im, b1.re} : (cpx){b1.im, -b1.re};
      out[k] = cadd(a0, b0);
      out[k + m] = cadd(a1, jb1);
      out[k + 2 * m] = csub(a0, b0);
      out[k + 3 * m] = csub(a1, jb1);
    } else if (p == 3) {
      /* 3-point DFT with w = exp(sign 2 pi i / 3) = -1/2 + sign i sqrt(3)/2 */
      const double s3 = 0.86602540378443864676372317075294;
      cpx sum = cadd(y[1], y[2]), dif = csub(y[1], y[2]);
      cpx mid = {y[0].re - 0.5 * sum.re, y[0].im - 0.5 * sum.im};
      /* sign * i * sqrt(3)/2 * dif */
      cpx rot = {-(double)sign * s3 * dif.im, (double)sign * s3 * dif.re};
      out[k] = cadd(y[0], sum);
      out[k + m] = cadd(mid, rot);
      out[k + 2 * m] = csub(mid, rot);
    } else {
      /* any other prime: the DFT of the p values by its definition */
      cpx *z = scratch + p;
      for (int64_t s = 0; s < p; ++s) {
        cpx acc = {0.0, 0.0};
        for (int64_t r = 0; r < p; ++r)
          acc = cadd(acc, cmul(y[r], twiddle(t, p, r * s, sign)));
        z[s] = acc;
      }
      for (int64_t s = 0; s < p; ++s) out[k + s * m] = z[s];
    }
  }
}

/* Largest radix used anywhere in the recursion for length n. */
static int64_t largest_factor(int64_t n) {
  int64_t big = 1;
  while (n > 1) {
    int64_t p = smallest_factor(n);
    if (p > big) big = p;
    n /= p;
  }
  return big;
}

static int64_t depth_of(int64_t n) {
  int64_t d = 0;
  while (n > 1) {
    n /= smallest_factor(n);
    ++d;
  }
  return d;
}

/* Scratch size (complex values) for one transform of length n. */
static int64_t scratch_len(int64_t n) {
  return 2 * largest_factor(n) * (depth_of(n) + 1) + 2;
}

/*
 * Unnormalised complex DFT of length n: out[f] = sum_j in[j] exp(sign 2 pi i f j / n),
 * sign = -1 (forward) or +1 (inverse, no scaling).
 */
static int fft(const fft_table *t, const cpx *in, cpx *out, int sign, cpx *scratch) {
  fft_rec(t, in, 1, out, t->n, sign, scratch);
  return ORACLE_OK;
}

int oracle_fft(int64_t n, const double *re_in, const double *im_in, double *re_out,
               double *im_out, int sign) {
  if (n < 1 || !re_in || !re_out || !im_out || (sign != 1 && sign != -1))
    return ORACLE_EINVAL;
  fft_table t;
  if (table_init(&t, n)) return ORACLE_ENOMEM;
  cpx *a = (cpx *)malloc(sizeof(cpx) * (size_t)n);
  cpx *b = (cpx *)malloc(sizeof(cpx) * (size_t)n);
  cpx *s = (cpx *)malloc(sizeof(cpx) * (size_t)scratch_len(n));
  if (!a || !b || !s) {
    free(a);
    free(b);
    free(s);
    table_free(&t);
    return ORACLE_ENOMEM;
  }
  for (int64_t j = 0; j < n; ++j) {
    a[j].re = re_in[j];
    a[j].im = im_in ? im_in[j] : 0.0;
  }
  fft(&t, a, b, sign, s);
  for (int64_t j = 0; j < n; ++j) {
    re_out[j] = b[j].re;
    im_out[j] = b[j].im;
  }
  free(a);
  free(b);
  free(s);
  table_free(&t);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Storage decoding                                                          */
/* ------------------------------------------------------------------------ */

static inline double load_elem(const void *base, int dtype, int64_t i) {
  if (dtype == 0) return (double)((const float *)base)[i];
  if (dtype == 2) return ((const double *)base)[i]; /* internal: the chunked mix's block means */
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* The spectral mix, one column at a time                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  const void *q, *k, *v;
  const float *gate;
  int64_t B, H, L, D, keep;
  int dtype;
  int gate_kind; /* 0 real, 1 logit (sigmoid), 2 complex (re, im pairs) */
  const fft_table *tab;
  /* output: either the full y [B, L, H*D] or sampled tokens */
  double *y;             /* full output, or NULL */
  const int64_t *tokens; /* sampled flat token ids b*L + t, or NULL */
  int64_t ntok;
  double *y_tok; /* [ntok, H*D] when tokens != NULL */
  int64_t next;  /* shared column counter */
  int status;
  double max_imag_ratio;
  pthread_mutex_t mu;
} mix_job;

/* The gate multiplier of head h at half-spectrum bin f (see the variants in
 * the header). */
static cpx gate_at(const mix_job *J, int64_t h, int64_t f, int64_t nbins) {
  cpx g = {0.0, 0.0};
  if (J->gate_kind == 2) {
    g.re = (double)J->gate[2 * (h * nbins + f)];
    g.im = (double)J->gate[2 * (h * nbins + f) + 1];
  } else {
    double a = (double)J->gate[h * nbins + f];
    g.re = J->gate_kind == 1 ? 1.0 / (1.0 + exp(-a)) : a;
  }
  return g;
}

/* y for one column (b, c): fills ycol[0..L). Returns the largest |Im| seen
 * after the inverse transform, relative to max |Re| (a self-check). */
static double mix_column(const mix_job *J, int64_t b, int64_t c, cpx *bufq, cpx *bufk,
                         cpx *bufv, cpx *tmp, cpx *scr, double *ycol) {
  const int64_t L = J->L, C = J->H * J->D;
  const int64_t h = c / J->D;
  const int64_t base = b * L * C + c;
  const int64_t half = L / 2; /* bins f = 0 .. half */

  /* Q, K, V: forward transforms of the real columns (imaginary part zero). */
  for (int64_t n = 0; n < L; ++n) {
    tmp[n].re = load_elem(J->q, J->dtype, base + n * C);
    tmp[n].im = 0.0;
  }
  fft(J->tab, tmp, bufq, -1, scr);
  for (int64_t n = 0; n < L; ++n) {
    tmp[n].re = load_elem(J->k, J->dtype, base + n * C);
    tmp[n].im = 0.0;
  }
  fft(J->tab, tmp, bufk, -1, scr);
  for (int64_t n = 0; n < L; ++n) {
    tmp[n].re = load_elem(J->v, J->dtype, base + n * C);
    tmp[n].im = 0.0;
  }
  fft(J->tab, tmp, bufv, -1, scr);

  /* O[f] = (G[h][f] / L) Q[f] conj(K[f]) V[f] on the half spectrum, zero at
   * f >= keep; then the Hermitian extension fills the other half. */
  const double invL = 1.0 / (double)L;
  const int64_t nbins = half + 1;
  for (int64_t f = 0; f <= half; ++f) {
    cpx o = {0.0, 0.0};
    if (f < J->keep) {
      cpx g = gate_at(J, h, f, nbins);
      o = cscale(cmul(cmul(cmul(bufq[f], cconj(bufk[f])), bufv[f]), g), invL);
    }
    if (f == 0 || (L % 2 == 0 && f == half)) o.im = 0.0;
    tmp[f] = o;
  }
  for (int64_t f = half + 1; f < L; ++f) tmp[f] = cconj(tmp[L - f]);

  /* Inverse transform, 1/L normalisation, real part. */
  fft(J->tab, tmp, bufq, +1, scr);
  double max_re = 0.0, max_im = 0.0;
  for (int64_t t = 0; t < L; ++t) {
    double re = bufq[t].re * invL, im = bufq[t].im * invL;
    ycol[t] = re;
    if (fabs(re) > max_re) max_re = fabs(re);
    if (fabs(im) > max_im) max_im = fabs(im);
  }
  return max_re > 0.0 ? max_im / max_re : max_im;
}

static void *mix_worker(void *arg) {
  mix_job *J = (mix_job *)arg;
  const int64_t L = J->L, C = J->H * J->D, ncol = J->B * C;
  cpx *bq = (cpx *)malloc(sizeof(cpx) * (size_t)L);
  cpx *bk = (cpx *)malloc(sizeof(cpx) * (size_t)L);
  cpx *bv = (cpx *)malloc(sizeof(cpx) * (size_t)L);
  cpx *tmp = (cpx *)malloc(sizeof(cpx) * (size_t)L);
  cpx *scr = (cpx *)malloc(sizeof(cpx) * (size_t)scratch_len(L));
  double *ycol = (double *)malloc(sizeof(double) * (size_t)L);
  double worst = 0.0;
  if (!bq || !bk || !bv || !tmp || !scr || !ycol) {
    pthread_mutex_lock(&J->mu);
    J->status = ORACLE_ENOMEM;
    pthread_mutex_unlock(&J->mu);
  } else {
    for (;;) {
      int64_t col = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
      if (col >= ncol) break;
      int64_t b = col / C, c = col % C;
      double r = mix_column(J, b, c, bq, bk, bv, tmp, scr, ycol);
      if (r > worst) worst = r;
      if (J->y) {
        double *dst = J->y + b * L * C + c;
        for (int64_t t = 0; t < L; ++t) dst[t * C] = ycol[t];
      } else {
        for (int64_t i = 0; i < J->ntok; ++i) {
          int64_t tok = J->tokens[i];
          if (tok / L == b) J->y_tok[i * C + c] = ycol[tok % L];
        }
      }
    }
  }
  pthread_mutex_lock(&J->mu);
  if (worst > J->max_imag_ratio) J->max_imag_ratio = worst;
  pthread_mutex_unlock(&J->mu);
  free(bq);
  free(bk);
  free(bv);
  free(tmp);
  free(scr);
  free(ycol);
  return NULL;
}

static int resolve_threads(int nthreads) {
  if (nthreads > 0) return nthreads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static int run_mix(mix_job *J, int nthreads) {
  fft_table tab;
  if (table_init(&tab, J->L)) return ORACLE_ENOMEM;
  J->tab = &tab;
  J->next = 0;
  J->status = ORACLE_OK;
  J->max_imag_ratio = 0.0;
  pthread_mutex_init(&J->mu, NULL);
  nthreads = resolve_threads(nthreads);
  int64_t ncol = J->B * J->H * J->D;
  if (nthreads > ncol) nthreads = (int)ncol;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  if (!th) {
    table_free(&tab);
    return ORACLE_ENOMEM;
  }
  int started = 0;
  for (int i = 0; i < nthreads; ++i)
    if (pthread_create(&th[i], NULL, mix_worker, J) == 0) ++started;
  if (started == 0) mix_worker(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J->mu);
  table_free(&tab);
  if (J->status) return J->status;
  /* An inverse real FFT of a Hermitian spectrum is real: anything above
   * rounding level means the Hermitian extension is wrong. */
  if (J->max_imag_ratio > 1e-9) return ORACLE_EIMAG;
  return ORACLE_OK;
}

static int check_dims(int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep, int dtype) {
  if (B < 1 || H < 1 || L < 1 || D < 1) return ORACLE_EINVAL;
  if (keep < 0 || keep > L / 2 + 1) return ORACLE_EINVAL;
  if (dtype != 0 && dtype != 1) return ORACLE_EINVAL;
  return ORACLE_OK;
}

static int check_variant(int gate_kind, int norm_order) {
  if (gate_kind < 0 || gate_kind > 2 || norm_order < 0 || norm_order > 3) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/* y[b, t, h*D + d] for every token, double. */
int oracle_spectre_y_ex(const void *q, const void *k, const void *v, const float *gate,
                        int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep, int dtype,
                        int gate_kind, double *y, int nthreads) {
  if (!q || !k || !v || !gate || !y) return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, keep, dtype);
  if (!s) s = check_variant(gate_kind, 0);
  if (s) return s;
  mix_job J;
  memset(&J, 0, sizeof J);
  J.q = q;
  J.k = k;
  J.v = v;
  J.gate = gate;
  J.B = B;
  J.H = H;
  J.L = L;
  J.D = D;
  J.keep = keep;
  J.dtype = dtype;
  J.gate_kind = gate_kind;
  J.y = y;
  return run_mix(&J, nthreads);
}

int oracle_spectre_y(const void *q, const void *k, const void *v, const float *gate,
                     int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep, int dtype,
                     double *y, int nthreads) {
  return oracle_spectre_y_ex(q, k, v, gate, B, H, L, D, keep, dtype, 0, y, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Residual + LayerNorm over the H*D channels of each token                  */
/* ------------------------------------------------------------------------ */

/*
 * Post-norm (pre = 0): out[i, c] = (z - mean) / sqrt(var + 1e-5) * gamma[c] +
 * beta[c], with z = x[xrow_i, c] + y[i, c], mean and biased variance over c
 * (two passes).  Pre-norm (pre = 1): z = y[i, c], and x[xrow_i, c] is added
 * after the affine step.  xrow[i] selects the row of x for row i of y (NULL:
 * row i).
 */
/* The norm and the residual, token by token.  norm_order: bit 0 pre-norm
 * (out = x + N(y)) instead of post-norm (out = N(x + y)); bit 1 RMSNorm
 * (nothing subtracted, the mean square in place of the variance) instead of
 * LayerNorm. */
static void layernorm_rows(const double *y, const void *x, int dtype, const int64_t *xrow,
                           const float *gamma, const float *beta, int64_t nrows, int64_t C,
                           int norm_order, double *out) {
  const double eps = 1e-5;
  const int pre = norm_order & 1, rms = (norm_order & 2) != 0;
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t xr = xrow ? xrow[i] : i;
    const double *yr = y + i * C;
    double *o = out + i * C;
    double sum = 0.0;
    for (int64_t c = 0; c < C; ++c) {
      o[c] = pre ? yr[c] : load_elem(x, dtype, xr * C + c) + yr[c];
      sum += o[c];
    }
    double mean = rms ? 0.0 : sum / (double)C;
    double var = 0.0;
    for (int64_t c = 0; c < C; ++c) var += (o[c] - mean) * (o[c] - mean);
    var /= (double)C;
    double rstd = 1.0 / sqrt(var + eps);
    for (int64_t c = 0; c < C; ++c) {
      o[c] = (o[c] - mean) * rstd * (double)gamma[c] + (double)beta[c];
      if (pre) o[c] += load_elem(x, dtype, xr * C + c);
    }
  }
}

int oracle_layernorm_residual_ex(const double *y, const void *x, const float *gamma,
                                 const float *beta, int64_t ntok, int64_t C, int dtype,
                                 int norm_order, double *out) {
  if (!y || !x || !gamma || !beta || !out || ntok < 0 || C < 1) return ORACLE_EINVAL;
  if (dtype != 0 && dtype != 1) return ORACLE_EINVAL;
  if (check_variant(0, norm_order)) return ORACLE_EINVAL;
  layernorm_rows(y, x, dtype, NULL, gamma, beta, ntok, C, norm_order, out);
  return ORACLE_OK;
}

int oracle_layernorm_residual(const double *y, const void *x, const float *gamma,
                              const float *beta, int64_t ntok, int64_t C, int dtype,
                              double *out) {
  return oracle_layernorm_residual_ex(y, x, gamma, beta, ntok, C, dtype, 0, out);
}

/* The whole mix: out (and optionally y) for every token, double. */
int oracle_spectre_mix_ex(const void *q, const void *k, const void *v, const void *x,
                          const float *gate, const float *gamma, const float *beta, int64_t B,
                          int64_t H, int64_t L, int64_t D, int64_t keep, int dtype,
                          int gate_kind, int norm_order, double *out, double *y_out,
                          int nthreads) {
  if (!x || !gamma || !beta || !out) return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, keep, dtype);
  if (!s) s = check_variant(gate_kind, norm_order);
  if (s) return s;
  const int64_t C = H * D, ntok = B * L;
  double *y = y_out ? y_out : (double *)malloc(sizeof(double) * (size_t)(ntok * C));
  if (!y) return ORACLE_ENOMEM;
  s = oracle_spectre_y_ex(q, k, v, gate, B, H, L, D, keep, dtype, gate_kind, y, nthreads);
  if (s == ORACLE_OK) layernorm_rows(y, x, dtype, NULL, gamma, beta, ntok, C, norm_order, out);
  if (!y_out) free(y);
  return s;
}

int oracle_spectre_mix(const void *q, const void *k, const void *v, const void *x,
                       const float *gate, const float *gamma, const float *beta, int64_t B,
                       int64_t H, int64_t L, int64_t D, int64_t keep, int dtype, double *out,
                       double *y_out, int nthreads) {
  return oracle_spectre_mix_ex(q, k, v, x, gate, gamma, beta, B, H, L, D, keep, dtype, 0, 0,
                               out, y_out, nthreads);
}

/*
 * The mix at a sample of tokens only (flat ids b*L + t): every column is still
 * transformed in full, but only the sampled positions of y are kept, so memory
 * stays O(ntok * H * D) at any L.  out_tok and y_tok (optional) are
 * [ntok, H*D].
 */
int oracle_spectre_mix_tokens_ex(const void *q, const void *k, const void *v, const void *x,
                                 const float *gate, const float *gamma, const float *beta,
                                 int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep,
                                 int dtype, int gate_kind, int norm_order,
                                 const int64_t *tokens, int64_t ntok, double *out_tok,
                                 double *y_tok, int nthreads) {
  if (!q || !k || !v || !x || !gate || !gamma || !beta || !tokens || !out_tok || ntok < 1)
    return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, keep, dtype);
  if (!s) s = check_variant(gate_kind, norm_order);
  if (s) return s;
  for (int64_t i = 0; i < ntok; ++i)
    if (tokens[i] < 0 || tokens[i] >= B * L) return ORACLE_EINVAL;
  const int64_t C = H * D;
  double *y = y_tok ? y_tok : (double *)malloc(sizeof(double) * (size_t)(ntok * C));
  if (!y) return ORACLE_ENOMEM;
  mix_job J;
  memset(&J, 0, sizeof J);
  J.q = q;
  J.k = k;
  J.v = v;
  J.gate = gate;
  J.B = B;
  J.H = H;
  J.L = L;
  J.D = D;
  J.keep = keep;
  J.dtype = dtype;
  J.gate_kind = gate_kind;
  J.tokens = tokens;
  J.ntok = ntok;
  J.y_tok = y;
  s = run_mix(&J, nthreads);
  if (s == ORACLE_OK)
    layernorm_rows(y, x, dtype, tokens, gamma, beta, ntok, C, norm_order, out_tok);
  if (!y_tok) free(y);
  return s;
}

int oracle_spectre_mix_tokens(const void *q, const void *k, const void *v, const void *x,
                              const float *gate, const float *gamma, const float *beta,
                              int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep,
                              int dtype, const int64_t *tokens, int64_t ntok,
                              double *out_tok, double *y_tok, int nthreads) {
  return oracle_spectre_mix_tokens_ex(q, k, v, x, gate, gamma, beta, B, H, L, D, keep, dtype,
                                      0, 0, tokens, ntok, out_tok, y_tok, nthreads);
}

/* The chunked mix (see the header): out and optionally y, for every token. */
int oracle_spectre_mix_chunked(const void *q, const void *k, const void *v, const void *x,
                               const float *gate, const float *gate_blocks, const float *gamma,
                               const float *beta, int64_t B, int64_t H, int64_t L, int64_t D,
                               int64_t F, int64_t keep, int64_t keep_blocks, int dtype,
                               double *out, double *y_out, int nthreads) {
  if (!q || !k || !v || !x || !gate || !gate_blocks || !gamma || !beta || !out)
    return ORACLE_EINVAL;
  if (F < 1 || L < 1 || L % F != 0) return ORACLE_EINVAL;
  const int64_t nb = L / F;
  int s = check_dims(B, H, L, D, 0, dtype);
  if (!s) s = check_dims(B * nb, H, F, D, keep, dtype);
  if (!s && (keep_blocks < 0 || keep_blocks > nb / 2 + 1)) s = ORACLE_EINVAL;
  if (s) return s;
  const int64_t C = H * D, ntok = B * L;
  double *y = y_out ? y_out : (double *)malloc(sizeof(double) * (size_t)(ntok * C));
  double *means = (double *)malloc(sizeof(double) * (size_t)(3 * B * nb * C));
  double *y2 = (double *)malloc(sizeof(double) * (size_t)(B * nb * C));
  if (!y || !means || !y2) {
    if (!y_out) free(y);
    free(means);
    free(y2);
    return ORACLE_ENOMEM;
  }
  /* each block on its own: [B, L, H, D] read as [B * nb, F, H, D] */
  s = oracle_spectre_y_ex(q, k, v, gate, B * nb, H, F, D, keep, dtype, 0, y, nthreads);
  if (s == ORACLE_OK) {
    /* block means of q, k, v: [3][B][nb][C] */
    const void *src[3] = {q, k, v};
    for (int a = 0; a < 3; ++a)
      for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < nb; ++j)
          for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t t = 0; t < F; ++t)
              acc += load_elem(src[a], dtype, (b * L + j * F + t) * C + c);
            means[((a * B + b) * nb + j) * C + c] = acc / (double)F;
          }
    /* the same mix over the block axis, on the double block means */
    mix_job J;
    memset(&J, 0, sizeof J);
    J.q = means;
    J.k = means + B * nb * C;
    J.v = means + 2 * B * nb * C;
    J.gate = gate_blocks;
    J.B = B;
    J.H = H;
    J.L = nb;
    J.D = D;
    J.keep = keep_blocks;
    J.dtype = 2;
    J.y = y2;
    s = run_mix(&J, nthreads);
  }
  if (s == ORACLE_OK) {
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < L; ++t)
        for (int64_t c = 0; c < C; ++c) y[(b * L + t) * C + c] += y2[(b * nb + t / F) * C + c];
    layernorm_rows(y, x, dtype, NULL, gamma, beta, ntok, C, 0, out);
  }
  if (!y_out) free(y);
  free(means);
  free(y2);
  return s;
}

/* One query of the local branch: token t of batch b, head h -- softmax of the
 * scores (q_t . k_j) / sqrt(D) over the keys j in t - win_left .. t + win_right
 * inside the sequence, times v; the D values go to yq.  sc holds
 * win_left + win_right + 1 doubles of scratch. */
static void local_query(const void *q, const void *k, const void *v, int64_t B, int64_t H,
                        int64_t L, int64_t D, int64_t win_left, int64_t win_right, int dtype,
                        int64_t b, int64_t h, int64_t t, double *sc, double *yq) {
  (void)B;
  const int64_t C = H * D;
  const double scale = 1.0 / sqrt((double)D);
  const int64_t j0 = t - win_left < 0 ? 0 : t - win_left;
  const int64_t j1 = t + win_right > L - 1 ? L - 1 : t + win_right;
  const int64_t qb = (b * L + t) * C + h * D;
  double mx = -INFINITY;
  for (int64_t j = j0; j <= j1; ++j) {
    const int64_t kb = (b * L + j) * C + h * D;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += load_elem(q, dtype, qb + d) * load_elem(k, dtype, kb + d);
    sc[j - j0] = dot * scale;
    if (sc[j - j0] > mx) mx = sc[j - j0];
  }
  double sum = 0.0;
  for (int64_t j = j0; j <= j1; ++j) {
    sc[j - j0] = exp(sc[j - j0] - mx);
    sum += sc[j - j0];
  }
  for (int64_t d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int64_t j = j0; j <= j1; ++j) acc += sc[j - j0] * load_elem(v, dtype, (b * L + j) * C + h * D + d);
    yq[d] = acc / sum;
  }
}

/* The local branch alone: y_loc [B, L, H, D], double (see the header). */
int oracle_local_attention(const void *q, const void *k, const void *v, int64_t B, int64_t H,
                           int64_t L, int64_t D, int64_t win_left, int64_t win_right, int dtype,
                           double *y) {
  if (!q || !k || !v || !y) return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, 0, dtype);
  if (s) return s;
  if (win_left < 0 || win_right < 0) return ORACLE_EINVAL;
  const int64_t C = H * D;
  double *sc = (double *)malloc(sizeof(double) * (size_t)(win_left + win_right + 1));
  if (!sc) return ORACLE_ENOMEM;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t t = 0; t < L; ++t)
        local_query(q, k, v, B, H, L, D, win_left, win_right, dtype, b, h, t, sc,
                    y + (b * L + t) * C + h * D);
  free(sc);
  return ORACLE_OK;
}

/* The local branch at listed tokens only: tokens[i] = b * L + t, and row i
 * of y_tok [ntok, H, D] gets y_loc of that token (the same per-query
 * arithmetic as oracle_local_attention). */
int oracle_local_attention_tokens(const void *q, const void *k, const void *v, int64_t B,
                                  int64_t H, int64_t L, int64_t D, int64_t win_left,
                                  int64_t win_right, int dtype, const int64_t *tokens, int64_t ntok,
                                  double *y_tok) {
  if (!q || !k || !v || !tokens || !y_tok || ntok < 1) return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, 0, dtype);
  if (s) return s;
  if (win_left < 0 || win_right < 0) return ORACLE_EINVAL;
  for (int64_t i = 0; i < ntok; ++i)
    if (tokens[i] < 0 || tokens[i] >= B * L) return ORACLE_EINVAL;
  const int64_t C = H * D;
  double *sc = (double *)malloc(sizeof(double) * (size_t)(win_left + win_right + 1));
  if (!sc) return ORACLE_ENOMEM;
  for (int64_t i = 0; i < ntok; ++i)
    for (int64_t h = 0; h < H; ++h)
      local_query(q, k, v, B, H, L, D, win_left, win_right, dtype, tokens[i] / L, h,
                  tokens[i] % L, sc, y_tok + i * C + h * D);
  free(sc);
  return ORACLE_OK;
}

int oracle_spectre_mix_local_gated(const void *q, const void *k, const void *v, const void *x,
                                   const float *gate, const float *mix, const float *gamma,
                                   const float *beta, int64_t B, int64_t H, int64_t L, int64_t D,
                                   int64_t keep, int64_t win_left, int64_t win_right, int dtype,
                                   int gate_kind, int norm_order, double *out, double *y_out,
                                   int nthreads);

/* The mix with the local branch: out = LN(x + y + y_loc) (norm order 0) or
 * x + LN(y + y_loc) (norm order 1), y with the given gate kind; optionally
 * y + y_loc. */
int oracle_spectre_mix_local_ex(const void *q, const void *k, const void *v, const void *x,
                                const float *gate, const float *gamma, const float *beta,
                                int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep,
                                int64_t win_left, int64_t win_right, int dtype, int gate_kind,
                                int norm_order, double *out, double *y_out, int nthreads) {
  return oracle_spectre_mix_local_gated(q, k, v, x, gate, NULL, gamma, beta, B, H, L, D, keep,
                                        win_left, win_right, dtype, gate_kind, norm_order, out,
                                        y_out, nthreads);
}

/* The mix with the local branch, the branches weighted per channel:
 * y_sum = mix[c] * y + (1 - mix[c]) * y_loc (mix null: the plain sum
 * y + y_loc), then the residual and the norm of the given order; y_out, if
 * given, receives y_sum. */
int oracle_spectre_mix_local_gated(const void *q, const void *k, const void *v, const void *x,
                                   const float *gate, const float *mix, const float *gamma,
                                   const float *beta, int64_t B, int64_t H, int64_t L, int64_t D,
                                   int64_t keep, int64_t win_left, int64_t win_right, int dtype,
                                   int gate_kind, int norm_order, double *out, double *y_out,
                                   int nthreads) {
  if (!x || !gamma || !beta || !out) return ORACLE_EINVAL;
  if (check_variant(gate_kind, norm_order)) return ORACLE_EINVAL;
  int s = check_dims(B, H, L, D, keep, dtype);
  if (s) return s;
  const int64_t C = H * D, ntok = B * L;
  double *y = y_out ? y_out : (double *)malloc(sizeof(double) * (size_t)(ntok * C));
  double *yl = (double *)malloc(sizeof(double) * (size_t)(ntok * C));
  if (!y || !yl) {
    if (!y_out) free(y);
    free(yl);
    return ORACLE_ENOMEM;
  }
  s = oracle_spectre_y_ex(q, k, v, gate, B, H, L, D, keep, dtype, gate_kind, y, nthreads);
  if (s == ORACLE_OK) s = oracle_local_attention(q, k, v, B, H, L, D, win_left, win_right, dtype, yl);
  if (s == ORACLE_OK) {
    if (mix) {
      for (int64_t i = 0; i < ntok * C; ++i) {
        const double g = (double)mix[i % C];
        y[i] = g * y[i] + (1.0 - g) * yl[i];
      }
    } else {
      for (int64_t i = 0; i < ntok * C; ++i) y[i] += yl[i];
    }
    layernorm_rows(y, x, dtype, NULL, gamma, beta, ntok, C, norm_order, out);
  }
  if (!y_out) free(y);
  free(yl);
  return s;
}

int oracle_spectre_mix_local(const void *q, const void *k, const void *v, const void *x,
                             const float *gate, const float *gamma, const float *beta,
                             int64_t B, int64_t H, int64_t L, int64_t D, int64_t keep,
                             int64_t win_left, int64_t win_right, int dtype, double *out,
                             double *y_out, int nthreads) {
  return oracle_spectre_mix_local_ex(q, k, v, x, gate, gamma, beta, B, H, L, D, keep, win_left,
                                     win_right, dtype, 0, 0, out, y_out, nthreads);
}

/* Number of threads a call with `nthreads` would use (0 = all online CPUs). */
int oracle_threads(int nthreads) { return resolve_threads(nthreads); }
