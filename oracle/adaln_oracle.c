/*
 * adaln_oracle.c -- plain, slow CPU oracle of the eager adaLN chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or constant with the HIP
 * library: every helper below (bf16 rounding included) is written here.
 *
 * What it computes (sources are the pages on the SGLang-Diffusion fused
 * kernels):
 *   - "Fused Kernels" (SGLang Diffusion docs), section "Numerical contracts
 *     and quality tiers": the fused chain must reproduce every bf16 rounding
 *     boundary of the eager PyTorch chain.
 *   - prhub report on sglang PR #34015 (Sana fused adaLN), 关键源码片段,
 *     layernorm_modulate.py pass 2: x_hat = bf16(rstd*(x-mean)),
 *     one_plus = bf16(1+scale), y = bf16(x_hat*one_plus), out = bf16(y+shift).
 *   - prhub report on sglang PR #34008 (GLM-Image), 关键源码片段 _welford_push:
 *     delta = x-mean; mean' = fma(delta, 1/(cnt+1), mean);
 *     m2' = fma(delta, x-mean', m2).
 *   - same report, 实现拆解: per-head q/k LayerNorm; residual + gate*update.
 *   - PR #37075 report (Wan2.2 bias + GELU), 实现拆解 §1: add bias in fp32,
 *     round to bf16, then tanh-GELU, round again.
 *
 * Two modes for the LayerNorm statistics:
 *   ORC_FP64_TWO_PASS  the plain definition: mean = sum(x)/D and
 *                      var = sum((x-mean)^2)/D in double, rstd =
 *                      1/sqrt(var+eps); every later step in double, rounded
 *                      once to bf16 (round-to-nearest-even).
 *   ORC_FP32_FIXED     the fp32 Welford algorithm in one fixed, documented
 *                      order, parameterised by (V, L):
 *                        * the row is cut into vectors of V consecutive
 *                          elements; vector v belongs to lane (v mod L);
 *                        * each lane pushes its elements in increasing
 *                          position into its own (mean, m2, n) Welford state,
 *                          with 1/n the correctly rounded fp32 reciprocal;
 *                        * lanes are merged pairwise, nearest first: at
 *                          offset 1, 2, 4, ... lane l (l mod 2*off == 0)
 *                          takes combine(state[l], state[l+off]) with the
 *                          Chan-Golub-LeVeque update (lower lane first);
 *                        * var = m2/D, rstd = 1/sqrt(var+eps), IEEE fp32.
 *                      Every later step is done in fp32 and rounded to bf16
 *                      exactly where the eager chain rounds.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp (no -ffast-math):
 * fp32 arithmetic is plain IEEE binary32 with round-to-nearest-even and
 * gradual underflow.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FP64_TWO_PASS 0
#define ORC_FP32_FIXED 1

#define ORC_OK 0
#define ORC_EINVAL -1

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32 / fp64                                                 */
/* ------------------------------------------------------------------ */

static uint32_t bits_of_f32(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

static float f32_of_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* bf16 is the upper half of a binary32: widening is exact. */
float orc_f32_from_bf16(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/*
 * Round a binary32 to the nearest bf16, ties to even.
 * Sign-magnitude encoding: dropping the low 16 bits gives the neighbour of
 * smaller magnitude; adding one to the kept magnitude gives the next one up
 * (a carry into the exponent field is the correct next value, and rounding
 * past the largest finite value yields infinity).  NaN stays NaN (quiet).
 */
uint16_t orc_bf16_from_f32(float f) {
  uint32_t u = bits_of_f32(f);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xffffu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept;
}

/*
 * Round a binary64 straight to the nearest bf16, ties to even (no detour
 * through binary32).  The two candidates are the bf16 values that bracket
 * |d|; the nearer one wins, a tie goes to the even encoding.
 */
uint16_t orc_bf16_from_f64(double d) {
  if (isnan(d)) return (uint16_t)0x7fc0u;
  uint16_t sign = signbit(d) ? 0x8000u : 0u;
  double a = fabs(d);
  if (isinf(a)) return (uint16_t)(sign | 0x7f80u);
  /* lower candidate: largest bf16 magnitude <= a (search on the encoding,
     which is monotone in magnitude for non-negative values) */
  uint32_t lo = 0, hi = 0x7f80u; /* 0x7f80 = +inf */
  while (hi - lo > 1) {
    uint32_t mid = (lo + hi) / 2;
    if ((double)orc_f32_from_bf16((uint16_t)mid) <= a)
      lo = mid;
    else
      hi = mid;
  }
  /* now value(lo) <= a < value(lo+1) (value(0x7f80) taken as 2^128) */
  double vlo = (double)orc_f32_from_bf16((uint16_t)lo);
  if (vlo == a) return (uint16_t)(sign | lo);
  uint32_t up = lo + 1;
  double vup = (up == 0x7f80u) ? ldexp(1.0, 128) : (double)orc_f32_from_bf16((uint16_t)up);
  double below = a - vlo; /* exact: both operands share the binade scale */
  double above = vup - a;
  uint32_t pick;
  if (below < above)
    pick = lo;
  else if (above < below)
    pick = up;
  else
    pick = (lo & 1u) ? up : lo;
  return (uint16_t)(sign | pick);
}

void orc_bf16_from_f32_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(in[i]);
}

void orc_bf16_from_f64_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(in[i]);
}

/* round an fp32 value to bf16 and widen it back: the value eager stores */
static float rb(float f) { return orc_f32_from_bf16(orc_bf16_from_f32(f)); }
static double rb64(double d) { return (double)orc_f32_from_bf16(orc_bf16_from_f64(d)); }

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3       */
/* mantissa bits, no infinities, S.1111.111 is NaN, largest finite      */
/* 448, subnormals k * 2^-9).  Value of a code, and the nearest code to */
/* a real value with ties to the even code, written from that           */
/* definition.  Magnitudes that round past 448 (above 464) have no      */
/* finite code: NaN, as torch's conversion gives (no saturation).       */
/* ------------------------------------------------------------------ */

double orc_f64_from_fp8e4m3(uint8_t c) {
  int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return sgn ? -v : v;
}

static uint8_t fp8_nearest(double a, int sgn) {
  /* a >= 0 finite.  Codes 0x00..0x7E increase in value; the slot after
     448 (code 0x7F, which would be 480) is NaN, so a value rounding to it
     -- anything above the midpoint 464, or at or beyond 480 -- is NaN. */
  if (a >= 480.0) return (uint8_t)(0x7F | (sgn << 7));
  int lo = 0;
  while (lo < 0x7E && orc_f64_from_fp8e4m3((uint8_t)(lo + 1)) <= a) ++lo;
  double v1 = orc_f64_from_fp8e4m3((uint8_t)lo);
  double v2 = lo < 0x7E ? orc_f64_from_fp8e4m3((uint8_t)(lo + 1)) : 480.0;
  double mid = 0.5 * (v1 + v2); /* exact: both values have few significant bits */
  int code = lo;
  if (a > mid || (a == mid && ((lo + 1) & 1) == 0)) code = lo + 1;
  return (uint8_t)(code | (sgn << 7));
}

uint8_t orc_fp8e4m3_from_f64(double d) {
  if (isnan(d)) return 0x7F;
  return fp8_nearest(fabs(d), signbit(d) ? 1 : 0);
}

uint8_t orc_fp8e4m3_from_f32(float f) { return orc_fp8e4m3_from_f64((double)f); }

void orc_fp8e4m3_from_f32_array(const float* in, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8e4m3_from_f32(in[i]);
}

/* ------------------------------------------------------------------ */
/* Welford (Welford 1962) and the pairwise merge (Chan, Golub, LeVeque) */
/* ------------------------------------------------------------------ */

typedef struct {
  float mean;
  float m2;
  float n;
} orc_wstate;

/* one Welford step, the order printed for _welford_push in the PR #34008
   report, with 1/n the correctly rounded fp32 reciprocal of the new count */
static void welford_push(orc_wstate* s, float x) {
  s->n = s->n + 1.0f;
  float r = 1.0f / s->n;
  float delta = x - s->mean;
  s->mean = fmaf(delta, r, s->mean);
  s->m2 = fmaf(delta, x - s->mean, s->m2);
}

/* merge two partial states; a comes from the lower lane.  An empty side
   leaves the other one untouched (the "guarded" merge). */
static orc_wstate welford_combine(orc_wstate a, orc_wstate b) {
  if (b.n == 0.0f) return a;
  if (a.n == 0.0f) return b;
  orc_wstate c;
  c.n = a.n + b.n;
  float f = b.n / c.n;
  float delta = b.mean - a.mean;
  c.mean = fmaf(delta, f, a.mean);
  c.m2 = (a.m2 + b.m2) + (delta * delta) * (a.n * f);
  return c;
}

/* exported for the oracle's own pins */
void orc_welford_seq(const float* x, int64_t n, float* mean, float* m2) {
  orc_wstate s = {0.0f, 0.0f, 0.0f};
  for (int64_t i = 0; i < n; ++i) welford_push(&s, x[i]);
  *mean = s.mean;
  *m2 = s.m2;
}

void orc_welford_combine(const float* a /*mean,m2,n*/, const float* b, float* out) {
  orc_wstate sa = {a[0], a[1], a[2]};
  orc_wstate sb = {b[0], b[1], b[2]};
  orc_wstate c = welford_combine(sa, sb);
  out[0] = c.mean;
  out[1] = c.m2;
  out[2] = c.n;
}

static int is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

#define ORC_MAX_LANES 1024

/* statistics of one row of D bf16 values in the fixed fp32 order (V, L) */
static void row_stats_fp32(const uint16_t* x, int64_t D, float eps, int V, int L, float* mean_out,
                           float* rstd_out) {
  orc_wstate lane[ORC_MAX_LANES];
  for (int l = 0; l < L; ++l) lane[l] = (orc_wstate){0.0f, 0.0f, 0.0f};
  int64_t nvec = D / V;
  for (int l = 0; l < L; ++l)
    for (int64_t v = l; v < nvec; v += L)
      for (int e = 0; e < V; ++e) welford_push(&lane[l], orc_f32_from_bf16(x[v * V + e]));
  for (int off = 1; off < L; off *= 2)
    for (int l = 0; l < L; l += 2 * off) lane[l] = welford_combine(lane[l], lane[l + off]);
  float var = lane[0].m2 / (float)D;
  float t = var + eps;
  float s = sqrtf(t);
  *mean_out = lane[0].mean;
  *rstd_out = 1.0f / s;
}

/* statistics of one row in the plain two-pass double definition */
static void row_stats_fp64(const uint16_t* x, int64_t D, float eps, double* mean_out, double* rstd_out) {
  double sum = 0.0;
  for (int64_t j = 0; j < D; ++j) sum += (double)orc_f32_from_bf16(x[j]);
  double mean = sum / (double)D;
  double ss = 0.0;
  for (int64_t j = 0; j < D; ++j) {
    double c = (double)orc_f32_from_bf16(x[j]) - mean;
    ss += c * c;
  }
  double var = ss / (double)D;
  *mean_out = mean;
  *rstd_out = 1.0 / sqrt(var + (double)eps);
}

static int check_order(int64_t D, int V, int L) {
  if (D <= 0) return ORC_EINVAL;
  if (V != 4 && V != 8) return ORC_EINVAL;
  if (D % V != 0) return ORC_EINVAL;
  if (!is_pow2(L) || L > ORC_MAX_LANES) return ORC_EINVAL;
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* LayerNorm statistics only                                            */
/* ------------------------------------------------------------------ */

int orc_layernorm_stats(const uint16_t* x, int64_t R, int64_t D, float eps, int mode, int V, int L,
                        double* mean, double* rstd) {
  if (R < 0) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(D, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    if (mode == ORC_FP32_FIXED) {
      float m, s;
      row_stats_fp32(x + r * D, D, eps, V, L, &m, &s);
      mean[r] = m;
      rstd[r] = s;
    } else {
      row_stats_fp64(x + r * D, D, eps, &mean[r], &rstd[r]);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* The adaLN modulate tail shared by the LayerNorm and RMSNorm chains:  */
/* given the normalized value n (before its rounding), x_hat = bf16(n), */
/* one_plus = bf16(1 + scale), y = bf16(x_hat * one_plus),              */
/* out = bf16(y + shift) -- one rounding per eager op.                  */
/* ------------------------------------------------------------------ */

static uint16_t modulate_tail_f32(float n, uint16_t sc, uint16_t sh) {
  float xhat = rb(n);
  float one_plus = rb(1.0f + orc_f32_from_bf16(sc));
  float y = rb(xhat * one_plus);
  return orc_bf16_from_f32(y + orc_f32_from_bf16(sh));
}

static uint16_t modulate_tail_f64(double n, uint16_t sc, uint16_t sh) {
  double xhat = rb64(n);
  double one_plus = rb64(1.0 + (double)orc_f32_from_bf16(sc));
  double y = rb64(xhat * one_plus);
  return orc_bf16_from_f64(y + (double)orc_f32_from_bf16(sh));
}

/* ------------------------------------------------------------------ */
/* ln_modulate: LN(x) * (1 + scale) + shift, per-sample scale/shift     */
/* x [B*S, D] logical row-major; scale, shift [B, D]; out [B*S, D]      */
/* ------------------------------------------------------------------ */

int orc_ln_modulate(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                    const uint16_t* shift, float eps, int mode, int V, int L, uint16_t* out,
                    double* mean_out, double* rstd_out) {
  if (B < 0 || S < 0 || D <= 0) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(D, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
  int64_t R = B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* xr = x + r * D;
    const uint16_t* sc = scale + (r / S) * D;
    const uint16_t* sh = shift + (r / S) * D;
    uint16_t* o = out + r * D;
    if (mode == ORC_FP32_FIXED) {
      float mean, rstd;
      row_stats_fp32(xr, D, eps, V, L, &mean, &rstd);
      for (int64_t j = 0; j < D; ++j) o[j] = modulate_tail_f32((orc_f32_from_bf16(xr[j]) - mean) * rstd, sc[j], sh[j]);
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    } else {
      double mean, rstd;
      row_stats_fp64(xr, D, eps, &mean, &rstd);
      for (int64_t j = 0; j < D; ++j)
        o[j] = modulate_tail_f64(((double)orc_f32_from_bf16(xr[j]) - mean) * rstd, sc[j], sh[j]);
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* residual_gate_add: residual + gate * update (two eager ops)          */
/* res, upd [B*S, D]; gate [B, D]                                       */
/* ------------------------------------------------------------------ */

int orc_residual_gate_add(const uint16_t* res, const uint16_t* gate, const uint16_t* upd, int64_t B,
                          int64_t S, int64_t D, int mode, uint16_t* out) {
  if (B < 0 || S < 0 || D < 0) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
  int64_t R = B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* g = gate + (r / S) * D;
    for (int64_t j = 0; j < D; ++j) {
      int64_t i = r * D + j;
      if (mode == ORC_FP32_FIXED) {
        float t = rb(orc_f32_from_bf16(g[j]) * orc_f32_from_bf16(upd[i]));
        out[i] = orc_bf16_from_f32(orc_f32_from_bf16(res[i]) + t);
      } else {
        double t = rb64((double)orc_f32_from_bf16(g[j]) * (double)orc_f32_from_bf16(upd[i]));
        out[i] = orc_bf16_from_f64((double)orc_f32_from_bf16(res[i]) + t);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* RMSNorm statistics.  The pages' RMSNorm fusions ("Fused Kernels"     */
/* page, table "Normalization": rmsnorm_scale_shift, qk_rmsnorm_native; */
/* the request-gated fusion table: rms_norm(x) * (1 + scale) + shift)   */
/* normalize by the root mean square: x_hat = x / sqrt(mean(x^2) + eps) */
/* with no mean subtraction.                                            */
/*   fp64: ss = sum of x^2 in double (sequential), rinv =               */
/*         1/sqrt(ss/D + eps).                                          */
/*   fp32(V, L): lane l owns vectors l, l+L, ... of V elements and      */
/*         accumulates ss = fma(x, x, ss) in increasing position; lanes */
/*         are summed pairwise nearest-first (lane l takes              */
/*         ss[l] + ss[l+off], lower first); then ms = ss/D,             */
/*         rinv = 1/sqrt(ms + eps), IEEE fp32.                          */
/* ------------------------------------------------------------------ */

static float row_rinv_fp32(const uint16_t* x, int64_t D, float eps, int V, int L) {
  float lane[ORC_MAX_LANES];
  for (int l = 0; l < L; ++l) lane[l] = 0.0f;
  int64_t nvec = D / V;
  for (int l = 0; l < L; ++l)
    for (int64_t v = l; v < nvec; v += L)
      for (int e = 0; e < V; ++e) {
        float xv = orc_f32_from_bf16(x[v * V + e]);
        lane[l] = fmaf(xv, xv, lane[l]);
      }
  for (int off = 1; off < L; off *= 2)
    for (int l = 0; l < L; l += 2 * off) lane[l] = lane[l] + lane[l + off];
  float ms = lane[0] / (float)D;
  float t = ms + eps;
  float s = sqrtf(t);
  return 1.0f / s;
}

static double row_rinv_fp64(const uint16_t* x, int64_t D, float eps) {
  double ss = 0.0;
  for (int64_t j = 0; j < D; ++j) {
    double xv = (double)orc_f32_from_bf16(x[j]);
    ss += xv * xv;
  }
  return 1.0 / sqrt(ss / (double)D + (double)eps);
}

/* rmsnorm_scale_shift: RMSNorm(x) * (1 + scale) + shift, the eager ops  */
/* of that chain each rounded to bf16 (x_hat = bf16(x * rinv), then the  */
/* modulate tail).  x [B*S, D]; scale, shift [B, D].                     */
int orc_rmsnorm_scale_shift(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                            const uint16_t* shift, float eps, int mode, int V, int L, uint16_t* out,
                            double* rinv_out) {
  if (B < 0 || S < 0 || D <= 0) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(D, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
  int64_t R = B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* xr = x + r * D;
    const uint16_t* sc = scale + (r / S) * D;
    const uint16_t* sh = shift + (r / S) * D;
    uint16_t* o = out + r * D;
    if (mode == ORC_FP32_FIXED) {
      float rinv = row_rinv_fp32(xr, D, eps, V, L);
      for (int64_t j = 0; j < D; ++j) o[j] = modulate_tail_f32(orc_f32_from_bf16(xr[j]) * rinv, sc[j], sh[j]);
      if (rinv_out) rinv_out[r] = rinv;
    } else {
      double rinv = row_rinv_fp64(xr, D, eps);
      for (int64_t j = 0; j < D; ++j) o[j] = modulate_tail_f64((double)orc_f32_from_bf16(xr[j]) * rinv, sc[j], sh[j]);
      if (rinv_out) rinv_out[r] = rinv;
    }
  }
  return ORC_OK;
}

/* qk_rmsnorm: RMSNorm over each head row of Dh with an optional weight, */
/* one eager op (torch's rms_norm: x * rinv, times the weight, computed  */
/* in fp32 and rounded once): out = bf16((x * rinv) * w).  x [R, Dh];    */
/* w [Dh] or NULL.                                                        */
int orc_qk_rmsnorm(const uint16_t* x, int64_t R, int64_t Dh, const uint16_t* w, float eps, int mode, int V,
                   int L, uint16_t* out) {
  if (R < 0 || Dh <= 0) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(Dh, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* xr = x + r * Dh;
    uint16_t* o = out + r * Dh;
    if (mode == ORC_FP32_FIXED) {
      float rinv = row_rinv_fp32(xr, Dh, eps, V, L);
      for (int64_t j = 0; j < Dh; ++j) {
        float xn = orc_f32_from_bf16(xr[j]) * rinv;
        float y = w ? xn * orc_f32_from_bf16(w[j]) : xn;
        o[j] = orc_bf16_from_f32(y);
      }
    } else {
      double rinv = row_rinv_fp64(xr, Dh, eps);
      for (int64_t j = 0; j < Dh; ++j) {
        double xn = (double)orc_f32_from_bf16(xr[j]) * rinv;
        double y = w ? xn * (double)orc_f32_from_bf16(w[j]) : xn;
        o[j] = orc_bf16_from_f64(y);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* ln_modulate_fold: the single-rounding variant the pages offer in the  */
/* high-quality tier ("Fused Kernels" page, request-gated fusion table:  */
/* layer_norm(x, weight=(1 + scale), bias=shift) in place of an affine- */
/* free LayerNorm plus a separate modulate).  One eager affine LayerNorm */
/* op with the bf16 weight tensor (1 + scale): out = bf16(fma(w, n, b)), */
/* n = RN(RN(x - mean) * rstd) in fp32 (fp64 mode: w * n + b in double), */
/* w = bf16(1 + scale), b = shift.  Not the eager four-op chain's bits:  */
/* it drops the roundings of x_hat and of the product.                   */
/* ------------------------------------------------------------------ */

int orc_ln_modulate_fold(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                         const uint16_t* shift, float eps, int mode, int V, int L, uint16_t* out, double* mean_out,
                         double* rstd_out) {
  if (B < 0 || S < 0 || D <= 0) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(D, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
  int64_t R = B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* xr = x + r * D;
    const uint16_t* sc = scale + (r / S) * D;
    const uint16_t* sh = shift + (r / S) * D;
    uint16_t* o = out + r * D;
    if (mode == ORC_FP32_FIXED) {
      float mean, rstd;
      row_stats_fp32(xr, D, eps, V, L, &mean, &rstd);
      for (int64_t j = 0; j < D; ++j) {
        float n = (orc_f32_from_bf16(xr[j]) - mean) * rstd;
        float w = rb(1.0f + orc_f32_from_bf16(sc[j]));
        o[j] = orc_bf16_from_f32(fmaf(w, n, orc_f32_from_bf16(sh[j])));
      }
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    } else {
      double mean, rstd;
      row_stats_fp64(xr, D, eps, &mean, &rstd);
      for (int64_t j = 0; j < D; ++j) {
        double n = ((double)orc_f32_from_bf16(xr[j]) - mean) * rstd;
        double w = rb64(1.0 + (double)orc_f32_from_bf16(sc[j]));
        o[j] = orc_bf16_from_f64(w * n + (double)orc_f32_from_bf16(sh[j]));
      }
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* ln_modulate_fp8: ln_modulate with its bf16 output quantized straight  */
/* to static FP8 ("Fused Kernels" page, table "Quantized layout          */
/* producers": flux2_layernorm_modulate_fp8_quant, LayerNorm plus adaLN  */
/* modulation directly into static FP8 output).  With y the eager chain's */
/* bf16 output and s the static per-tensor scale:                        */
/*   fp32 mode: q = e4m3(RN(y * RN(1/s))) after clamping to [-448, 448]   */
/*   fp64 mode: q = e4m3(y / s) after the same clamp (exact quotient)     */
/* (NaN stays NaN).  out is one byte per element, [B*S, D].              */
/* ------------------------------------------------------------------ */

int orc_ln_modulate_fp8(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                        const uint16_t* shift, float eps, float qscale, int mode, int V, int L, uint8_t* out,
                        double* mean_out, double* rstd_out) {
  if (B < 0 || S < 0 || D <= 0) return ORC_EINVAL;
  if (!(qscale > 0.0f) || isinf(qscale)) return ORC_EINVAL;
  int64_t R = B * S;
  uint16_t* y = (uint16_t*)malloc((size_t)(R > 0 ? R * D : 1) * sizeof(uint16_t));
  if (!y) return ORC_EINVAL;
  int rc = orc_ln_modulate(x, B, S, D, scale, shift, eps, mode, V, L, y, mean_out, rstd_out);
  if (rc == ORC_OK) {
    const float inv = 1.0f / qscale;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < R * D; ++i) {
      if (mode == ORC_FP32_FIXED) {
        float v = orc_f32_from_bf16(y[i]) * inv;
        if (v > 448.0f) v = 448.0f;
        if (v < -448.0f) v = -448.0f;
        out[i] = orc_fp8e4m3_from_f32(v);
      } else {
        double v = (double)orc_f32_from_bf16(y[i]) / (double)qscale;
        if (v > 448.0) v = 448.0;
        if (v < -448.0) v = -448.0;
        out[i] = orc_fp8e4m3_from_f64(v);
      }
    }
  }
  free(y);
  return rc;
}

/* ------------------------------------------------------------------ */
/* residual_gate_add_ln_modulate: the gated residual update, then        */
/* ln_modulate of the updated residual ("Fused Kernels" page, table      */
/* "Normalization", scale_residual_norm_scale_shift: the norm + scale/   */
/* shift with the preceding residual + gate * update folded in).  Both   */
/* results are outputs: res_out = bf16(res + bf16(gate*upd)) and         */
/* out = ln_modulate(res_out).  res, upd [B*S, D]; gate, scale, shift    */
/* [B, D]; res_out, out [B*S, D].                                        */
/* ------------------------------------------------------------------ */

int orc_residual_gate_add_ln_modulate(const uint16_t* res, const uint16_t* gate, const uint16_t* upd,
                                      int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                                      const uint16_t* shift, float eps, int mode, int V, int L,
                                      uint16_t* res_out, uint16_t* out, double* mean_out,
                                      double* rstd_out) {
  int rc = orc_residual_gate_add(res, gate, upd, B, S, D, mode, res_out);
  if (rc != ORC_OK) return rc;
  return orc_ln_modulate(res_out, B, S, D, scale, shift, eps, mode, V, L, out, mean_out, rstd_out);
}

/* ------------------------------------------------------------------ */
/* modulate_scale_shift: x * (1 + scale) + shift as eager bf16 ops      */
/* ("Fused Kernels" page, table "adaLN modulation and gating";          */
/* one affine row per token for LingBot World's camera conditioning):   */
/* the modulate tail with x itself in place of the normalized value     */
/* (rounding a bf16 value to bf16 changes nothing).  x [B*S, D]; scale  */
/* and shift element (b,s,d) at base + b*s_b + s*s_s + d (s_s = 0: one  */
/* row per sample).                                                      */
/* ------------------------------------------------------------------ */

int orc_modulate_scale_shift(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                             int64_t ssc_b, int64_t ssc_s, const uint16_t* shift, int64_t ssh_b, int64_t ssh_s,
                             int mode, uint16_t* out) {
  if (B < 0 || S < 0 || D < 0) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
  int64_t R = B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const int64_t b = r / S, s = r % S;
    const uint16_t* sc = scale + b * ssc_b + s * ssc_s;
    const uint16_t* sh = shift + b * ssh_b + s * ssh_s;
    for (int64_t j = 0; j < D; ++j) {
      const uint16_t xv = x[r * D + j];
      out[r * D + j] = mode == ORC_FP32_FIXED ? modulate_tail_f32(orc_f32_from_bf16(xv), sc[j], sh[j])
                                              : modulate_tail_f64((double)orc_f32_from_bf16(xv), sc[j], sh[j]);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* temb_table_slices: the eager (table + temb.float()).chunk(nmod, dim=2)*/
/* with every slice made contiguous ("Fused Kernels" page, table "adaLN  */
/* modulation and gating", temb_table_slices and the note under it):    */
/* out[m][b, l, d] = table[m, d] + float(temb[b, l, m, d]), one fp32    */
/* addition.  table fp32 [nmod, D]; temb [B, L, nmod, D] contiguous,    */
/* bf16 (temb_f32 = 0) or fp32; out fp32 [nmod, B, L, D].               */
/* ------------------------------------------------------------------ */

int orc_temb_table_slices(const float* table, const void* temb, int temb_f32, int64_t B, int64_t L, int64_t nmod,
                          int64_t D, float* out) {
  if (B < 0 || L < 0 || nmod < 0 || D < 0) return ORC_EINVAL;
  int64_t R = B * L;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r)
    for (int64_t m = 0; m < nmod; ++m)
      for (int64_t d = 0; d < D; ++d) {
        const int64_t i = (r * nmod + m) * D + d;
        const float t = temb_f32 ? ((const float*)temb)[i] : orc_f32_from_bf16(((const uint16_t*)temb)[i]);
        out[(m * R + r) * D + d] = table[m * D + d] + t;
      }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* qk_head_layernorm: affine LayerNorm over each head row of Dh         */
/* x [R, Dh]; w, b [Dh] or both NULL (no affine); out [R, Dh]           */
/* One eager LayerNorm op, so one bf16 rounding at its output.          */
/* ------------------------------------------------------------------ */

int orc_qk_head_layernorm(const uint16_t* x, int64_t R, int64_t Dh, const uint16_t* w, const uint16_t* b,
                          float eps, int mode, int V, int L, uint16_t* out) {
  if (R < 0 || Dh <= 0) return ORC_EINVAL;
  if ((w == 0) != (b == 0)) return ORC_EINVAL;
  if (mode == ORC_FP32_FIXED && check_order(Dh, V, L) != ORC_OK) return ORC_EINVAL;
  if (mode != ORC_FP32_FIXED && mode != ORC_FP64_TWO_PASS) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* xr = x + r * Dh;
    uint16_t* o = out + r * Dh;
    if (mode == ORC_FP32_FIXED) {
      float mean, rstd;
      row_stats_fp32(xr, Dh, eps, V, L, &mean, &rstd);
      for (int64_t j = 0; j < Dh; ++j) {
        float xn = (orc_f32_from_bf16(xr[j]) - mean) * rstd;
        float y = w ? fmaf(orc_f32_from_bf16(w[j]), xn, orc_f32_from_bf16(b[j])) : xn;
        o[j] = orc_bf16_from_f32(y);
      }
    } else {
      double mean, rstd;
      row_stats_fp64(xr, Dh, eps, &mean, &rstd);
      for (int64_t j = 0; j < Dh; ++j) {
        double xn = ((double)orc_f32_from_bf16(xr[j]) - mean) * rstd;
        double y = w ? (double)orc_f32_from_bf16(w[j]) * xn + (double)orc_f32_from_bf16(b[j]) : xn;
        o[j] = orc_bf16_from_f64(y);
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* bias_gelu_tanh: z = bf16(x + bias); out = bf16(gelu_tanh(z))         */
/* x, out [rows, width]; bias [width].  Double precision.               */
/* gelu_tanh(z) = 0.5 z (1 + tanh(k0 (z + k1 z^3))), k0 = sqrt(2/pi),   */
/* k1 = 0.044715 (Hendrycks & Gimpel).  Evaluated through the identity  */
/* 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), which keeps full relative     */
/* accuracy where 1 + tanh(u) cancels (large negative z).               */
/* ------------------------------------------------------------------ */

double orc_gelu_tanh_f64(double z) {
  const double k0 = sqrt(2.0 / 3.14159265358979323846);
  const double k1 = 0.044715;
  double u = k0 * (z + k1 * z * z * z);
  return z / (1.0 + exp(-2.0 * u));
}

int orc_bias_gelu_tanh(const uint16_t* x, int64_t rows, int64_t width, const uint16_t* bias, uint16_t* out,
                       double* value_out) {
  if (rows < 0 || width < 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t j = 0; j < width; ++j) {
      int64_t i = r * width + j;
      double z = rb64((double)orc_f32_from_bf16(x[i]) + (double)orc_f32_from_bf16(bias[j]));
      double g = orc_gelu_tanh_f64(z);
      out[i] = orc_bf16_from_f64(g);
      if (value_out) value_out[i] = g;
    }
  }
  return ORC_OK;
}

/* OpenMP threads the row loops use (rows are independent: results do not
   depend on the thread count). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int orc_abi_version(void) { return 1; }
