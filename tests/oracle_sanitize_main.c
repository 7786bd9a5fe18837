/*
 * oracle_sanitize_main.c -- a stand-alone driver of the CPU oracle
 * (oracle/adaln_oracle.c) for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py compiles it
 * with gcc, CPU only).  It runs every oracle entry point on small ragged
 * problems -- tails, one-element rows, every lane count from 16 to 1024, the
 * worked D = 4 row -- so that an out-of-bounds access, a use of uninitialized
 * memory the sanitizers see, signed overflow or a misaligned access in the
 * oracle stops the run.  It also checks the closed forms it can state
 * exactly (the worked row, constant rows, empty problems), and prints "ok".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float orc_f32_from_bf16(uint16_t h);
uint16_t orc_bf16_from_f32(float f);
uint16_t orc_bf16_from_f64(double d);
uint8_t orc_fp8e4m3_from_f32(float f);
double orc_f64_from_fp8e4m3(uint8_t c);
int orc_layernorm_stats(const uint16_t* x, int64_t R, int64_t D, float eps, int mode, int V, int L, double* mean,
                        double* rstd);
int orc_ln_modulate(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale, const uint16_t* shift,
                    float eps, int mode, int V, int L, uint16_t* out, double* mean_out, double* rstd_out);
int orc_residual_gate_add(const uint16_t* res, const uint16_t* gate, const uint16_t* upd, int64_t B, int64_t S,
                          int64_t D, int mode, uint16_t* out);
int orc_rmsnorm_scale_shift(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                            const uint16_t* shift, float eps, int mode, int V, int L, uint16_t* out, double* rinv_out);
int orc_qk_rmsnorm(const uint16_t* x, int64_t R, int64_t Dh, const uint16_t* w, float eps, int mode, int V, int L,
                   uint16_t* out);
int orc_ln_modulate_fold(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                         const uint16_t* shift, float eps, int mode, int V, int L, uint16_t* out, double* mean_out,
                         double* rstd_out);
int orc_ln_modulate_fp8(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                        const uint16_t* shift, float eps, float qscale, int mode, int V, int L, uint8_t* out,
                        double* mean_out, double* rstd_out);
int orc_residual_gate_add_ln_modulate(const uint16_t* res, const uint16_t* gate, const uint16_t* upd, int64_t B,
                                      int64_t S, int64_t D, const uint16_t* scale, const uint16_t* shift, float eps,
                                      int mode, int V, int L, uint16_t* res_out, uint16_t* out, double* mean_out,
                                      double* rstd_out);
int orc_modulate_scale_shift(const uint16_t* x, int64_t B, int64_t S, int64_t D, const uint16_t* scale,
                             int64_t ssc_b, int64_t ssc_s, const uint16_t* shift, int64_t ssh_b, int64_t ssh_s,
                             int mode, uint16_t* out);
int orc_temb_table_slices(const float* table, const void* temb, int temb_f32, int64_t B, int64_t L, int64_t nmod,
                          int64_t D, float* out);
int orc_qk_head_layernorm(const uint16_t* x, int64_t R, int64_t Dh, const uint16_t* w, const uint16_t* b, float eps,
                          int mode, int V, int L, uint16_t* out);
int orc_bias_gelu_tanh(const uint16_t* x, int64_t rows, int64_t width, const uint16_t* bias, uint16_t* out,
                       double* value_out);

#define FP64 0
#define FP32 1

static int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

/* deterministic pseudo-normal bf16 values (sum of uniforms), exact sizes */
static uint64_t rng_state = 12345;
static double urand(void) {
  rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(rng_state >> 11) / 9007199254740992.0;
}
static uint16_t* rand_bf16(int64_t n, double mean, double std) {
  uint16_t* p = (uint16_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(uint16_t));
  for (int64_t i = 0; i < n; ++i) {
    double s = 0;
    for (int k = 0; k < 4; ++k) s += urand() - 0.5;
    p[i] = orc_bf16_from_f64(mean + std * s * 1.7320508075688772);
  }
  return p;
}

static void worked_row(void) {
  const float xs[4] = {-3, -1, 1, 3};
  const float want[4] = {-1.34375f, -0.447265625f, 0.447265625f, 1.34375f};
  uint16_t x[4], z[4], out[4];
  for (int i = 0; i < 4; ++i) {
    x[i] = orc_bf16_from_f32(xs[i]);
    z[i] = 0;
  }
  for (int mode = 0; mode < 2; ++mode) {
    double m, r;
    CHECK(orc_ln_modulate(x, 1, 1, 4, z, z, 1e-6f, mode, 4, 64, out, &m, &r) == 0, "worked row rc");
    for (int i = 0; i < 4; ++i) CHECK(orc_f32_from_bf16(out[i]) == want[i], "worked row element %d mode %d", i, mode);
    CHECK(m == 0.0, "worked row mean");
  }
}

static void row_ops(int64_t B, int64_t S, int64_t D, int V, int L) {
  const int64_t R = B * S;
  uint16_t* x = rand_bf16(R * D, 0.5, 2.0);
  uint16_t* u = rand_bf16(R * D, 0.0, 1.0);
  uint16_t* sc = rand_bf16(B * D, 0.0, 0.1);
  uint16_t* sh = rand_bf16(B * D, 0.0, 0.1);
  uint16_t* gt = rand_bf16(B * D, 0.0, 0.5);
  uint16_t* out = (uint16_t*)malloc((size_t)(R * D) * 2);
  uint16_t* out2 = (uint16_t*)malloc((size_t)(R * D) * 2);
  uint8_t* q8 = (uint8_t*)malloc((size_t)(R * D));
  double* m = (double*)malloc((size_t)R * sizeof(double));
  double* r = (double*)malloc((size_t)R * sizeof(double));
  for (int mode = 0; mode < 2; ++mode) {
    CHECK(orc_layernorm_stats(x, R, D, 1e-6f, mode, V, L, m, r) == 0, "stats D=%ld L=%d", (long)D, L);
    CHECK(orc_ln_modulate(x, B, S, D, sc, sh, 1e-6f, mode, V, L, out, m, r) == 0, "lnm D=%ld", (long)D);
    CHECK(orc_rmsnorm_scale_shift(x, B, S, D, sc, sh, 1e-6f, mode, V, L, out, r) == 0, "rms D=%ld", (long)D);
    CHECK(orc_ln_modulate_fold(x, B, S, D, sc, sh, 1e-6f, mode, V, L, out, m, r) == 0, "fold D=%ld", (long)D);
    CHECK(orc_ln_modulate_fp8(x, B, S, D, sc, sh, 1e-6f, 0.37f, mode, V, L, q8, m, r) == 0, "fp8 D=%ld", (long)D);
    CHECK(orc_residual_gate_add(x, gt, u, B, S, D, mode, out) == 0, "rga D=%ld", (long)D);
    CHECK(orc_residual_gate_add_ln_modulate(x, gt, u, B, S, D, sc, sh, 1e-6f, mode, V, L, out, out2, m, r) == 0,
          "fused D=%ld", (long)D);
    CHECK(orc_modulate_scale_shift(x, B, S, D, sc, D, 0, sh, D, 0, mode, out) == 0, "mod D=%ld", (long)D);
    CHECK(orc_modulate_scale_shift(x, B, S, D, x, S * D, D, u, S * D, D, mode, out) == 0, "mod per token");
  }
  /* constant rows: +0 out with zero scale/shift, mean exact */
  for (int64_t i = 0; i < R * D; ++i) x[i] = orc_bf16_from_f32(-3.5f);
  memset(sc, 0, (size_t)(B * D) * 2);
  memset(sh, 0, (size_t)(B * D) * 2);
  CHECK(orc_ln_modulate(x, B, S, D, sc, sh, 1e-6f, FP32, V, L, out, m, r) == 0, "const rc");
  for (int64_t i = 0; i < R * D; ++i) CHECK(out[i] == 0, "constant row output %ld", (long)i);
  for (int64_t i = 0; i < R; ++i) CHECK(m[i] == -3.5, "constant row mean");
  free(x);
  free(u);
  free(sc);
  free(sh);
  free(gt);
  free(out);
  free(out2);
  free(q8);
  free(m);
  free(r);
}

static void head_ops(int64_t R, int64_t Dh) {
  const int V = Dh % 8 == 0 ? 8 : 4;
  uint16_t* x = rand_bf16(R * Dh, 0.0, 1.0);
  uint16_t* w = rand_bf16(Dh, 1.0, 0.05);
  uint16_t* b = rand_bf16(Dh, 0.0, 0.02);
  uint16_t* out = (uint16_t*)malloc((size_t)(R * Dh) * 2);
  for (int mode = 0; mode < 2; ++mode) {
    CHECK(orc_qk_head_layernorm(x, R, Dh, w, b, 1e-6f, mode, V, 16, out) == 0, "qk Dh=%ld", (long)Dh);
    CHECK(orc_qk_head_layernorm(x, R, Dh, 0, 0, 1e-6f, mode, V, 16, out) == 0, "qk no affine");
    CHECK(orc_qk_rmsnorm(x, R, Dh, w, 1e-6f, mode, V, 16, out) == 0, "qk rms Dh=%ld", (long)Dh);
    CHECK(orc_qk_rmsnorm(x, R, Dh, 0, 1e-6f, mode, V, 16, out) == 0, "qk rms no weight");
  }
  free(x);
  free(w);
  free(b);
  free(out);
}

int main(void) {
  worked_row();
  /* row lengths with tails, V = 4 and 8, lane counts 16 .. 1024 (W = 1 .. 16 waves) */
  const int64_t Ds[] = {4, 8, 12, 60, 520, 2240, 4100, 8200, 16392};
  for (size_t i = 0; i < sizeof Ds / sizeof Ds[0]; ++i) {
    const int64_t D = Ds[i];
    const int V = D % 8 == 0 ? 8 : 4;
    for (int L = 16; L <= 1024; L *= 2) row_ops(2, 3, D, V, L);
  }
  row_ops(1, 1, 65532, 4, 1024);
  row_ops(0, 5, 64, 8, 64); /* empty */
  const int64_t Dhs[] = {4, 12, 64, 128, 132, 256};
  for (size_t i = 0; i < sizeof Dhs / sizeof Dhs[0]; ++i) head_ops(7, Dhs[i]);
  /* GELU, temb slices, FP8 conversions */
  {
    uint16_t* x = rand_bf16(5 * 37, 0.0, 3.0);
    uint16_t* bias = rand_bf16(37, 0.0, 0.1);
    uint16_t* out = (uint16_t*)malloc(5 * 37 * 2);
    double* val = (double*)malloc(5 * 37 * sizeof(double));
    CHECK(orc_bias_gelu_tanh(x, 5, 37, bias, out, val) == 0, "gelu");
    free(x);
    free(bias);
    free(out);
    free(val);
    float table[6 * 20];
    for (int i = 0; i < 6 * 20; ++i) table[i] = (float)urand();
    uint16_t* temb = rand_bf16(2 * 3 * 6 * 20, 0.0, 1.0);
    float* slices = (float*)malloc(6 * 2 * 3 * 20 * sizeof(float));
    CHECK(orc_temb_table_slices(table, temb, 0, 2, 3, 6, 20, slices) == 0, "temb");
    free(temb);
    free(slices);
    for (int c = 0; c < 256; ++c) {
      const double v = orc_f64_from_fp8e4m3((uint8_t)c);
      if (!isnan(v)) CHECK(orc_fp8e4m3_from_f32((float)v) == (uint8_t)c || v == 0.0, "fp8 code %d", c);
    }
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
