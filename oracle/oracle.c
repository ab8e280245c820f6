/* ORACLE — test infrastructure only; see oracle.h for the sources and readings.
 * Plain fp64. OpenMP splits independent rows across threads; each row's sum is still one
 * left-to-right loop. */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* GN+ summary, "Kernel de dequantización optimizado con FMA": a weight is nibble*scale + bias.
 * Scale and bias are shared by `group` consecutive elements along a row (the input dimension). */
void oracle_dequant(int64_t rows, int64_t cols, int64_t group, const uint8_t* q, const uint16_t* scale,
                    const uint16_t* bias, double* W) {
  const int64_t ng = cols / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      const double s = bf16_value(scale[r * ng + c / group]);
      const double b = bf16_value(bias[r * ng + c / group]);
      W[r * cols + c] = s * (double)q[r * cols + c] + b;
    }
  }
}

/* GN+ summary, "Metal Compute Shaders": dequant matrix-vector product. */
void oracle_matvec(int64_t rows, int64_t cols, const double* W, const double* v, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double acc = 0.0;
    for (int64_t c = 0; c < cols; ++c) acc += W[r * cols + c] * v[c];
    out[r] = acc;
  }
}

/* HN thread: the router's result decides which experts are read. Logit e is router row e times x. */
void oracle_router_logits(int64_t E, int64_t H, const uint16_t* R, const double* x, double* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int64_t j = 0; j < H; ++j) acc += bf16_value(R[e * H + j]) * x[j];
    logits[e] = acc;
  }
}

typedef struct {
  double v;
  int32_t e;
} scored_t;

static int by_logit_then_index(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->e < y->e) ? -1 : (x->e > y->e);
}

/* GN+ summary, "Arquitectura del modelo": K experts are active per token. Selection is on the
 * logits (not on rounded probabilities); equal logits go to the lower expert index. */
void oracle_topk(int64_t E, int64_t K, const double* logits, int32_t* idx) {
  scored_t* s = (scored_t*)malloc((size_t)E * sizeof(scored_t));
  for (int64_t e = 0; e < E; ++e) {
    s[e].v = logits[e];
    s[e].e = (int32_t)e;
  }
  qsort(s, (size_t)E, sizeof(scored_t), by_logit_then_index);
  for (int64_t k = 0; k < K; ++k) idx[k] = s[k].e;
  free(s);
}

/* Softmax over all experts, then the chosen experts' probabilities renormalised to sum to 1. */
void oracle_route_weights(int64_t E, int64_t K, const double* logits, const int32_t* idx, double* w) {
  double m = logits[0];
  for (int64_t e = 1; e < E; ++e)
    if (logits[e] > m) m = logits[e];
  double z = 0.0;
  for (int64_t e = 0; e < E; ++e) z += exp(logits[e] - m);
  double sel = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    w[k] = exp(logits[idx[k]] - m) / z;
    sel += w[k];
  }
  for (int64_t k = 0; k < K; ++k) w[k] = w[k] / sel;
}

/* GN+ summary, "Metal Compute Shaders" (MoE combine + residual + gate): the shared expert's
 * output is scaled by a gate, read here as sigmoid of a learned vector dotted with x. */
double oracle_shared_gate(int64_t H, const uint16_t* gs, const double* x) {
  double acc = 0.0;
  for (int64_t j = 0; j < H; ++j) acc += bf16_value(gs[j]) * x[j];
  return 1.0 / (1.0 + exp(-acc));
}

/* GN+ summary, "Metal Compute Shaders": dequant mat-vec for gate and up, SwiGLU, dequant mat-vec
 * for down. silu(a) = a / (1 + exp(-a)). */
void oracle_expert(int64_t H, int64_t I, int64_t group, const double* x, const uint8_t* const q[3],
                   const uint16_t* const scale[3], const uint16_t* const bias[3], double* y, double* h_out) {
  double* Wg = (double*)malloc((size_t)(I * H) * sizeof(double));
  double* Wu = (double*)malloc((size_t)(I * H) * sizeof(double));
  double* Wd = (double*)malloc((size_t)(H * I) * sizeof(double));
  double* a = (double*)malloc((size_t)I * sizeof(double));
  double* c = (double*)malloc((size_t)I * sizeof(double));
  double* h = (double*)malloc((size_t)I * sizeof(double));
  oracle_dequant(I, H, group, q[0], scale[0], bias[0], Wg);
  oracle_dequant(I, H, group, q[1], scale[1], bias[1], Wu);
  oracle_dequant(H, I, group, q[2], scale[2], bias[2], Wd);
  oracle_matvec(I, H, Wg, x, a);
  oracle_matvec(I, H, Wu, x, c);
  for (int64_t i = 0; i < I; ++i) h[i] = a[i] / (1.0 + exp(-a[i])) * c[i];
  oracle_matvec(H, I, Wd, h, y);
  if (h_out) memcpy(h_out, h, (size_t)I * sizeof(double));
  free(Wg);
  free(Wu);
  free(Wd);
  free(a);
  free(c);
  free(h);
}

/* E2M1 (OCP MX element format for FP4): sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0.
 * Exponent 0 is subnormal: value = mantissa * 2^-1. Otherwise value = (1 + mantissa/2) * 2^(e - 1). */
static double e2m1_value(uint8_t q) {
  const int sign = (q >> 3) & 1, e = (q >> 1) & 3, m = q & 1;
  const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -v : v;
}

/* E8M0 (OCP MX scale format): 2^(s - 127), and 255 is NaN. */
static double e8m0_value(uint16_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* The page "300b on 32gb MoE-streaming findings + optimisations": MXFP4 experts. A block of 32
 * consecutive elements along a row shares one E8M0 scale. */
void oracle_dequant_mx(int64_t rows, int64_t cols, const uint8_t* q, const uint16_t* scale, double* W) {
  const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) W[r * cols + c] = e2m1_value(q[r * cols + c]) * e8m0_value(scale[r * nb + c / 32]);
}

void oracle_expert_mx(int64_t H, int64_t I, const double* x, const uint8_t* const q[3], const uint16_t* const scale[3],
                      double* y, double* h_out) {
  double* Wg = (double*)malloc((size_t)(I * H) * sizeof(double));
  double* Wu = (double*)malloc((size_t)(I * H) * sizeof(double));
  double* Wd = (double*)malloc((size_t)(H * I) * sizeof(double));
  double* a = (double*)malloc((size_t)I * sizeof(double));
  double* c = (double*)malloc((size_t)I * sizeof(double));
  double* h = (double*)malloc((size_t)I * sizeof(double));
  oracle_dequant_mx(I, H, q[0], scale[0], Wg);
  oracle_dequant_mx(I, H, q[1], scale[1], Wu);
  oracle_dequant_mx(H, I, q[2], scale[2], Wd);
  oracle_matvec(I, H, Wg, x, a);
  oracle_matvec(I, H, Wu, x, c);
  for (int64_t i = 0; i < I; ++i) h[i] = a[i] / (1.0 + exp(-a[i])) * c[i];
  oracle_matvec(H, I, Wd, h, y);
  if (h_out) memcpy(h_out, h, (size_t)I * sizeof(double));
  free(Wg);
  free(Wu);
  free(Wd);
  free(a);
  free(c);
  free(h);
}

/* GN+ summary, "Metal Compute Shaders" (MoE combine + residual + gate). */
void oracle_combine(int64_t H, int64_t K, const double* res, const double* y, const double* w, double g,
                    const double* ys, double* out) {
  for (int64_t r = 0; r < H; ++r) {
    double acc = res[r];
    for (int64_t k = 0; k < K; ++k) acc += w[k] * y[k * H + r];
    if (ys) acc += g * ys[r];
    out[r] = acc;
  }
}

/* GN+ summary, "Metal Compute Shaders" (RMS normalisation) and "Deferred GPU Expert Compute"
 * (combine + norm + residual feed the next layer). */
void oracle_rmsnorm(int64_t H, double eps, const double* h, double* u) {
  double ss = 0.0;
  for (int64_t j = 0; j < H; ++j) ss += h[j] * h[j];
  const double inv = 1.0 / sqrt(ss / (double)H + eps);
  for (int64_t j = 0; j < H; ++j) u[j] = h[j] * inv;
}
