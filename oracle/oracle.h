/* ORACLE — test infrastructure only.
 *
 * A plain, slow, fp64 CPU reference for the quantised Mixture-of-Experts layer: router ->
 * softmax top-K -> group-affine dequantisation -> SwiGLU experts -> weighted combine with the
 * sigmoid-gated shared expert and the residual. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the GPU library never does, and the two share no code.
 *
 * Sources (the Flash-MoE pages):
 *  - GN+ summary "Flash-MoE - Ejecutar un modelo de 397 mil millones de parámetros en una laptop"
 *    (es) / "Flash-MoE - Menjalankan model 397 miliar parameter di laptop" (id):
 *      "Arquitectura del modelo": 512 experts per layer, K=4 active per token including one shared
 *        expert, hidden size 4096, 60 layers;
 *      "Tecnologías clave > Kernel de dequantización optimizado con FMA": a weight is
 *        nibble*scale + bias and multiplies the activation;
 *      "Tecnologías clave > Metal Compute Shaders": 4-bit/2-bit dequant mat-vec, SwiGLU, RMS norm,
 *        MoE combine + residual + gate;
 *      "Tecnologías clave > Deferred GPU Expert Compute": combine + norm + residual hand off to the
 *        next layer.
 *  - HN thread "Flash-MoE: Running a 397B Parameter Model on a Laptop": expert loads start once
 *    the router result is in (the reads are gated by the router's top-K choice).
 * Readings where the pages are silent (router has no bias; ties go to the lower index; softmax
 * over all experts then renormalised over the K chosen; g = sigmoid(shared-gate . x); SwiGLU is
 * silu(gate)*up; RMS norm has unit weight) are stated at each function.
 *
 * Precision: every value is widened exactly to double (bf16 and fp32 are subsets of double) and
 * every sum is a plain left-to-right double sum. Nothing is blocked, fused or reordered.
 * Parity pins: every function is pinned by tests/test_oracle.py (brute force, closed forms,
 * invariants, textbook routines); none is "parity unpinned".
 */
#ifndef BQ_ORACLE_H
#define BQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* W[r][c] = scale[r][c/group] * q[r][c] + bias[r][c/group], dense, rows x cols, fp64. */
void oracle_dequant(int64_t rows, int64_t cols, int64_t group, const uint8_t* q, const uint16_t* scale,
                    const uint16_t* bias, double* W);
/* out[r] = sum_c W[r][c] * v[c]. */
void oracle_matvec(int64_t rows, int64_t cols, const double* W, const double* v, double* out);
/* logits[e] = sum_j R[e][j] * x[j]; R is bf16 [E][H]. No bias term. */
void oracle_router_logits(int64_t E, int64_t H, const uint16_t* R, const double* x, double* logits);
/* The K largest logits, by a full sort on (logit descending, expert index ascending). */
void oracle_topk(int64_t E, int64_t K, const double* logits, int32_t* idx);
/* p = softmax over all E logits; w[k] = p[idx[k]] / sum_k' p[idx[k']]. */
void oracle_route_weights(int64_t E, int64_t K, const double* logits, const int32_t* idx, double* w);
/* g = 1 / (1 + exp(-(sum_j gs[j] * x[j]))); gs is bf16 [H]. */
double oracle_shared_gate(int64_t H, const uint16_t* gs, const double* x);
/* One expert: a = Wg x, c = Wu x, h = silu(a) * c, y = Wd h. Wg, Wu are I x H; Wd is H x I.
 * q/scale/bias point to the canonical arrays of gate, up, down (index 0, 1, 2). h_out may be NULL. */
void oracle_expert(int64_t H, int64_t I, int64_t group, const double* x, const uint8_t* const q[3],
                   const uint16_t* const scale[3], const uint16_t* const bias[3], double* y, double* h_out);
/* MXFP4 experts (the page "300b on 32gb MoE-streaming findings + optimisations", its summary: the
 * expert pool is stored as MXFP4; the format is read as the OCP Microscaling specification defines
 * MXFP4). q holds one E2M1 code per byte (sign bit 3, exponent bits 2-1 with bias 1, mantissa bit 0;
 * exponent 0 is subnormal, value mantissa/2); scale holds one E8M0 byte per (row, block of 32
 * columns) in uint16 slots, value 2^(s - 127), with 255 meaning NaN. There is no bias.
 * W[r][c] = e2m1(q[r][c]) * 2^(scale[r][c/32] - 127), dense, rows x cols, fp64 (exact). */
void oracle_dequant_mx(int64_t rows, int64_t cols, const uint8_t* q, const uint16_t* scale, double* W);
/* One MXFP4 expert: as oracle_expert with oracle_dequant_mx weights. */
void oracle_expert_mx(int64_t H, int64_t I, const double* x, const uint8_t* const q[3], const uint16_t* const scale[3],
                      double* y, double* h_out);
/* out = res + sum_k w[k] * y[k] + g * ys (the shared term only when ys != NULL); y is K x H. */
void oracle_combine(int64_t H, int64_t K, const double* res, const double* y, const double* w, double g,
                    const double* ys, double* out);
/* u = h / sqrt(mean(h^2) + eps) (unit weight). */
void oracle_rmsnorm(int64_t H, double eps, const double* h, double* u);

#ifdef __cplusplus
}
#endif
#endif
