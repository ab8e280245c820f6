/* moe.h — C ABI of the quantised Mixture-of-Experts expert-layer library for AMD MI355X (gfx950).
 *
 * The library computes one MoE layer per token, for the 397B, 512-expert, hidden-4096 model
 * described on the Flash-MoE pages:
 *   router GEMV -> softmax top-K -> group-affine 4-bit or 2-bit dequantised GEMVs for each
 *   selected expert's gate/up/down -> SwiGLU -> weighted combine with the sigmoid-gated
 *   shared expert and the residual.
 * Sources: GN+ summary "Flash-MoE - Ejecutar un modelo de 397 mil millones de parámetros en una
 * laptop" (es) and its (id) twin, sections "Arquitectura del modelo" and "Tecnologías clave"
 * (subsections "Kernel de dequantización optimizado con FMA", "Metal Compute Shaders" and
 * "Deferred GPU Expert Compute"); HN thread "Flash-MoE: Running a 397B Parameter Model on a
 * Laptop" (the router's result gates which experts are read).
 *
 * Conventions
 *  - Pointers named *_dev are device (HBM) pointers. The caller allocates and owns every buffer;
 *    the library never allocates or frees device memory, and every call runs all of its work on
 *    the caller's stream.
 *  - Calls that take a stream enqueue work on it (a hipStream_t; NULL means the default stream)
 *    and return at once. Results are valid once the stream has reached that point. No call
 *    synchronises the host, so calls can be captured into a HIP graph.
 *  - Return value: MOE_OK (0) or a negative MOE_E* code. Arguments are validated on the host
 *    before any HIP call, so a rejected call enqueues nothing. moe_last_error() gives a one-line
 *    reason (thread-local).
 *  - Dtypes: activations, residuals and outputs are fp32. Router and shared-gate weights are bf16
 *    (uint16 bit patterns). Expert weights live in packed blobs (format below).
 *  - Thread safety: concurrent calls on distinct streams are safe, except calls of
 *    moe_layer_forward_noalloc on one GPU, which share that GPU's scratch array.
 *
 * Packed expert blob (one expert = gate I x H, up I x H, down H x I; bits b in {2, 4}; group G):
 *   [gate codes][up codes][down codes][gate sb][up sb][down sb]
 *   - codes: row-major. Element c of a row is stored at byte c*b/8, at bit offset
 *     b*(c mod (8/b)), lowest bits first.
 *   - sb: one uint32 per (row, group) with row-major [rows][cols/G] order. The low half is the
 *     bf16 scale and the high half the bf16 bias.
 *   - A dequantised weight is W[r][c] = scale[r][c/G] * q[r][c] + bias[r][c/G]: the pages' form
 *     nibble*scale + bias ("Kernel de dequantización optimizado con FMA").
 *   - Size: 3*I*H*b/8 + 3*I*(H/G)*4 bytes, which is 7,077,888 B (6.75 MiB) at 4-bit and
 *     3,932,160 B at 2-bit for H = 4096, I = 1024.
 *
 * MXFP4 expert blob (bits 4, group 32): the expert format of the page "300b on 32gb MoE-streaming
 * findings + optimisations" (its summary), as the OCP Microscaling (MX) format defines it:
 *   [gate codes][up codes][down codes][gate scales][up scales][down scales]
 *   - codes: 4-bit E2M1 values (sign bit, 2 exponent bits with bias 1, 1 mantissa bit), packed as
 *     above (element c at byte c/2, lower nibble first).
 *   - scales: one E8M0 byte per (row, block of 32 columns), row-major [rows][cols/32]; 255 is NaN.
 *   - W[r][c] = e2m1(q[r][c]) * 2^(e[r][c/32] - 127); there is no bias.
 *   - Size: 3*I*H/2 + 3*I*H/32 bytes, 6,684,672 B for H = 4096, I = 1024.
 * In decode, a layer in this format computes exact fp32 products of the dequantised weights and
 * the fp32 activations. Its prefill (from MOE_PREFILL_MIN_TOKENS tokens, with inter >= 128) runs on
 * the scaled MX MFMA, with the activations expanded into three MXFP8 terms (E4M3 values with an
 * E8M0 scale per 32); below inter 128 the per-token kernels run at every T.
 */
#ifndef BQ_MOE_H
#define BQ_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null or misaligned pointer, bad sizes, expert index out of range */
#define MOE_EUNSUPPORTED (-2) /* a shape or format the library does not implement (see moe_layer_t) */
#define MOE_ENOSPC (-3)       /* workspace smaller than moe_workspace_bytes() */
#define MOE_EHIP (-4)         /* a HIP call or kernel launch failed */
#define MOE_ETIMEOUT (-5)     /* written to a device error word: the decode's first kernel gave up waiting */

#define MOE_MAX_TOP_K 8
#define MOE_MAX_EXPERTS 1024
/* Token counts at or above this run the prefill path in moe_layer_forward (grouped by expert). Below
 * it, per-token streaming is faster on MI355X (measured crossover: between 48 and 56 tokens for a
 * 512-expert, top-3, 4-bit layer; below 48 for the 2-bit and the top-6 MXFP4 layers). */
#define MOE_PREFILL_MIN_TOKENS 48
/* Token counts at or above this route all tokens in one fp64 router GEMM instead of per-token
 * router rows. */
#define MOE_ROUTER_BATCH_MIN_TOKENS 96
/* Token counts at or above this, when moe_router is not asked for the logits (and in
 * moe_layer_forward's prefill), take the certified router instead: bf16 MFMA logits with an error
 * bound, then fp64 for every row the bound cannot rule out (measured crossover with the fp64 GEMM
 * on a 512 x 4096 router: between 384 and 512 tokens). */
#define MOE_ROUTER_CERTIFIED_MIN_TOKENS 512

/* moe_layer_t.flags values, an A/B ablation of the one kernel claim on the pages ("Kernel de
 * dequantización optimizado con FMA"). By default the decode GEMVs use the per-chunk form
 * s * sum(q x) + b * sum(x). MOE_FLAG_DEQUANT_LITERAL computes every weight's term in the pages'
 * form fma(q, s*x, b*x); MOE_FLAG_DEQUANT_NAIVE in the form it replaced, (q*s + b)*x. Results
 * differ only by rounding. The prefill GEMMs ignore the flag. */
#define MOE_FLAG_DEQUANT_LITERAL 1
#define MOE_FLAG_DEQUANT_NAIVE 2
/* Single-token calls of moe_layer_forward run as two launches when the layer and the device allow it
 * (MOE_PLAN_PAIR, see moe_layer_plan); this flag makes them run as the three-kernel chain (router;
 * top-K + gate/up + SwiGLU; down + combine) instead. Both give the same results bit for bit. */
#define MOE_FLAG_DECODE_CHAIN 4

/* Workspace sync region. The first MOE_WS_SYNC_BYTES bytes of every workspace hold the cross-block
 * state of the two-launch decode (a call counter and the router logits tagged with it). They must
 * be zero before the first call that uses the workspace (allocate it zeroed, or call
 * moe_workspace_init once); calls keep them valid afterwards, and nothing else in the library writes there. A call
 * whose first kernel cannot have all of its blocks resident within about 20 ms writes NaN to its
 * output and marks the region; every later such call on that workspace then writes NaN until the
 * region is zeroed again. */
#define MOE_WS_SYNC_BYTES 32768

/* One MoE layer.
 *   hidden H, inter I: powers of two with 256 <= H <= 8192 and 64 <= I <= 2048. bits 2 or 4 with
 *   group 64 (affine format), or bits 4 with group 32 (MXFP4 format).
 *   n_experts E: 1..MOE_MAX_EXPERTS. top_k K: 1..min(E, MOE_MAX_TOP_K).
 *   experts_dev: E packed blobs, expert e at experts_dev + e*expert_stride. expert_stride is at
 *   least moe_blob_bytes(H, I, bits, group) and a multiple of 256.
 *   shared_blob_dev and shared_gate_dev: the shared expert's blob and its gate vector (bf16 [H]).
 *   Required when has_shared is 1, ignored when it is 0.
 *   router_dev: bf16 [E][H] row-major; logit e = row e . x, with no bias.
 *   flags: 0, MOE_FLAG_DEQUANT_LITERAL or MOE_FLAG_DEQUANT_NAIVE (the latter two affine only),
 *   optionally or'ed with MOE_FLAG_DECODE_CHAIN; other values: MOE_EUNSUPPORTED. */
typedef struct moe_layer_t {
  int32_t hidden;
  int32_t inter;
  int32_t n_experts;
  int32_t top_k;
  int32_t has_shared;
  int32_t bits;
  int32_t group;
  int32_t flags;
  const void* experts_dev;
  uint64_t expert_stride;
  const void* shared_blob_dev;
  const uint16_t* router_dev;
  const uint16_t* shared_gate_dev;
} moe_layer_t;

/* Canonical (unpacked) arrays of one expert, as host or device pointers. Matrix m = 0 gate, 1 up,
 * 2 down. q[m] holds one code per byte, row-major [rows][cols]. scale[m] and bias[m] are bf16
 * [rows][cols/G]. */
typedef struct moe_expert_arrays_t {
  const uint8_t* q[3];
  const uint16_t* scale[3];
  const uint16_t* bias[3];
} moe_expert_arrays_t;

/* ---- sizes -------------------------------------------------------------------------------------- */

/* Bytes of one packed expert blob, or 0 if the shape or format is unsupported. */
size_t moe_blob_bytes(int hidden, int inter, int bits, int group);

/* Workspace bytes that moe_router / moe_expert_ffn / moe_layer_forward need for T tokens
 * (and moe_stack_forward, which needs the same plus two [T][H] fp32 buffers). Returns 0 for an
 * invalid layer. */
size_t moe_workspace_bytes(const moe_layer_t* layer, int T);
size_t moe_stack_workspace_bytes(const moe_layer_t* layer, int T);

/* Zeroes a workspace's sync region (its first MOE_WS_SYNC_BYTES bytes) on `stream` with a fill
 * kernel (no memset node, so it may be captured in a graph): once before the first call on a
 * workspace that was not allocated zeroed, or to clear a region that a call marked.
 * ws_dev 256-byte aligned, ws_bytes >= MOE_WS_SYNC_BYTES (MOE_EINVAL, MOE_ENOSPC otherwise). */
int moe_workspace_init(void* ws_dev, size_t ws_bytes, void* stream);

/* ---- packing -------------------------------------------------------------------------------------- */

/* Pack one expert from canonical host arrays into a host blob of moe_blob_bytes() bytes.
 * Codes must be < 2^bits (MOE_EINVAL otherwise). For MXFP4 (group 32), scale[m] holds the E8M0
 * bytes as uint16 values <= 255 and bias may be NULL. Pure host code; usable without a GPU. */
int moe_pack_expert(int hidden, int inter, int bits, int group, const moe_expert_arrays_t* arrays_host,
                    void* blob_host);

/* As moe_pack_expert, but every array pointer and blob_dev are device pointers. The pack runs on
 * `stream`. arrays_dev itself (the struct) lives in host memory. */
int moe_pack_expert_device(int hidden, int inter, int bits, int group, const moe_expert_arrays_t* arrays_dev,
                           void* blob_dev, void* stream);

/* Dense dequantisation of one matrix (test export). expert -1 selects the shared expert, matrix is
 * 0 gate, 1 up, 2 down. out_dtype 0 writes fp32 [rows][cols]. out_dtype 1 writes the bf16
 * (round-to-nearest-even) of each weight. Every 2-bit and 4-bit weight in the supported ranges is
 * exact in fp32. The pages' form: nibble*scale + bias ("Kernel de dequantización optimizado con
 * FMA"); for MXFP4, e2m1(q) * 2^(e - 127). */
int moe_dequant(const moe_layer_t* layer, int expert, int matrix, int out_dtype, void* w_out_dev, void* stream);

/* ---- the layer, step by step --------------------------------------------------------------------- */

/* Router (HN thread: the router result decides which experts are read; GN+ "Arquitectura del modelo":
 * K routed experts per token plus the shared one).
 *   x_dev fp32 [T][H] -> idx_dev int32 [T][K] (descending logit, ties to the lower index),
 *   w_dev fp32 [T][K] (softmax over all E logits renormalised over the K chosen),
 *   shared_g_dev fp32 [T] (sigmoid(shared_gate . x); may be NULL; ignored if !has_shared),
 *   logits_dev fp64 [T][E] (may be NULL).
 * Logits are accumulated in fp64, so the top-K decision is exact up to fp64 rounding. From
 * MOE_ROUTER_CERTIFIED_MIN_TOKENS tokens with logits_dev NULL (and in moe_layer_forward's prefill), the
 * logits are first approximated on bf16 MFMAs and only the rows whose error bound overlaps the K-th
 * are recomputed in fp64; the choice is the same as the top-K of the fp64 logits. */
int moe_router(const moe_layer_t* layer, const float* x_dev, int T, int32_t* idx_dev, float* w_dev,
               float* shared_g_dev, double* logits_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* Expert FFNs ("Metal Compute Shaders": dequant mat-vec, SwiGLU; "Kernel de dequantización optimizado
 * con FMA"). For each token t and slot k < K, expert idx[t][k] computes
 *   y = W_down (silu(W_gate x) * (W_up x)),
 * and slot K is the shared expert when has_shared is 1.
 *   idx_dev int32 [T][K] (device). An entry outside [0, E) reads no weights (it never addresses
 *   memory outside the pool) and makes the call write NaN to that slot's output row.
 *   y_dev fp32 [T][K + has_shared][H]. */
int moe_expert_ffn(const moe_layer_t* layer, const float* x_dev, int T, const int32_t* idx_dev, float* y_dev,
                   void* ws_dev, size_t ws_bytes, void* stream);

/* moe_expert_ffn with a device error word: err_dev (int32, device, 4-byte aligned; may be NULL) is
 * set to MOE_EINVAL by the kernels when an index of idx_dev lies outside [0, E), and is otherwise
 * left untouched, so the caller clears it before the call and reads it after a stream sync. The
 * indices live on the device, so the host cannot check them without a sync; this is how a caller
 * whose indices come from its own GPU code learns that one was out of range. */
int moe_expert_ffn_checked(const moe_layer_t* layer, const float* x_dev, int T, const int32_t* idx_dev, float* y_dev,
                           void* ws_dev, size_t ws_bytes, int32_t* err_dev, void* stream);

/* Test export: the first stage of the certified router that moe_router (without a logits buffer)
 * and the prefill use from MOE_ROUTER_CERTIFIED_MIN_TOKENS tokens. The HN thread "Flash-MoE:
 * Running a 397B Parameter Model on a Laptop": the router's result decides which experts are read,
 * so the approximation only narrows the rows that are then recomputed exactly.
 * logits_dev fp64 [T][E+1]: column e < E receives router row e . x_t on bf16 MFMAs with each x
 * split into two bf16 terms; column E is not written. *kc_host (may be NULL) receives the factor
 * of the error bound the certified top-K relies on:
 *   |approx - exact| <= kc * |r_e| * |x_t| + (|r_e| + 1) * 2^-100,
 * |r_e| and |x_t| the Euclidean norms of router row e and token t. */
int moe_router_approx_logits(const moe_layer_t* layer, const float* x_dev, int T, double* logits_dev, double* kc_host,
                             void* stream);

/* Combine ("Metal Compute Shaders": MoE combine + residual + gate):
 *   out[t] = residual[t] + sum_k w[t][k] * y[t][k] + g[t] * y[t][K]   (shared term if has_shared)
 * y_dev fp32 [T][K + has_shared][H]; w_dev fp32 [T][K]; shared_g_dev fp32 [T] (NULL iff !has_shared). */
int moe_combine(const moe_layer_t* layer, const float* residual_dev, const float* y_dev, const float* w_dev,
                const float* shared_g_dev, int T, float* out_dev, void* stream);

/* ---- fused ------------------------------------------------------------------------------------- */

/* The whole layer: router -> top-K -> experts -> combine + residual, with out = residual + MoE(x).
 * T < MOE_PREFILL_MIN_TOKENS runs the decode path, in which each token streams its experts'
 * weights with GEMV kernels. Larger T runs the prefill path, which groups tokens by expert
 * ("Deferred GPU Expert Compute" is the one-stream, no-host-sync submission model both follow).
 * A single token (T = 1) runs as two launches where moe_layer_plan says so, else as three kernels.
 * idx_out_dev int32 [T][K] may be NULL. x_dev and out_dev may not alias; residual_dev may alias x_dev.
 * The workspace's first MOE_WS_SYNC_BYTES bytes must be zero before its first use (see there). */
int moe_layer_forward(const moe_layer_t* layer, const float* x_dev, const float* residual_dev, int T, float* out_dev,
                      int32_t* idx_out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* How moe_layer_forward runs T tokens of this layer on the current device: MOE_PLAN_PAIR (router,
 * top-K and gate/up + SwiGLU in one launch, then the down + combine kernel), MOE_PLAN_CHAIN (three
 * kernels per call), MOE_PLAN_PREFILL (tokens grouped by expert), or a negative error code. PAIR
 * takes T = 1 on layers with H = 4096, I = 1024, E <= 512 and a shared expert, either affine
 * (2- or 4-bit) at top_k 3 with the per-chunk dequant form or MXFP4 at top_k 6, without
 * MOE_FLAG_DECODE_CHAIN, on a device where all 256 blocks of 512 threads of its first kernel can be
 * resident at once. moe_stack_forward runs each layer of a single-token call the same way. The
 * answer is fixed for a layer and device. */
#define MOE_PLAN_PAIR 1
#define MOE_PLAN_CHAIN 2
#define MOE_PLAN_PREFILL 3
int moe_layer_plan(const moe_layer_t* layer, int T);

/* Instrumented moe_layer_forward, for timing kernels in place: the same kernels on `stream`. In
 * the PAIR plan the first launch takes events[0] and events[1], the down kernel events[4] and
 * events[5]. In the three-kernel decode
 * kernel p (0 router, 1 gate/up + SwiGLU of the routed and shared experts,
 * 2 down + combine) is launched with events[2p] and events[2p+1] as its start and stop events
 * (hipExtLaunchKernel). They then carry the dispatch's own begin and end timestamps, with no
 * extra packets in between. In the prefill path, events[0] and events[5] are recorded
 * (hipEventRecord) before and after all of its kernels. events is a host array of 6 hipEvent_t
 * created by the caller, and a NULL entry is skipped. Returns as moe_layer_forward. */
int moe_layer_forward_timed(const moe_layer_t* layer, const float* x_dev, const float* residual_dev, int T,
                            float* out_dev, int32_t* idx_out_dev, void* ws_dev, size_t ws_bytes, void* stream,
                            void* const* events);

/* moe_layer_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. It takes no workspace and allocates
 * nothing. Its workspace is a fixed device array of MOE_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends; the first call on a device looks up that device's
 * address. Same kernels and results as moe_layer_forward. A layer and T whose moe_workspace_bytes()
 * exceeds MOE_NOALLOC_SCRATCH_BYTES return MOE_ENOSPC before any HIP call. Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams, other threads) race;
 * calls in order on one stream are safe. Nothing in the array needs clearing between calls. A
 * decode call whose bounded wait gave up (MOE_ETIMEOUT) marks the array, and later calls on that
 * GPU write NaN outputs until the process ends: the caller has no handle to clear it. */
#define MOE_NOALLOC_SCRATCH_BYTES 33554432
int moe_layer_forward_noalloc(const moe_layer_t* layer, const float* x_dev, const float* residual_dev, int T,
                              float* out_dev, int32_t* idx_out_dev, void* stream);

/* A stack of L layers, decode only ("Deferred GPU Expert Compute": combine + norm + residual on the
 * GPU hand off to the next layer). With h_0 = x:
 *   u_l = h_l for l = 0, u_l = h_l / sqrt(mean(h_l^2) + eps) for l >= 1 (unit-weight RMS norm);
 *   h_{l+1} = h_l + MoE_l(u_l), where the router, experts and shared gate of layer l all read u_l.
 * out_dev = h_L, fp32 [T][H]. layers is a host array of L descriptors. All layers must share
 * H, I, E, K, bits, group, flags and has_shared (MOE_EINVAL otherwise, before any launch).
 * idx_out_dev int32 [L][T][K] may be NULL. */
int moe_stack_forward(const moe_layer_t* layers, int L, float eps, const float* x_dev, int T, float* out_dev,
                      int32_t* idx_out_dev, void* ws_dev, size_t ws_bytes, void* stream);

/* ---- errors ------------------------------------------------------------------------------------- */

const char* moe_strerror(int code);
/* Reason for the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BQ_MOE_H */
