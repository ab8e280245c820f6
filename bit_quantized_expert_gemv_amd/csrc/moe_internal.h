// Internal interface between the host entry points (moe_host.cpp) and the kernels (moe_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "moe.h"

// The token count from which moe_layer_forward and moe_expert_ffn take the prefill path (a build
// may set another value to time both paths at the same T).
#ifndef BQ_PREFILL_MIN
#define BQ_PREFILL_MIN MOE_PREFILL_MIN_TOKENS
#endif

namespace bqmoe {

// Shape and blob layout of one layer, validated on the host.
struct Geometry {
  int H, I, E, K, NE;  // NE = K + has_shared: expert slots per token
  int bits, G, has_shared;
  int form;               // decode GEMV arithmetic: 0 per-chunk x-sums, 1 fma(q, s*x, b*x), 2 (q*s + b)*x
  int chain;              // MOE_FLAG_DECODE_CHAIN: single tokens as the three-kernel chain
  uint64_t off_codes[3];  // byte offsets of gate / up / down codes inside a blob
  uint64_t off_sb[3];     // byte offsets of gate / up / down (scale, bias) words
  uint64_t blob_bytes;
};

struct LayerPtrs {
  const uint8_t* experts;
  uint64_t stride;
  const uint8_t* shared;
  const uint16_t* router;
  const uint16_t* sgate;
};

// Device workspace carved from the caller's buffer (per token t).
struct Workspace {
  double* logits;  // [T][E + 1]: router logits, then the shared-gate logit
  int32_t* idx;    // [T][K]
  float* w;        // [T][K]
  float* g;        // [T]
  float* h;        // [T][NE][I]: SwiGLU outputs
  float* u;        // [T][H]: normalised layer input (stack only)
  double* rnorm;   // [E]: router row norms (certified top-K only)
};

// Prefill (grouped) workspace for T tokens; N = T*K routed entries, R = N + T*has_shared rows.
struct PrefillWorkspace {
  Workspace layer;  // logits [T][E+1], idx [T][K], w [T][K], g [T]; h and u unused
  uint16_t* xq;     // [T][H] fp16 activations (each 8-block stored in the order 0,2,4,6,1,3,5,7)
  float* xs;        // [T][H/64] group sums of the fp16 activations (scaled, like xq)
  float* xu;        // [T] per-token power of two 2^-e that undoes the scaling of xq and xs
  int32_t* hist;    // [ceil(N/256)][E]
  int32_t* counts;  // [E]
  int32_t* offsets; // [E+1]
  int32_t* tile_e;  // [E + ceil(N/32)]
  int32_t* tile_first;
  int32_t* ntiles;  // [1]
  int32_t* pos;     // [N] entry -> position
  int32_t* perm;    // [N] position -> entry
  uint16_t* hq;     // [R][I] SwiGLU outputs in fp16 (same 8-block order as xq)
  float* hs;        // [R][I/64] group sums of the fp16 SwiGLU outputs, already scaled back
  float* hu;        // [R][I/64] per (row, group) power of two 2^-e that undoes the scaling of hq
  float* y;         // [R][H] down outputs
  // MXFP4 layers only (null otherwise): 3-term MXFP8 expansions of the activations and of the
  // SwiGLU outputs (term planes of E4M3 bytes, E8M0 scales per 32), and the fp32 SwiGLU outputs
  uint8_t* x8;      // [3][T][H]
  uint8_t* xsc;     // [3][T][H/32]
  float* h32;       // [R][I]
  uint8_t* h8;      // [3][R][I]
  uint8_t* hsc;     // [3][R][I/32]
};

bool geometry_from(const moe_layer_t* L, Geometry* g, const char** why);
size_t workspace_prefill_bytes(const Geometry& g, int T);
PrefillWorkspace carve_prefill(const Geometry& g, int T, void* base);
size_t workspace_layer_bytes(const Geometry& g, int T);
Workspace carve_workspace(const Geometry& g, int T, void* base);

// ---- launchers (moe_kernels.hip); all return hipSuccess or the launch error ----

// Optional start/stop events that a launch hands to the dispatch itself (hipExtLaunchKernel), so
// that they carry the kernel's own begin and end timestamps.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Phase 1: router logits and the shared-gate logit into ws.logits. If norm_src is non-null the layer
// input is RMSNorm(norm_src) with the given eps (also written to ws.u); otherwise the input is x.
hipError_t launch_router_phase(const Geometry& g, const LayerPtrs& p, const float* x, const float* norm_src,
                               float eps, int T, const Workspace& ws, hipStream_t s, const KernelEvents& ev = {});
// Phase 2: gate/up SwiGLU of the routed experts (slots 0..K-1), plus slot K (shared) if with_shared.
// If idx_in is null the top-K is computed from ws.logits and written to ws.idx/w/g (and idx_out). A
// caller's index outside [0, E) makes that slot's h NaN (nothing is read) and, if err is non-null,
// stores MOE_EINVAL to *err.
hipError_t launch_gateup(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                         const int32_t* idx_in, int32_t* idx_out, bool with_shared, int32_t* err, hipStream_t s,
                         const KernelEvents& ev = {});
// Phase 3: down projections. combine: out = residual + sum_k w_k y_k + g y_s; otherwise y[t][k][:] = y_k.
hipError_t launch_down(const Geometry& g, const LayerPtrs& p, int T, const Workspace& ws, const int32_t* idx,
                       const float* residual, float* out, float* y, hipStream_t s, const KernelEvents& ev = {});
// Certified top-K (many tokens, no logits output): ws.logits must hold approximate logits whose
// error is at most kc * |r_e| * |x_t| (plus a subnormal slack); computes the router row norms into
// ws.rnorm, recomputes in fp64 the rows the bound cannot rule out, and writes idx, w and sg.
hipError_t launch_topk_certified(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                 double kc, int32_t* idx, float* w, float* sg, int32_t* idx_b, hipStream_t s);
// The certified router's first stage: approximate logits (bf16 MFMAs, x split into two bf16 terms)
// into logits [T][E+1] (column E untouched), and in *kc the factor of their error bound
// |approx - exact| <= kc |r_e| |x_t| + (|r_e| + 1) 2^-100.
hipError_t launch_router_approx(const Geometry& g, const LayerPtrs& p, const float* x, int T, double* logits,
                                double* kc, hipStream_t s);
// Routing of T tokens into idx/w/sg (and the fp64 logits into logits_out, a copy of idx into idx_b,
// each when non-null): the certified bf16-MFMA path for many tokens without logits_out, otherwise
// fp64 logits then the top-K.
hipError_t launch_router_select(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                int32_t* idx, float* w, float* sg, double* logits_out, int32_t* idx_b,
                                hipStream_t s);
// The two-launch decode of one token: whether this layer and the current device take it, and the
// launches (router, top-K and gate/up + SwiGLU in one kernel, then the down + combine kernel). sync
// is the workspace's zero-initialised sync region of MOE_WS_SYNC_BYTES; err (optional, device)
// receives MOE_ETIMEOUT if the first kernel gives up waiting for its blocks.
// With norm_src non-null (the stack's layers after the first) the layer input is RMSNorm(norm_src)
// with eps, computed as kernel 1 does; otherwise it is x.
bool pair_supported(const Geometry& g);
hipError_t launch_pair(const Geometry& g, const LayerPtrs& p, const float* x, const float* norm_src, float eps,
                       const float* residual, float* out, int32_t* idx_out, const Workspace& ws, uint8_t* sync,
                       int32_t* err, hipStream_t s, const KernelEvents& ev_front = {},
                       const KernelEvents& ev_down = {});
// Top-K + weights from ws.logits (router-only path); idx_b, if non-null, receives a copy of idx.
hipError_t launch_topk(const Geometry& g, int T, const Workspace& ws, int32_t* idx, float* w, float* sg,
                       double* logits_out, int32_t* idx_b, hipStream_t s);
hipError_t launch_combine(const Geometry& g, int T, const float* residual, const float* y, const float* w,
                          const float* sg, float* out, hipStream_t s);
// Device address of the no-allocation entry point's scratch array (MOE_NOALLOC_SCRATCH_BYTES) on
// the current device, looked up on the first call per device and cached.
hipError_t noalloc_scratch(void** out);
// Zeroes n bytes (a multiple of 16, 16-byte aligned) at p with a fill kernel.
hipError_t launch_zero(void* p, size_t n, hipStream_t s);
hipError_t launch_dequant(const Geometry& g, const uint8_t* blob, int matrix, int out_dtype, void* out, hipStream_t s);
hipError_t launch_pack(int H, int I, int bits, int G, const moe_expert_arrays_t* a, uint8_t* blob, hipStream_t s);

// Prefill (moe_prefill.hip). With idx_in null the router runs first (fp64 GEMM + top-K). Then come
// grouping, the grouped gate/up and down GEMMs, and either out = residual + combine (out non-null) or
// y_out[t][k][:] = expert outputs (y_out non-null).
hipError_t launch_prefill(const Geometry& g, const LayerPtrs& p, const float* x, const float* residual, int T,
                          const PrefillWorkspace& w, const int32_t* idx_in, int32_t* idx_out, float* out,
                          float* y_out, int32_t* err, hipStream_t s);
// Router logits of T tokens into ws.logits: the fp64 MFMA GEMM for many tokens, per-token router
// rows (phase 1) for few.
hipError_t launch_router_tokens(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                hipStream_t s);
// Router logits of T tokens as one fp64 GEMM into ws.logits.
hipError_t launch_router_gemm(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                              hipStream_t s);

}  // namespace bqmoe
