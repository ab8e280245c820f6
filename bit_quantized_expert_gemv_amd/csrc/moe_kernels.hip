// Decode-path kernels of the quantised MoE layer for MI355X (gfx950, wave64).
//
// One token's layer runs as three stream-ordered kernels; nothing synchronises the host.
//   1. router phase: the router logits and the shared-gate logit (fp64 accumulation), plus the
//      shared expert's gate/up/SwiGLU, which does not depend on the routing;
//   2. gate/up: each block picks the top-K itself from the logits, then runs gate/up/SwiGLU
//      for the K routed experts;
//   3. down: the down projections of all K+1 experts, combined with the routing weights, the
//      shared gate and the residual. Each output row sums all experts, so the result is a
//      deterministic gather with no atomics.
// GN+ summary "Flash-MoE - Ejecutar un modelo de 397 mil millones de parámetros en una laptop",
// "Tecnologías clave": "Metal Compute Shaders" lists these operations; "Deferred GPU Expert
// Compute" submits them without a host round trip; combine + norm + residual stay on the GPU.
//
// Dequantised mat-vec. The pages rewrite (nibble*scale + bias)*x as fma(nibble, scale*x, bias*x)
// ("Kernel de dequantización optimizado con FMA"). Here the bias term leaves the inner loop
// instead: per 16-byte chunk of codes (half a group at 4-bit, one group at 2-bit)
//   sum_j (s q_j + b) x_j = s * sum_j q_j x_j + b * S,   S = sum_j x_j,
// so the inner loop is one FMA per weight and the bias costs one FMA per chunk. Codes are
// widened without masking each one: a 4-bit code in a byte is an OCP e4m3 subnormal-range value,
// q * 2^-9, which v_cvt_pk_f32_fp8 converts two at a time. A 2-bit code in a nibble is an e2m1
// value, q/2, which v_cvt_scalef32_pk_f32_fp4 (scale 2) converts two at a time. Both widenings
// are exact, and the 2^-9 is folded into the group scale.
//
// Lane layout. A row is split into 16-byte chunks. LPR lanes share a row, and lane i of the row
// owns chunks i, i+LPR, ..., so each wave-wide load is contiguous. A lane keeps the activations
// of its own columns in registers for every row it processes. Rows are reduced across their LPR
// lanes with butterfly shuffles, which give every lane the bitwise-same sum.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "moe_internal.h"

namespace bqmoe {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / 64;

// Lane layout of a row of COLS codes at BITS bits (16-byte chunks).
template <int BITS, int COLS>
struct RowCfg {
  static constexpr int CH = 128 / BITS;                  // codes per chunk
  static constexpr int NC = COLS / CH;                   // chunks per row
  static constexpr int LPR = NC < 64 ? NC : 64;          // lanes per row
  static constexpr int CPL = NC / LPR;                   // chunks per lane
  static constexpr int RPW = 64 / LPR;                   // rows per wave step
  static constexpr int XPL = CPL * CH;                   // activations per lane
  static constexpr int ROW_BYTES = COLS * BITS / 8;
  static constexpr int GROUPS = COLS / 64;
  static_assert(NC >= 1 && NC % LPR == 0, "unsupported row length");
};

// Lane layout of a bf16 router row of COLS elements (8 per 16-byte chunk).
template <int COLS>
struct RouterCfg {
  static constexpr int NC = COLS / 8;
  static constexpr int LPR = NC < 64 ? NC : 64;
  static constexpr int CPL = NC / LPR;
  static constexpr int RPW = 64 / LPR;
  static constexpr int XPL = CPL * 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// sum_j q_j x_j * 2^-9 over 32 4-bit codes (chunk element order; byte k holds elements 2k, 2k+1)
__device__ __forceinline__ float chunk_dot4(const uint4 w, const float* x) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ws[i] & 0x0F0F0F0Fu;          // elements 8i+0, +2, +4, +6
    const uint32_t hi = (ws[i] >> 4) & 0x0F0F0F0Fu;   // elements 8i+1, +3, +5, +7
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    acc = fmaf(a[0], x[8 * i + 0], acc);
    acc = fmaf(c[0], x[8 * i + 1], acc);
    acc = fmaf(a[1], x[8 * i + 2], acc);
    acc = fmaf(c[1], x[8 * i + 3], acc);
    acc = fmaf(b[0], x[8 * i + 4], acc);
    acc = fmaf(d[0], x[8 * i + 5], acc);
    acc = fmaf(b[1], x[8 * i + 6], acc);
    acc = fmaf(d[1], x[8 * i + 7], acc);
  }
  return acc;
}

// byte N of lo/hi: elements 4N, 4N+2 (lo) and 4N+1, 4N+3 (hi) of a 16-code word
template <int N>
__device__ __forceinline__ float dot2_byte(uint32_t lo, uint32_t hi, const float* x, float acc) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 2.0f, N);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 2.0f, N);
  acc = fmaf(a[0], x[4 * N + 0], acc);
  acc = fmaf(c[0], x[4 * N + 1], acc);
  acc = fmaf(a[1], x[4 * N + 2], acc);
  acc = fmaf(c[1], x[4 * N + 3], acc);
  return acc;
}

// sum_j q_j x_j over 64 2-bit codes (byte k holds elements 4k..4k+3, lowest bits first)
__device__ __forceinline__ float chunk_dot2(const uint4 w, const float* x) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ws[i] & 0x33333333u;          // nibble n: element 16i + 2n
    const uint32_t hi = (ws[i] >> 2) & 0x33333333u;   // nibble n: element 16i + 2n + 1
    acc = dot2_byte<0>(lo, hi, x + 16 * i, acc);
    acc = dot2_byte<1>(lo, hi, x + 16 * i, acc);
    acc = dot2_byte<2>(lo, hi, x + 16 * i, acc);
    acc = dot2_byte<3>(lo, hi, x + 16 * i, acc);
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float* x) {
  if constexpr (BITS == 4) return chunk_dot4(w, x);
  else return chunk_dot2(w, x);
}

// This lane's share of one row: sum over its chunks of s * sum(q x) + b * S.
template <int BITS, class C>
__device__ __forceinline__ float row_partial(const uint4 (&cw)[C::CPL], const uint32_t (&sb)[C::CPL],
                                             const float (&xr)[C::XPL], const float (&S)[C::CPL]) {
  constexpr float kCvt = BITS == 4 ? 512.0f : 1.0f;  // undo the e4m3 2^-9
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const float d = chunk_dot<BITS>(cw[j], &xr[j * C::CH]);
    a = fmaf(bf16_lo(sb[j]) * kCvt, d, fmaf(bf16_hi(sb[j]), S[j], a));
  }
  return a;
}

// Load this lane's activations (scaled) and their per-chunk sums.
template <class C>
__device__ __forceinline__ void load_act(const float* __restrict__ v, int lir, float scale, float (&xr)[C::XPL],
                                         float (&S)[C::CPL]) {
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const float4* p = reinterpret_cast<const float4*>(v + (lir + j * C::LPR) * C::CH);
#pragma unroll
    for (int q = 0; q < C::CH / 4; ++q) {
      const float4 t = p[q];
      xr[j * C::CH + 4 * q + 0] = t.x * scale;
      xr[j * C::CH + 4 * q + 1] = t.y * scale;
      xr[j * C::CH + 4 * q + 2] = t.z * scale;
      xr[j * C::CH + 4 * q + 3] = t.w * scale;
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < C::CH; ++i) s += xr[j * C::CH + i];
    S[j] = s;
  }
}

template <class C>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ codes, const uint32_t* __restrict__ sbp, int r,
                                         int lir, uint4 (&cw)[C::CPL], uint32_t (&sb)[C::CPL]) {
  const uint8_t* row = codes + (size_t)r * C::ROW_BYTES;
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const int c = lir + j * C::LPR;
    cw[j] = *reinterpret_cast<const uint4*>(row + (size_t)c * 16);
    sb[j] = sbp[(size_t)r * C::GROUPS + (c * C::CH) / 64];
  }
}

template <int LPR, class T>
__device__ __forceinline__ T seg_sum(T v) {
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float silu_mul(float a, float c) { return a / (1.0f + expf(-a)) * c; }

struct LayerArgs {
  int H, I, E, K, NE, has_shared;
  uint64_t off_codes[3], off_sb[3];
  const uint8_t* experts;
  uint64_t stride;
  const uint8_t* shared;
  const uint16_t* router;
  const uint16_t* sgate;
  Workspace ws;
};

LayerArgs make_args(const Geometry& g, const LayerPtrs& p, const Workspace& ws) {
  LayerArgs a;
  a.H = g.H; a.I = g.I; a.E = g.E; a.K = g.K; a.NE = g.NE; a.has_shared = g.has_shared;
  for (int m = 0; m < 3; ++m) { a.off_codes[m] = g.off_codes[m]; a.off_sb[m] = g.off_sb[m]; }
  a.experts = p.experts; a.stride = p.stride; a.shared = p.shared; a.router = p.router; a.sgate = p.sgate;
  a.ws = ws;
  return a;
}

// gate/up/SwiGLU for P row steps of one expert; writes h rows (lane 0 of each row).
template <int BITS, int COLS, int P>
__device__ __forceinline__ void gateup_rows(const LayerArgs& a, const uint8_t* __restrict__ blob,
                                            const float (&xr)[RowCfg<BITS, COLS>::XPL],
                                            const float (&S)[RowCfg<BITS, COLS>::CPL], int lir, int rig, int step0,
                                            float* __restrict__ h) {
  using C = RowCfg<BITS, COLS>;
  const uint8_t* gc = blob + a.off_codes[0];
  const uint8_t* uc = blob + a.off_codes[1];
  const uint32_t* gs = reinterpret_cast<const uint32_t*>(blob + a.off_sb[0]);
  const uint32_t* us = reinterpret_cast<const uint32_t*>(blob + a.off_sb[1]);
  uint4 cg[P][C::CPL], cu[P][C::CPL];
  uint32_t sg[P][C::CPL], su[P][C::CPL];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = (step0 + p) * C::RPW + rig;
    if (r < a.I) {
      load_row<C>(gc, gs, r, lir, cg[p], sg[p]);
      load_row<C>(uc, us, r, lir, cu[p], su[p]);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = (step0 + p) * C::RPW + rig;
    if (r < a.I) {
      const float ga = seg_sum<C::LPR>(row_partial<BITS, C>(cg[p], sg[p], xr, S));
      const float ua = seg_sum<C::LPR>(row_partial<BITS, C>(cu[p], su[p], xr, S));
      if (lir == 0) h[r] = silu_mul(ga, ua);
    }
  }
}

// Wave-wide top-K over logits[0..E): descending value, ties to the lower index. Result is wave-uniform.
__device__ __forceinline__ void wave_topk(const double* __restrict__ logits, int E, int K, int lane, int32_t* sel,
                                          double* val) {
  double v[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? logits[e] : -INFINITY;
  }
  for (int k = 0; k < K; ++k) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + 64 * i;
      if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel[k] = bi;
    val[k] = bv;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (lane + 64 * i == bi) v[i] = -INFINITY;
  }
}

// Softmax of the K chosen logits (the full softmax over E renormalised over the chosen set reduces to this).
__device__ __forceinline__ void route_weights(const double* val, int K, float* w) {
  double z = 0.0;
  for (int k = 0; k < K; ++k) z += exp(val[k] - val[0]);
  for (int k = 0; k < K; ++k) w[k] = (float)(exp(val[k] - val[0]) / z);
}

// RMS norm scale of h (fp64 accumulation, one fixed order for every block).
__device__ float block_rms_inv(const float* __restrict__ h, int H, float eps, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += kBlock) ss += (double)h[i] * (double)h[i];
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int s = kBlock / 2; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double tot = red[0];
  __syncthreads();
  return (float)(1.0 / sqrt(tot / (double)H + (double)eps));
}

// ---------------------------------------------------------------------------------------------
// Kernel 1: router logits (+ shared-gate logit) and the shared expert's gate/up.
// Blocks [0, n_router_blocks) do router rows (row E is the shared-gate vector); the rest do the
// shared expert's gate/up rows.
template <int BITS, int H, int P>
__global__ __launch_bounds__(kBlock) void k_router_phase(LayerArgs a, const float* __restrict__ x,
                                                         const float* __restrict__ norm_src, float eps,
                                                         int n_router_blocks, int router_steps) {
  using C = RowCfg<BITS, H>;
  using R = RouterCfg<H>;
  __shared__ double red[kBlock];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float scale = 1.0f;
  const float* src = x + (size_t)t * H;
  if (norm_src != nullptr) {
    src = norm_src + (size_t)t * H;
    scale = block_rms_inv(src, H, eps, red);
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < H; i += kBlock) a.ws.u[(size_t)t * H + i] = src[i] * scale;
  }
  if ((int)blockIdx.x < n_router_blocks) {
    const int lir = lane % R::LPR, rig = lane / R::LPR;
    float xr[R::XPL];
#pragma unroll
    for (int j = 0; j < R::CPL; ++j) {
      const float4* p = reinterpret_cast<const float4*>(src + (lir + j * R::LPR) * 8);
      const float4 u0 = p[0], u1 = p[1];
      xr[j * 8 + 0] = u0.x * scale; xr[j * 8 + 1] = u0.y * scale; xr[j * 8 + 2] = u0.z * scale;
      xr[j * 8 + 3] = u0.w * scale; xr[j * 8 + 4] = u1.x * scale; xr[j * 8 + 5] = u1.y * scale;
      xr[j * 8 + 6] = u1.z * scale; xr[j * 8 + 7] = u1.w * scale;
    }
    const int nrows = a.E + a.has_shared;
    for (int s = 0; s < router_steps; ++s) {
      const int r = ((blockIdx.x * kWaves + wave) * router_steps + s) * R::RPW + rig;
      if (r >= nrows) break;  // uniform across the LPR lanes of a row
      const uint16_t* row = (r < a.E) ? a.router + (size_t)r * H : a.sgate;
      uint4 w[R::CPL];
#pragma unroll
      for (int j = 0; j < R::CPL; ++j) w[j] = *reinterpret_cast<const uint4*>(row + (lir + j * R::LPR) * 8);
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < R::CPL; ++j) {
        const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = fma((double)bf16_lo(ww[q]), (double)xr[j * 8 + 2 * q], acc);
          acc = fma((double)bf16_hi(ww[q]), (double)xr[j * 8 + 2 * q + 1], acc);
        }
      }
      acc = seg_sum<R::LPR>(acc);
      if (lir == 0) a.ws.logits[(size_t)t * (a.E + 1) + r] = acc;
    }
    return;
  }
  // shared expert gate/up
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  float xr[C::XPL], S[C::CPL];
  load_act<C>(src, lir, scale, xr, S);
  const int step0 = ((blockIdx.x - n_router_blocks) * kWaves + wave) * P;
  gateup_rows<BITS, H, P>(a, a.shared, xr, S, lir, rig, step0, a.ws.h + ((size_t)t * a.NE + a.K) * a.I);
}

// Kernel 2: gate/up/SwiGLU of routed experts (blockIdx.y = slot; slot K = shared when included).
template <int BITS, int H, int P>
__global__ __launch_bounds__(kBlock) void k_gateup(LayerArgs a, const float* __restrict__ x,
                                                   const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out) {
  using C = RowCfg<BITS, H>;
  const int t = blockIdx.z, slot = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  const uint8_t* blob;
  if (slot < a.K) {
    int e;
    if (idx_in != nullptr) {
      e = idx_in[(size_t)t * a.K + slot];
    } else {
      int32_t sel[MOE_MAX_TOP_K];
      double val[MOE_MAX_TOP_K];
      wave_topk(a.ws.logits + (size_t)t * (a.E + 1), a.E, a.K, lane, sel, val);
      e = sel[slot];
      if (blockIdx.x == 0 && blockIdx.y == 0 && wave == 0 && lane == 0) {
        float w[MOE_MAX_TOP_K];
        route_weights(val, a.K, w);
        for (int k = 0; k < a.K; ++k) {
          a.ws.idx[(size_t)t * a.K + k] = sel[k];
          a.ws.w[(size_t)t * a.K + k] = w[k];
          if (idx_out) idx_out[(size_t)t * a.K + k] = sel[k];
        }
        if (a.has_shared) a.ws.g[t] = (float)(1.0 / (1.0 + exp(-a.ws.logits[(size_t)t * (a.E + 1) + a.E])));
      }
    }
    if (e < 0 || e >= a.E) {  // never read outside the pool: mark the slot's output as invalid
      const int step0 = (blockIdx.x * kWaves + wave) * P;
      for (int p = 0; p < P; ++p) {
        const int r = (step0 + p) * C::RPW + rig;
        if (r < a.I && lir == 0) a.ws.h[((size_t)t * a.NE + slot) * a.I + r] = NAN;
      }
      return;
    }
    blob = a.experts + (size_t)e * a.stride;
  } else {
    blob = a.shared;
  }
  float xr[C::XPL], S[C::CPL];
  load_act<C>(x + (size_t)t * H, lir, 1.0f, xr, S);
  const int step0 = (blockIdx.x * kWaves + wave) * P;
  gateup_rows<BITS, H, P>(a, blob, xr, S, lir, rig, step0, a.ws.h + ((size_t)t * a.NE + slot) * a.I);
}

// Kernel 3: down projections of all expert slots for a block of output rows; combine or store.
template <int BITS, int I, int P>
__global__ __launch_bounds__(kBlock) void k_down(LayerArgs a, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ residual, float* __restrict__ out,
                                                 float* __restrict__ y) {
  using C = RowCfg<BITS, I>;
  constexpr int RB = C::RPW * P;
  __shared__ float part[kWaves][RB];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  const int row0 = blockIdx.x * RB;
  const bool combine = out != nullptr;
  bool first = true;
  for (int k = wave; k < a.NE; k += kWaves) {
    const uint8_t* blob;
    float coef = 1.0f;
    bool valid = true;
    if (k < a.K) {
      const int e = idx[(size_t)t * a.K + k];
      valid = (e >= 0 && e < a.E);
      blob = a.experts + (size_t)(valid ? e : 0) * a.stride;
      if (combine) coef = a.ws.w[(size_t)t * a.K + k];
    } else {
      blob = a.shared;
      if (combine) coef = a.ws.g[t];
    }
    float yv[P];
    if (valid) {
      float xr[C::XPL], S[C::CPL];
      load_act<C>(a.ws.h + ((size_t)t * a.NE + k) * I, lir, 1.0f, xr, S);
      const uint8_t* dc = blob + a.off_codes[2];
      const uint32_t* ds = reinterpret_cast<const uint32_t*>(blob + a.off_sb[2]);
      uint4 cw[P][C::CPL];
      uint32_t sb[P][C::CPL];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int r = row0 + p * C::RPW + rig;
        if (r < a.H) load_row<C>(dc, ds, r, lir, cw[p], sb[p]);
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int r = row0 + p * C::RPW + rig;
        yv[p] = (r < a.H) ? seg_sum<C::LPR>(row_partial<BITS, C>(cw[p], sb[p], xr, S)) : 0.0f;
      }
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) yv[p] = NAN;
    }
    if (lir == 0) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int r = row0 + p * C::RPW + rig;
        if (r >= a.H) continue;
        if (combine) {
          const float v = coef * yv[p];
          part[wave][p * C::RPW + rig] = first ? v : part[wave][p * C::RPW + rig] + v;
        } else {
          y[((size_t)t * a.NE + k) * a.H + r] = yv[p];
        }
      }
    }
    first = false;
  }
  if (!combine) return;
  __syncthreads();
  for (int i = threadIdx.x; i < RB; i += kBlock) {
    const int r = row0 + i;
    if (r >= a.H) continue;
    float acc = residual[(size_t)t * a.H + r];
    for (int w = 0; w < kWaves && w < a.NE; ++w) acc += part[w][i];
    out[(size_t)t * a.H + r] = acc;
  }
}

// Router-only top-K: one wave per token.
__global__ __launch_bounds__(64) void k_topk(LayerArgs a, int32_t* __restrict__ idx, float* __restrict__ w,
                                             float* __restrict__ sg, double* __restrict__ logits_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const double* lg = a.ws.logits + (size_t)t * (a.E + 1);
  int32_t sel[MOE_MAX_TOP_K];
  double val[MOE_MAX_TOP_K];
  wave_topk(lg, a.E, a.K, lane, sel, val);
  if (logits_out)
    for (int e = lane; e < a.E; e += 64) logits_out[(size_t)t * a.E + e] = lg[e];
  if (lane == 0) {
    float ww[MOE_MAX_TOP_K];
    route_weights(val, a.K, ww);
    for (int k = 0; k < a.K; ++k) {
      idx[(size_t)t * a.K + k] = sel[k];
      w[(size_t)t * a.K + k] = ww[k];
    }
    if (sg && a.has_shared) sg[t] = (float)(1.0 / (1.0 + exp(-lg[a.E])));
  }
}

__global__ void k_combine(int T, int H, int K, int has_shared, const float* __restrict__ res,
                          const float* __restrict__ y, const float* __restrict__ w, const float* __restrict__ sg,
                          float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * H) return;
  const int64_t t = i / H, r = i % H;
  const int NE = K + has_shared;
  float acc = res[i];
  for (int k = 0; k < K; ++k) acc += w[t * K + k] * y[(t * NE + k) * H + r];
  if (has_shared) acc += sg[t] * y[(t * NE + K) * H + r];
  out[i] = acc;
}

__global__ void k_dequant(int rows, int cols, int bits, const uint8_t* __restrict__ codes,
                          const uint32_t* __restrict__ sb, int out_dtype, void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * cols) return;
  const int64_t r = i / cols, c = i % cols;
  const int per = 8 / bits;
  const uint32_t q = (codes[(r * cols + c) / per] >> (bits * (int)(c % per))) & ((1u << bits) - 1u);
  const uint32_t p = sb[r * (cols / 64) + c / 64];
  const float v = fmaf(bf16_lo(p), (float)q, bf16_hi(p));  // exact for the supported ranges
  if (out_dtype == 0) {
    static_cast<float*>(out)[i] = v;
  } else {
    uint32_t b = __float_as_uint(v);
    b += 0x7FFFu + ((b >> 16) & 1u);  // round to nearest even (finite values)
    static_cast<uint16_t*>(out)[i] = (uint16_t)(b >> 16);
  }
}

__global__ void k_pack_codes(int64_t nbytes_out, int bits, const uint8_t* __restrict__ q, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nbytes_out) return;
  const int per = 8 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t v = 0;
  for (int j = 0; j < per; ++j) v |= ((uint32_t)q[i * per + j] & mask) << (bits * j);
  out[i] = (uint8_t)v;
}

__global__ void k_pack_sb(int64_t n, const uint16_t* __restrict__ s, const uint16_t* __restrict__ b,
                          uint32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  out[i] = (uint32_t)s[i] | ((uint32_t)b[i] << 16);
}

unsigned blocks_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs); }

// ---- dispatch over the supported (bits, row length) pairs ----------------------------------------

#define BQ_FOR_H(X) X(256) X(512) X(1024) X(2048) X(4096) X(8192)
#define BQ_FOR_I(X) X(64) X(128) X(256) X(512) X(1024) X(2048) X(4096) X(8192)

constexpr int kP1 = 1;  // row steps per wave: shared gate/up in kernel 1
constexpr int kP2 = 2;  // routed gate/up
constexpr int kP3 = 4;  // down

template <int BITS, int H>
hipError_t router_phase_impl(const LayerArgs& a, const float* x, const float* norm_src, float eps, int T,
                             bool with_shared_ffn, hipStream_t s) {
  using R = RouterCfg<H>;
  using C = RowCfg<BITS, H>;
  const int router_steps = 1;
  const int nrows = a.E + a.has_shared;
  const int rows_per_block = kWaves * router_steps * R::RPW;
  const int nrb = (nrows + rows_per_block - 1) / rows_per_block;
  int nsb = 0;
  if (with_shared_ffn && a.has_shared) {
    const int rows_per_sblock = kWaves * kP1 * C::RPW;
    nsb = (a.I + rows_per_sblock - 1) / rows_per_sblock;
  }
  hipLaunchKernelGGL((k_router_phase<BITS, H, kP1>), dim3(nrb + nsb, T), dim3(kBlock), 0, s, a, x, norm_src, eps, nrb,
                     router_steps);
  return hipGetLastError();
}

template <int BITS, int H>
hipError_t gateup_impl(const LayerArgs& a, const float* x, int T, const int32_t* idx_in, int32_t* idx_out,
                       bool with_shared, hipStream_t s) {
  using C = RowCfg<BITS, H>;
  const int rows_per_block = kWaves * kP2 * C::RPW;
  const int nb = (a.I + rows_per_block - 1) / rows_per_block;
  const int slots = a.K + ((with_shared && a.has_shared) ? 1 : 0);
  hipLaunchKernelGGL((k_gateup<BITS, H, kP2>), dim3(nb, slots, T), dim3(kBlock), 0, s, a, x, idx_in, idx_out);
  return hipGetLastError();
}

template <int BITS, int I>
hipError_t down_impl(const LayerArgs& a, int T, const int32_t* idx, const float* residual, float* out, float* y,
                     hipStream_t s) {
  using C = RowCfg<BITS, I>;
  constexpr int RB = C::RPW * kP3;
  const int nb = (a.H + RB - 1) / RB;
  hipLaunchKernelGGL((k_down<BITS, I, kP3>), dim3(nb, T), dim3(kBlock), 0, s, a, idx, residual, out, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_phase(const Geometry& g, const LayerPtrs& p, const float* x, const float* norm_src, float eps,
                               int T, const Workspace& ws, bool with_shared_ffn, hipStream_t s) {
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(HV)                                                                                 \
  case HV:                                                                                          \
    return g.bits == 4 ? router_phase_impl<4, HV>(a, x, norm_src, eps, T, with_shared_ffn, s)       \
                       : router_phase_impl<2, HV>(a, x, norm_src, eps, T, with_shared_ffn, s);
  switch (g.H) { BQ_FOR_H(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gateup(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                         const int32_t* idx_in, int32_t* idx_out, bool with_shared, hipStream_t s) {
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(HV)                                                                          \
  case HV:                                                                                   \
    return g.bits == 4 ? gateup_impl<4, HV>(a, x, T, idx_in, idx_out, with_shared, s)        \
                       : gateup_impl<2, HV>(a, x, T, idx_in, idx_out, with_shared, s);
  switch (g.H) { BQ_FOR_H(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_down(const Geometry& g, const LayerPtrs& p, int T, const Workspace& ws, const int32_t* idx,
                       const float* residual, float* out, float* y, hipStream_t s) {
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(IV)                                                               \
  case IV:                                                                        \
    return g.bits == 4 ? down_impl<4, IV>(a, T, idx, residual, out, y, s)         \
                       : down_impl<2, IV>(a, T, idx, residual, out, y, s);
  switch (g.I) { BQ_FOR_I(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const Geometry& g, int T, const Workspace& ws, int32_t* idx, float* w, float* sg,
                       double* logits_out, hipStream_t s) {
  LayerPtrs p{};
  const LayerArgs a = make_args(g, p, ws);
  hipLaunchKernelGGL(k_topk, dim3(T), dim3(64), 0, s, a, idx, w, sg, logits_out);
  return hipGetLastError();
}

hipError_t launch_combine(const Geometry& g, int T, const float* residual, const float* y, const float* w,
                          const float* sg, float* out, hipStream_t s) {
  const int64_t n = (int64_t)T * g.H;
  hipLaunchKernelGGL(k_combine, dim3(blocks_for(n, 256)), dim3(256), 0, s, T, g.H, g.K, g.has_shared, residual, y, w,
                     sg, out);
  return hipGetLastError();
}

hipError_t launch_dequant(const Geometry& g, const uint8_t* blob, int matrix, int out_dtype, void* out, hipStream_t s) {
  const int rows = matrix == 2 ? g.H : g.I;
  const int cols = matrix == 2 ? g.I : g.H;
  const int64_t n = (int64_t)rows * cols;
  hipLaunchKernelGGL(k_dequant, dim3(blocks_for(n, 256)), dim3(256), 0, s, rows, cols, g.bits,
                     blob + g.off_codes[matrix], reinterpret_cast<const uint32_t*>(blob + g.off_sb[matrix]), out_dtype,
                     out);
  return hipGetLastError();
}

hipError_t launch_pack(int H, int I, int bits, int G, const moe_expert_arrays_t* arr, uint8_t* blob, hipStream_t s) {
  const int64_t code_bytes = (int64_t)I * H * bits / 8;
  const int64_t ngroups = (int64_t)I * H / G;
  for (int m = 0; m < 3; ++m) {
    hipLaunchKernelGGL(k_pack_codes, dim3(blocks_for(code_bytes, 256)), dim3(256), 0, s, code_bytes, bits, arr->q[m],
                       blob + m * code_bytes);
    hipLaunchKernelGGL(k_pack_sb, dim3(blocks_for(ngroups, 256)), dim3(256), 0, s, ngroups, arr->scale[m],
                       arr->bias[m], reinterpret_cast<uint32_t*>(blob + 3 * code_bytes + m * ngroups * 4));
  }
  return hipGetLastError();
}

}  // namespace bqmoe
