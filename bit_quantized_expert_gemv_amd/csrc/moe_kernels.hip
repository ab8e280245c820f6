// Decode-path kernels of the quantised MoE layer for MI355X (gfx950, wave64).
//
// A single token runs as two stream-ordered launches (k_front: router, top-K and gate/up + SwiGLU,
// its blocks handing each other the logits inside the launch; then k_down), or, for several tokens
// per call and the layers k_front does not take, as three; nothing synchronises the host.
//   1. router phase: the router logits and the shared-gate logit (fp64 accumulation);
//   2. gate/up: one block per CU and 16-row slice of every expert slot. A routed slot's block
//      first picks the top-K itself from the logits (one wave, fp64 keys), then runs
//      gate/up/SwiGLU for its expert; the shared expert is one more slot, which starts its weight
//      loads at once. One block writes the routing (indices, weights, shared gate);
//   3. down (k_down): the down projections of all K+1 experts, combined with the routing weights,
//      the shared gate and the residual. Each output row sums all experts, so the result is a
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "moe_internal.h"

namespace bqmoe {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;

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

// sum_j e2m1(q_j) x_j over the 32 E2M1 codes of one MXFP4 block (byte k holds elements 2k, 2k+1,
// lower nibble first). The hardware conversion decodes E2M1 exactly (sign, 2 exponent bits with
// bias 1, 1 mantissa bit; the values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives).
template <int N>
__device__ __forceinline__ float mx_byte(uint32_t w, const float* x, float acc) {
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, N);  // byte N: elements 2N, 2N+1
  acc = fmaf(v[0], x[2 * N], acc);
  return fmaf(v[1], x[2 * N + 1], acc);
}
__device__ __forceinline__ float chunk_dot_mx(const uint4 w, const float* x) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = mx_byte<0>(ws[i], x + 8 * i, acc);
    acc = mx_byte<1>(ws[i], x + 8 * i, acc);
    acc = mx_byte<2>(ws[i], x + 8 * i, acc);
    acc = mx_byte<3>(ws[i], x + 8 * i, acc);
  }
  return acc;
}

// E8M0 block scale 2^(s - 127); 255 is NaN. Written as selects on the bit pattern (2^-127 is the
// subnormal 0x00400000): a branchy form kept the row's activations live across exec-mask branches
// and took the MXFP4 gate/up kernel from 7 to 4 waves per SIMD.
__device__ __forceinline__ float e8m0_value(uint32_t s) {
  uint32_t b = s << 23;
  b = s == 0u ? 0x00400000u : b;
  b = s == 255u ? 0x7FC00000u : b;
  return __uint_as_float(b);
}

template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 w, const float* x) {
  if constexpr (BITS == 4) return chunk_dot4(w, x);
  else return chunk_dot2(w, x);
}

// Per-element forms ("Kernel de dequantización optimizado con FMA"): every weight contributes
// fma(q, s*x, b*x) (the pages' rewrite) or (q*s + b)*x (the form it replaced). s carries the
// widening's scale (2^9 at 4-bit), so q here is the widened code. An A/B ablation of chunk_dot
// with the chunk sums.
// Per-element dequant forms of the ablation: 1 = the pages' fma(q, s*x, b*x); 2 = the naive
// (q*s + b)*x that the pages' rewrite replaced.
template <int FORM>
__device__ __forceinline__ float lit_term(float q, float x, float s, float b, float acc) {
  if constexpr (FORM == 1) return acc + fmaf(q, s * x, b * x);
  else return fmaf(fmaf(q, s, b), x, acc);
}

template <int FORM>
__device__ __forceinline__ float chunk_lit4(const uint4 w, const float* x, float s, float b, float acc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ws[i] & 0x0F0F0F0Fu;
    const uint32_t hi = (ws[i] >> 4) & 0x0F0F0F0Fu;
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const auto bq = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    acc = lit_term<FORM>(a[0], x[8 * i + 0], s, b, acc);
    acc = lit_term<FORM>(c[0], x[8 * i + 1], s, b, acc);
    acc = lit_term<FORM>(a[1], x[8 * i + 2], s, b, acc);
    acc = lit_term<FORM>(c[1], x[8 * i + 3], s, b, acc);
    acc = lit_term<FORM>(bq[0], x[8 * i + 4], s, b, acc);
    acc = lit_term<FORM>(d[0], x[8 * i + 5], s, b, acc);
    acc = lit_term<FORM>(bq[1], x[8 * i + 6], s, b, acc);
    acc = lit_term<FORM>(d[1], x[8 * i + 7], s, b, acc);
  }
  return acc;
}

template <int FORM, int N>
__device__ __forceinline__ float lit2_byte(uint32_t lo, uint32_t hi, const float* x, float s, float b, float acc) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(lo, 2.0f, N);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(hi, 2.0f, N);
  acc = lit_term<FORM>(a[0], x[4 * N + 0], s, b, acc);
  acc = lit_term<FORM>(c[0], x[4 * N + 1], s, b, acc);
  acc = lit_term<FORM>(a[1], x[4 * N + 2], s, b, acc);
  acc = lit_term<FORM>(c[1], x[4 * N + 3], s, b, acc);
  return acc;
}

template <int FORM>
__device__ __forceinline__ float chunk_lit2(const uint4 w, const float* x, float s, float b, float acc) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ws[i] & 0x33333333u;
    const uint32_t hi = (ws[i] >> 2) & 0x33333333u;
    acc = lit2_byte<FORM, 0>(lo, hi, x + 16 * i, s, b, acc);
    acc = lit2_byte<FORM, 1>(lo, hi, x + 16 * i, s, b, acc);
    acc = lit2_byte<FORM, 2>(lo, hi, x + 16 * i, s, b, acc);
    acc = lit2_byte<FORM, 3>(lo, hi, x + 16 * i, s, b, acc);
  }
  return acc;
}

// This lane's share of one row: sum over its chunks of s * sum(q x) + b * S (FORM 0), one of the
// per-element forms of the ablation (FORM 1, 2), or for MXFP4 (FORM 3, one block per chunk)
// 2^(e - 127) * sum(e2m1(q) x) with the block's E8M0 byte e in sb.
template <int BITS, class C, int FORM = 0>
__device__ __forceinline__ float row_partial(const uint4 (&cw)[C::CPL], const uint32_t (&sb)[C::CPL],
                                             const float (&xr)[C::XPL], const float (&S)[C::CPL]) {
  constexpr float kCvt = BITS == 4 ? 512.0f : 1.0f;  // undo the e4m3 2^-9
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    if constexpr (FORM == 3) {
      a = fmaf(e8m0_value(sb[j]), chunk_dot_mx(cw[j], &xr[j * C::CH]), a);
    } else if constexpr (FORM != 0) {
      if constexpr (BITS == 4) a = chunk_lit4<FORM>(cw[j], &xr[j * C::CH], bf16_lo(sb[j]) * kCvt, bf16_hi(sb[j]), a);
      else a = chunk_lit2<FORM>(cw[j], &xr[j * C::CH], bf16_lo(sb[j]) * kCvt, bf16_hi(sb[j]), a);
    } else {
      const float d = chunk_dot<BITS>(cw[j], &xr[j * C::CH]);
      a = fmaf(bf16_lo(sb[j]) * kCvt, d, fmaf(bf16_hi(sb[j]), S[j], a));
    }
  }
  return a;
}

// One row's chunks for this lane, with each chunk's (scale, bias) word, or for MXFP4 (MX) its E8M0
// byte (at 4-bit a 16-byte chunk is one block of 32).
template <class C, bool MX = false>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sbp, int r,
                                         int lir, uint4 (&cw)[C::CPL], uint32_t (&sb)[C::CPL]) {
  const uint8_t* row = codes + (size_t)r * C::ROW_BYTES;
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const int c = lir + j * C::LPR;
    cw[j] = *reinterpret_cast<const uint4*>(row + (size_t)c * 16);
    if constexpr (MX) sb[j] = sbp[(size_t)r * C::NC + c];
    else sb[j] = reinterpret_cast<const uint32_t*>(sbp)[(size_t)r * C::GROUPS + (c * C::CH) / 64];
  }
}

// ---- activation staging through LDS -------------------------------------------------------------
// A lane needs CH consecutive activations per chunk, and neighbouring lanes own neighbouring
// chunks. Loading that straight into registers makes each load instruction touch 64 cache
// lines. Instead the vector is read with coalesced 16-byte loads and parked in LDS, with the
// 16-byte slots of each chunk XOR-swizzled so that consecutive lanes hit distinct banks. Each
// lane then reads its slice back. The coalesced loads are issued before the expert weights
// and written to LDS only after the weight loads are in flight, so in-order completion
// counting never makes the weight loads wait for them.
template <class C>
__device__ __forceinline__ int xslot(int chunk, int q) {
  if constexpr (C::CH == 32) return chunk * 8 + (q ^ ((chunk >> 1) & 7));
  else return chunk * 16 + (q ^ (chunk & 15));
}

// COLS floats loaded by NT cooperating lanes: lane i takes float4 i, i + NT, ...
template <int COLS, int NT>
struct Stage {
  static constexpr int N4 = COLS / 4;
  static constexpr int PER = (N4 + NT - 1) / NT;
  float4 v[PER];
  __device__ __forceinline__ void load(const float* __restrict__ src, int tid) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      v[k] = (N4 % NT == 0 || i < N4) ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  template <class C>
  __device__ __forceinline__ void store(float4* __restrict__ xs, int tid, float scale) const {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * NT;
      if (N4 % NT == 0 || i < N4) {
        float4 t = v[k];
        t.x *= scale; t.y *= scale; t.z *= scale; t.w *= scale;
        xs[xslot<C>(i / (C::CH / 4), i % (C::CH / 4))] = t;
      }
    }
  }
};

// This lane's activations (from LDS) and their per-chunk sums.
// An fp32 product that is always rounded: the compiler may not fuse it into a later addition.
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// With SCALED, each value is multiplied by `scale` as it is read (the same rounded fp32 products as
// a scaled Stage::store).
template <class C, bool SCALED = false>
__device__ __forceinline__ void read_act(const float4* __restrict__ xs, int lir, float (&xr)[C::XPL],
                                         float (&S)[C::CPL], float scale = 1.0f) {
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const int chunk = lir + j * C::LPR;
#pragma unroll
    for (int q = 0; q < C::CH / 4; ++q) {
      float4 t = xs[xslot<C>(chunk, q)];
      if constexpr (SCALED) {  // rounded products, never contracted into the sums below
        t.x = mul_rounded(t.x, scale); t.y = mul_rounded(t.y, scale);
        t.z = mul_rounded(t.z, scale); t.w = mul_rounded(t.w, scale);
      }
      xr[j * C::CH + 4 * q + 0] = t.x;
      xr[j * C::CH + 4 * q + 1] = t.y;
      xr[j * C::CH + 4 * q + 2] = t.z;
      xr[j * C::CH + 4 * q + 3] = t.w;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < C::CH; ++i) sum += xr[j * C::CH + i];
    S[j] = sum;
  }
}

// ---- cross-lane reductions on the VALU with DPP (gfx9 controls) -----------------------------------
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i within each 16
constexpr int kDppBcast15 = 0x142;    // lane 15 of row r -> row r+1 (row mask 0xA)
constexpr int kDppBcast31 = 0x143;    // lane 31 -> rows 2 and 3 (row mask 0xC)

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d(double old, double v) {
  const long long o = __double_as_longlong(old), x = __double_as_longlong(v);
  const int lo = dpp_i<CTRL, ROWS>((int)(o & 0xFFFFFFFF), (int)(x & 0xFFFFFFFF));
  const int hi = dpp_i<CTRL, ROWS>((int)(o >> 32), (int)(x >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float pick_dpp(float old, float v) { return dpp_f<CTRL, ROWS>(old, v); }
template <int CTRL, int ROWS>
__device__ __forceinline__ double pick_dpp(double old, double v) { return dpp_d<CTRL, ROWS>(old, v); }

// Sum over aligned segments of LPR lanes. The full sum is valid in the LAST lane of each segment
// (lanes of a segment never read another segment). Same order on every call: deterministic.
template <int LPR, class T>
__device__ __forceinline__ T seg_sum(T v) {
  if constexpr (LPR >= 2) v += pick_dpp<kDppQuadXor1, 0xF>(T(0), v);
  if constexpr (LPR >= 4) v += pick_dpp<kDppQuadXor2, 0xF>(T(0), v);
  if constexpr (LPR >= 8) v += pick_dpp<kDppHalfMirror, 0xF>(T(0), v);
  if constexpr (LPR >= 16) v += pick_dpp<kDppRowMirror, 0xF>(T(0), v);
  if constexpr (LPR >= 32) v += pick_dpp<kDppBcast15, 0xA>(T(0), v);
  if constexpr (LPR >= 64) v += pick_dpp<kDppBcast31, 0xC>(T(0), v);
  return v;
}

__device__ __forceinline__ float silu_mul(float a, float c) { return a / (1.0f + expf(-a)) * c; }

// A store that writes through the XCD's L2 (a relaxed agent-scope atomic store), for values that the
// next kernel reads, mostly on other XCDs: they reach memory while this kernel runs instead of in
// its end-of-kernel write-back. Logits, routing and the layer output written this way, in
// interleaved runs: decode4 -0.02 to -0.13 us/token (15.47 -> 15.36 in the first), decodemx 20.12 ->
// 19.96, stack60 0.4-1.3% per step. The stack's normalised input stays in plain 16-byte stores.
template <class T>
__device__ __forceinline__ void store_through(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct LayerArgs {
  int H, I, E, K, NE, has_shared, form;
  uint64_t off_codes[3], off_sb[3];
  const uint8_t* experts;
  uint64_t stride;
  const uint8_t* shared;
  const uint16_t* router;
  const uint16_t* sgate;
  Workspace ws;
  int32_t* err;  // optional error word: set to MOE_EINVAL when a caller's expert index is out of range
};

LayerArgs make_args(const Geometry& g, const LayerPtrs& p, const Workspace& ws) {
  LayerArgs a;
  a.H = g.H; a.I = g.I; a.E = g.E; a.K = g.K; a.NE = g.NE; a.has_shared = g.has_shared; a.form = g.form;
  for (int m = 0; m < 3; ++m) { a.off_codes[m] = g.off_codes[m]; a.off_sb[m] = g.off_sb[m]; }
  a.experts = p.experts; a.stride = p.stride; a.shared = p.shared; a.router = p.router; a.sgate = p.sgate;
  a.ws = ws;
  a.err = nullptr;
  return a;
}

// ---- top-K ---------------------------------------------------------------------------------------
// (value, index) order of the top-K: larger value first, then lower index.
__device__ __forceinline__ bool better(double v, int i, double bv, int bi) { return v > bv || (v == bv && i < bi); }

template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
  const double ov = dpp_d<CTRL, ROWS>(-INFINITY, v);
  const int oi = dpp_i<CTRL, ROWS>(0x7FFFFFFF, i);
  if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Wave-wide top-K of logits[0..E): descending value, ties to the lower index. Lane l holds logits
// l, l+64, ... (PL per lane, E <= 64*PL). The loads are unconditional (indexes are clamped), so they
// leave back to back. Each round takes every lane's best remaining value and carries the best pair
// to lane 63 with DPP steps, with no LDS round trips. It is read back wave-uniform and retired.
// Lane 0 records the choices in sel/val (LDS) when `record` is set. Returns the expert at
// position `want`, clamped into [0, E) so that NaN logits can never address memory outside the pool.
template <int PL>
__device__ __forceinline__ void load_topk_values(const double* __restrict__ lg, int E, int lane, double (&v)[PL]) {
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    const double t = lg[min(e, E - 1)];
    v[i] = e < E ? t : -INFINITY;
  }
}

template <int PL>
__device__ __forceinline__ int wave_topk(double (&v)[PL], int E, int K, int lane, int want, bool record,
                                         int32_t* __restrict__ sel, double* __restrict__ val) {
  int chosen = 0;
  for (int k = 0; k < K; ++k) {
    double bv = v[0];
    int bi = lane;
#pragma unroll
    for (int i = 1; i < PL; ++i) {
      const bool c = v[i] > bv;  // strict: the earlier (lower) index keeps a tie
      bv = c ? v[i] : bv;
      bi = c ? lane + 64 * i : bi;
    }
    argmax_step<kDppQuadXor1, 0xF>(bv, bi);
    argmax_step<kDppQuadXor2, 0xF>(bv, bi);
    argmax_step<kDppHalfMirror, 0xF>(bv, bi);
    argmax_step<kDppRowMirror, 0xF>(bv, bi);
    argmax_step<kDppBcast15, 0xA>(bv, bi);
    argmax_step<kDppBcast31, 0xC>(bv, bi);
    // read back with every lane active (values computed under a partial exec mask would be stale)
    const long long bits = __double_as_longlong(bv);
    const int lo = __builtin_amdgcn_readlane((int)(bits & 0xFFFFFFFF), 63);
    const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), 63);
    const int win = min(max(__builtin_amdgcn_readlane(bi, 63), 0), E - 1);
    const double wv = __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
    if (k == want) chosen = win;
    if (record && lane == 0) {
      sel[k] = win;
      val[k] = wv;
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) v[i] = (lane + 64 * i == win) ? -INFINITY : v[i];
  }
  return chosen;
}

// The same top-K (descending value, ties to the lower index; the same choices, bit for bit) with a
// shorter dependent chain per round. Each fp64 logit becomes an order-preserving 64-bit key (the sign
// bit flips non-negative values, every bit flips negative ones; NaN, and the slots past E, become
// key 0, the lowest). A round first takes the wave maximum M of the keys' upper 32 bits with six
// one-instruction DPP steps. If exactly one key has upper half M, it is the round's winner, and no
// fp64 compare runs at all; only keys tied in their upper 32 bits (distinct logits agreeing in sign,
// exponent and 20 mantissa bits, or equal logits) take the full (key, index) comparison.
__device__ __forceinline__ double wave_read_f64(double v, int lane) {  // lane's v, wave-uniform
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {  // complete in lane 63
  v = max(v, (uint32_t)dpp_i<kDppQuadXor1, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kDppQuadXor2, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kDppHalfMirror, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kDppRowMirror, 0xF>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kDppBcast15, 0xA>(0, (int)v));
  v = max(v, (uint32_t)dpp_i<kDppBcast31, 0xC>(0, (int)v));
  return v;
}
// (key, index) argmax step for the tie case: larger key first, then lower index
template <int CTRL, int ROWS>
__device__ __forceinline__ void keymax_step(uint64_t& k, int& i) {
  const uint32_t ohi = (uint32_t)dpp_i<CTRL, ROWS>(0, (int)(k >> 32));
  const uint32_t olo = (uint32_t)dpp_i<CTRL, ROWS>(0, (int)(uint32_t)k);
  const int oi = dpp_i<CTRL, ROWS>(0x7FFFFFFF, i);
  const uint64_t ok = ((uint64_t)ohi << 32) | olo;
  if (ok > k || (ok == k && oi < i)) { k = ok; i = oi; }
}
// The keys of wave_topk_fast's rounds.
template <int PL>
__device__ __forceinline__ void topk_keys(const double (&v)[PL], int E, int lane, uint64_t (&key)[PL]) {
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint64_t b = (uint64_t)__double_as_longlong(v[i]);
    const uint64_t k = (b >> 63) ? ~b : (b | (1ull << 63));
    key[i] = (lane + 64 * i < E && !__builtin_isnan(v[i])) ? k : 0ull;
  }
}
// The fp64 value at expert index `win` (wave-uniform): each slot read from its lane, then a uniform
// select (a select among v[] itself compiles to a scratch copy).
template <int PL>
__device__ __forceinline__ double wave_value_at(const double (&v)[PL], int win) {
  const int src = win % 64, q = win / 64;
  double wv = wave_read_f64(v[0], src);
#pragma unroll
  for (int i = 1; i < PL; ++i) {
    const double t = wave_read_f64(v[i], src);
    wv = q == i ? t : wv;
  }
  return wv;
}
// One round: the winner among the remaining keys (retired from key[] on return), recorded as
// position r in sel (and its value in val, unless val is null) by lane 0 when `record` is set.
template <int PL>
__device__ __forceinline__ int topk_round(uint64_t (&key)[PL], const double (&v)[PL], int E, int lane, int r,
                                          bool record, int32_t* __restrict__ sel, double* __restrict__ val) {
  uint32_t m = (uint32_t)(key[0] >> 32);
#pragma unroll
  for (int i = 1; i < PL; ++i) m = max(m, (uint32_t)(key[i] >> 32));
  const uint32_t M = (uint32_t)__builtin_amdgcn_readlane((int)wave_max_u32(m), 63);
  uint32_t cm = 0;  // this lane's values whose upper half is M
#pragma unroll
  for (int i = 0; i < PL; ++i) cm |= ((uint32_t)(key[i] >> 32) == M ? 1u : 0u) << i;
  const uint64_t lanes = __ballot(cm != 0);
  const int wl0 = __builtin_ctzll(lanes);
  const uint32_t cm0 = (uint32_t)__builtin_amdgcn_readlane((int)cm, wl0);
  int win;
  if ((lanes & (lanes - 1)) == 0 && (cm0 & (cm0 - 1)) == 0) {
    win = wl0 + 64 * __builtin_ctz(cm0);  // a unique upper half decides the round
  } else {  // tied upper halves: the full (key, index) argmax over the tied keys
    uint64_t bk = 0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const bool c = ((cm >> i) & 1u) && (bi == 0x7FFFFFFF || key[i] > bk);  // strict: the lower index keeps a tie
      bk = c ? key[i] : bk;
      bi = c ? lane + 64 * i : bi;
    }
    keymax_step<kDppQuadXor1, 0xF>(bk, bi);
    keymax_step<kDppQuadXor2, 0xF>(bk, bi);
    keymax_step<kDppHalfMirror, 0xF>(bk, bi);
    keymax_step<kDppRowMirror, 0xF>(bk, bi);
    keymax_step<kDppBcast15, 0xA>(bk, bi);
    keymax_step<kDppBcast31, 0xC>(bk, bi);
    win = __builtin_amdgcn_readlane(bi, 63);
  }
  win = min(max(win, 0), E - 1);
  if (record && val == nullptr) {
    if (lane == 0) sel[r] = win;
  } else if (record) {
    const double wv = wave_value_at<PL>(v, win);
    if (lane == 0) {
      sel[r] = win;
      val[r] = wv;
    }
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) key[i] = (lane + 64 * i == win) ? 0ull : key[i];
  return win;
}
template <int PL>
__device__ __forceinline__ int wave_topk_fast(const double (&v)[PL], int E, int K, int lane, int want, bool record,
                                              int32_t* __restrict__ sel, double* __restrict__ val) {
  uint64_t key[PL];
  topk_keys<PL>(v, E, lane, key);
  int chosen = 0;
  for (int r = 0; r < K; ++r) {
    const int win = topk_round<PL>(key, v, E, lane, r, record, sel, val);
    if (r == want) chosen = win;
  }
  return chosen;
}

// Softmax of the K chosen logits (the full softmax over E renormalised over the chosen set reduces to
// this), written with the choices and the shared gate for token t. A whole wave calls this: lane k < K
// computes exp(l_k - l_0) in fp32 (l_k - l_0 <= 0 is formed in fp64, then rounded), the lanes' terms
// are added in slot order, and lane k writes slot k. In fp32 and across lanes, the routing write
// costs one exp's latency instead of K + 1 serial fp64 exps at the end of the block's work.
__device__ __forceinline__ void write_routing(const LayerArgs& a, int t, int lane, const int32_t* __restrict__ sel,
                                              const double* __restrict__ val, double gate_logit,
                                              int32_t* __restrict__ idx_a, float* __restrict__ w_a,
                                              int32_t* __restrict__ idx_b, float* __restrict__ g_out) {
  const float e = lane < a.K ? expf((float)(val[min(lane, a.K - 1)] - val[0])) : 0.0f;
  float z = 0.0f;
  for (int k = 0; k < a.K; ++k) z += __shfl(e, k);
  if (lane < a.K) {
    store_through(&idx_a[(size_t)t * a.K + lane], sel[lane]);
    store_through(&w_a[(size_t)t * a.K + lane], e / z);
    if (idx_b) idx_b[(size_t)t * a.K + lane] = sel[lane];
  }
  if (lane == 0 && g_out && a.has_shared) store_through(&g_out[t], 1.0f / (1.0f + expf(-(float)gate_logit)));
}

// RMS norm scale 1/sqrt(mean(h^2) + eps) from the fp64 sum of h^2 over the whole vector.
__device__ __forceinline__ double rms_inv(double ss, int H, float eps) {
  return 1.0 / sqrt(ss / (double)H + (double)eps);
}

// An fp64 value of one lane, made uniform across the wave.
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// ---------------------------------------------------------------------------------------------
// Kernel 1: router logits and the shared-gate logit (row E), accumulated in fp64. In a stack the
// input is RMS-normalised first, and the blocks together store the normalised vector for kernel 2.
// The arguments of the first requests (the input, the router and shared-gate rows, E, the row
// count, the row steps) lead the list, so they arrive preloaded in SGPRs.
#ifndef BQ_ROUTER_SPLIT
#define BQ_ROUTER_SPLIT 4
#endif
template <int H>
__global__ __launch_bounds__(kBlock) void k_router_phase(const float* __restrict__ src0,
                                                         const uint16_t* __restrict__ router,
                                                         const uint16_t* __restrict__ sgate, int E, int nrows,
                                                         int router_steps, LayerArgs a, const float* __restrict__ x,
                                                         const float* __restrict__ norm_src, float eps) {
  using R = RouterCfg<H>;
  constexpr int SPLIT = (R::CPL % BQ_ROUTER_SPLIT == 0) ? BQ_ROUTER_SPLIT : 1;  // waves per row
  constexpr int CPW = R::CPL / SPLIT;                                            // chunks per lane
  __shared__ double part[kWaves];
  __shared__ double psq[kWaves];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % R::LPR, rig = lane / R::LPR;
  const int piece = wave % SPLIT;
  auto row_of = [&](int s) {
    const int base = ((blockIdx.x * (kWaves / SPLIT) + wave / SPLIT) * router_steps + s) * R::RPW;
    return base + rig;
  };
  auto load_w = [&](int s, uint4 (&w)[CPW]) {
    const int rr = min(row_of(s), nrows - 1);
    const uint16_t* row = (rr < E) ? router + (size_t)rr * H : sgate;
#pragma unroll
    for (int j = 0; j < CPW; ++j) w[j] = *reinterpret_cast<const uint4*>(row + (lir + (j * SPLIT + piece) * R::LPR) * 8);
  };
  // The norm's scale is a scalar, so a row's dot product with the raw input is taken first and
  // scaled at the end: sum_j R[e][j] (s h_j) = s sum_j R[e][j] h_j, with every product exact in fp64.
  const bool norm = norm_src != nullptr;
  const float* src = src0 + (size_t)t * H;  // norm_src when norm, else x
  uint4 w[CPW];
  float4 xr[CPW][2];
  load_w(0, w);
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const float4* p = reinterpret_cast<const float4*>(src + (lir + (j * SPLIT + piece) * R::LPR) * 8);
    xr[j][0] = p[0];
    xr[j][1] = p[1];
  }
  // The mean square of h, from the activations already in registers: the SPLIT waves of a row set
  // hold the whole vector between them (each row group of a wave the same share), so every block
  // adds the same squares in the same order and gets the same scale, bit for bit.
  double scale = 1.0;
  if (norm) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const float xv[8] = {xr[j][0].x, xr[j][0].y, xr[j][0].z, xr[j][0].w,
                           xr[j][1].x, xr[j][1].y, xr[j][1].z, xr[j][1].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) ss = fma((double)xv[q], (double)xv[q], ss);
    }
    ss = seg_sum<R::LPR>(ss);  // the wave's share, complete in lane LPR - 1 of each row group
    if constexpr (SPLIT == 1) {
      scale = rms_inv(readlane_f64(ss, R::LPR - 1), H, eps);
    } else {
      if (lane == 63) psq[wave] = ss;  // summed after the first row step's barrier
    }
  }
  for (int s = 0; s < router_steps; ++s) {
    if (s > 0) load_w(s, w);
    const int r = row_of(s);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const float xv[8] = {xr[j][0].x, xr[j][0].y, xr[j][0].z, xr[j][0].w,
                           xr[j][1].x, xr[j][1].y, xr[j][1].z, xr[j][1].w};
      const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = fma((double)bf16_lo(ww[q]), (double)xv[2 * q], acc[q]);
        acc[q] = fma((double)bf16_hi(ww[q]), (double)xv[2 * q + 1], acc[q]);
      }
    }
    const double tot = seg_sum<R::LPR>((acc[0] + acc[1]) + (acc[2] + acc[3]));
    if constexpr (SPLIT == 1) {
      if (lir == R::LPR - 1 && r < nrows) store_through(&a.ws.logits[(size_t)t * (E + 1) + r], norm ? tot * scale : tot);
    } else {
      if (lane == 63) part[wave] = tot;
      __syncthreads();
      if (norm && s == 0) {
        double v = psq[wave - piece];
        for (int q = 1; q < SPLIT; ++q) v += psq[wave - piece + q];
        scale = rms_inv(v, H, eps);
      }
      if (piece == 0 && lane == 63 && r < nrows) {
        double v = part[wave];
        for (int q = 1; q < SPLIT; ++q) v += part[wave + q];
        store_through(&a.ws.logits[(size_t)t * (E + 1) + r], norm ? v * scale : v);
      }
      __syncthreads();
    }
  }
  // The normalised input for phase 2, written from the activations already in registers: block b
  // writes 8-float chunks b, b + gridDim.x, ..., each from the one lane that holds it (row group 0).
  // Spread this way no block waits on extra loads, and the next kernel does not wait on a straggler.
  if (norm) {
    const float fs = (float)scale;
    for (int c = blockIdx.x; c < R::NC; c += gridDim.x) {
      const int jp = c / R::LPR;  // chunk position j * SPLIT + piece
      if (rig != 0 || lir != c % R::LPR || piece != jp % SPLIT || wave / SPLIT != 0) continue;
#pragma unroll
      for (int j = 0; j < CPW; ++j) {
        if (j != jp / SPLIT) continue;
        float4* dst = reinterpret_cast<float4*>(a.ws.u + (size_t)t * H + (size_t)c * 8);
        dst[0] = make_float4(xr[j][0].x * fs, xr[j][0].y * fs, xr[j][0].z * fs, xr[j][0].w * fs);
        dst[1] = make_float4(xr[j][1].x * fs, xr[j][1].y * fs, xr[j][1].z * fs, xr[j][1].w * fs);
      }
    }
  }
}

// Kernel 1 for several tokens without the stack's norm: each block reads its router row once for a
// group of TG tokens, and every lane accumulates one fp64 dot product per token. A token's logits
// are summed in the same order as in k_router_phase, so they are bitwise the same; only the row
// traffic drops, from T reads of the router to T / TG. The arguments of the first requests lead the
// list, so they arrive preloaded in SGPRs.
template <int H, int TG>
__global__ __launch_bounds__(kBlock) void k_router_group(const float* __restrict__ x,
                                                        const uint16_t* __restrict__ router,
                                                        const uint16_t* __restrict__ sgate, int E, int nrows, int T,
                                                        LayerArgs a) {
  using R = RouterCfg<H>;
  constexpr int SPLIT = (R::CPL % BQ_ROUTER_SPLIT == 0) ? BQ_ROUTER_SPLIT : 1;  // waves per row
  constexpr int CPW = R::CPL / SPLIT;                                            // chunks per lane
  __shared__ double part[TG][kWaves];
  const int t0 = blockIdx.y * TG;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % R::LPR, rig = lane / R::LPR;
  const int piece = wave % SPLIT;
  const int r = (blockIdx.x * (kWaves / SPLIT) + wave / SPLIT) * R::RPW + rig;  // one row step per block
  uint4 w[CPW];
  {
    const int rr = min(r, nrows - 1);
    const uint16_t* row = (rr < E) ? router + (size_t)rr * H : sgate;
#pragma unroll
    for (int j = 0; j < CPW; ++j) w[j] = *reinterpret_cast<const uint4*>(row + (lir + (j * SPLIT + piece) * R::LPR) * 8);
  }
  float4 xr[TG][CPW][2];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    const float* src = x + (size_t)min(t0 + g, T - 1) * H;  // tokens past T re-read the last one
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const float4* p = reinterpret_cast<const float4*>(src + (lir + (j * SPLIT + piece) * R::LPR) * 8);
      xr[g][j][0] = p[0];
      xr[g][j][1] = p[1];
    }
  }
  double tot[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const float xv[8] = {xr[g][j][0].x, xr[g][j][0].y, xr[g][j][0].z, xr[g][j][0].w,
                           xr[g][j][1].x, xr[g][j][1].y, xr[g][j][1].z, xr[g][j][1].w};
      const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = fma((double)bf16_lo(ww[q]), (double)xv[2 * q], acc[q]);
        acc[q] = fma((double)bf16_hi(ww[q]), (double)xv[2 * q + 1], acc[q]);
      }
    }
    tot[g] = seg_sum<R::LPR>((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
  if constexpr (SPLIT == 1) {
    if (lir == R::LPR - 1 && r < nrows) {
#pragma unroll
      for (int g = 0; g < TG; ++g)
        if (t0 + g < T) store_through(&a.ws.logits[(size_t)(t0 + g) * (E + 1) + r], tot[g]);
    }
  } else {
    if (lane == 63) {
#pragma unroll
      for (int g = 0; g < TG; ++g) part[g][wave] = tot[g];
    }
    __syncthreads();
    if (piece == 0 && lane == 63 && r < nrows) {
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        if (t0 + g >= T) continue;
        double v = part[g][wave];
        for (int q = 1; q < SPLIT; ++q) v += part[g][wave + q];
        store_through(&a.ws.logits[(size_t)(t0 + g) * (E + 1) + r], v);
      }
    }
  }
}

// Kernel 2: gate/up/SwiGLU of the routed experts (blockIdx.y = slot) and, as slot K, of the shared
// expert; blockIdx.x is a slice of kSlice rows, blockIdx.z the token. One block per CU reads the
// activations once per CU (every row of gate and up needs all of them): a CU can keep only a limited
// number of cache lines in flight, so its time tracks the lines it touches, and the activations were
// most of them when four 4-wave blocks shared a CU. Wave 0 of a routed block picks the expert with
// the two-phase top-K and shares it through LDS; the shared slot's blocks, which need no routing,
// stream their weights meanwhile. h goes straight from the row lanes to memory. The arguments of
// the first requests (logits, x, the caller's indices, E, K) lead the list, so they arrive
// preloaded in SGPRs.
constexpr int kSlice = 16;  // rows of gate and up per block
template <int BITS, int H, int FORM, int PL, int NW>
__global__ __launch_bounds__(64 * NW) void k_gateup(const double* __restrict__ logits, const float* __restrict__ x,
                                                    const int32_t* __restrict__ idx_in, int E, int K, LayerArgs a,
                                                    int32_t* __restrict__ idx_out) {
  using C = RowCfg<BITS, H>;
  constexpr int NT = 64 * NW;
  constexpr bool MX = FORM == 3;
  constexpr int STEPS = kSlice / C::RPW;                 // row steps of a slice (gate and up rows)
  constexpr int PW = (STEPS + NW - 1) / NW;              // row steps per wave
  constexpr int PP0 = 8 / C::CPL > 0 ? 8 / C::CPL : 1;   // steps in registers at once
  constexpr int PP = PW < PP0 ? PW : PP0;
  constexpr int NPASS = (PW + PP - 1) / PP;
  static_assert(kSlice % C::RPW == 0, "a row step covers whole rows of the slice");
  __shared__ float4 xs[H / 4];
  __shared__ int32_t sel[MOE_MAX_TOP_K];
  __shared__ double val[MOE_MAX_TOP_K];

  const int t = blockIdx.z;
  // Routed slots in reverse when K > 4 (slot s needs top-K rounds 0..s, so the ones with the most
  // rounds start first); the shared expert's slot K stays last.
  const bool reversed = K > 4;
  const int slot = reversed && (int)blockIdx.y < K ? K - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // the rest of the arguments only after the first requests (below) have left
  auto rows_of_h = [&]() __attribute__((always_inline)) {  // this block's rows of h
    const int NSL = a.I / kSlice, bx = blockIdx.x;  // slices per expert
    const int slice = (NSL & 7) == 0 ? (bx & 7) * (NSL >> 3) + (bx >> 3) : bx;
    return a.ws.h + ((size_t)t * a.NE + slot) * a.I + (size_t)slice * kSlice;
  };
  int e = 0;
  Stage<H, NT> st;
  __shared__ int32_t chosen;
  // Wave 0 of a routed block picks the expert (the other waves would only repeat its work on the
  // same SIMDs) and, in the first routed block dispatched, records the choices; after the block's
  // work it writes the routing for the combine kernel (written earlier, the softmax's fp64 exps and
  // the gate logit's load would hold back the block's weight loads).
  bool writer = false;
  double gate_logit = 0.0;
  const bool routed = slot < K;
  if (routed) {
    if (idx_in != nullptr) {
      if (threadIdx.x == 0) chosen = idx_in[(size_t)t * K + slot];
      st.load(x + (size_t)t * H, threadIdx.x);
    } else if (wave == 0) {
      const double* lg = logits + (size_t)t * (E + 1);
      // the logits are requested first, so waiting for them never waits for the activations
      double v[PL];
      load_topk_values<PL>(lg, E, lane, v);
      gate_logit = lg[E];  // the shared-gate logit (row E), for the routing write at the end
      st.load(x + (size_t)t * H, threadIdx.x);
      writer = blockIdx.x == 0 && blockIdx.y == 0;  // in the first routed slot dispatched
      // slot s needs rounds 0..s only; the writer takes all K to record the routing
      const int e = wave_topk_fast<PL>(v, E, writer ? K : slot + 1, lane, slot, writer, sel, val);
      if (lane == 0) chosen = e;
    } else {
      st.load(x + (size_t)t * H, threadIdx.x);
    }
    // the activations go to LDS before the weights are requested: the block then computes each row
    // as soon as its data lands, instead of waiting at a barrier behind throttled load issue
    st.template store<C>(xs, threadIdx.x, 1.0f);
    __syncthreads();
    e = chosen;
    if (e < 0 || e >= E) {  // a caller's index outside the pool: the slot's h is NaN, nothing is read
      if ((int)threadIdx.x < kSlice) rows_of_h()[threadIdx.x] = NAN;
      if (a.err != nullptr && threadIdx.x == 0) *a.err = MOE_EINVAL;
      return;  // the whole block takes this branch (slot is per block)
    }
  } else {
    st.load(x + (size_t)t * H, threadIdx.x);
  }
  const int I = a.I;
  const int NSL = I / kSlice;  // slices per expert
  const int bx = blockIdx.x;
  const int slice = (NSL & 7) == 0 ? (bx & 7) * (NSL >> 3) + (bx >> 3) : bx;
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  float* hout = rows_of_h();
  const uint8_t* blob = routed ? a.experts + (size_t)e * a.stride : a.shared;

  // 1. weight loads: gate/up rows of the first pass
  const uint8_t* gc = blob + a.off_codes[0];
  const uint8_t* uc = blob + a.off_codes[1];
  const uint8_t* gs = blob + a.off_sb[0];
  const uint8_t* us = blob + a.off_sb[1];
  const int row0 = slice * kSlice;
  uint4 cg[PP][C::CPL], cu[PP][C::CPL];
  uint32_t sg[PP][C::CPL], su[PP][C::CPL];
  auto load_pass = [&](int pass) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int r = min((wave * PW + pass * PP + p) * C::RPW + rig, kSlice - 1);  // past the slice: its last row again
      load_row<C, MX>(gc, gs, row0 + r, lir, cg[p], sg[p]);
      load_row<C, MX>(uc, us, row0 + r, lir, cu[p], su[p]);
    }
  };
  load_pass(0);
  if (!routed) {  // the shared slot requested its weights first; its activations are parked now
    __builtin_amdgcn_sched_barrier(0);
    st.template store<C>(xs, threadIdx.x, 1.0f);
    __syncthreads();
  }
  float xr[C::XPL], S[C::CPL];
  read_act<C>(xs, lir, xr, S);

  // 2. gate/up rows and SwiGLU
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass > 0) load_pass(pass);
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int step = wave * PW + pass * PP + p;
      const int r = step * C::RPW + rig;
      const float ga = seg_sum<C::LPR>(row_partial<BITS, C, FORM>(cg[p], sg[p], xr, S));
      const float ua = seg_sum<C::LPR>(row_partial<BITS, C, FORM>(cu[p], su[p], xr, S));
      if (lir == C::LPR - 1 && step < STEPS && r < kSlice)  // written through: the down kernel reads it next
        __hip_atomic_store(&hout[r], silu_mul(ga, ua), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (writer) write_routing(a, t, lane, sel, val, gate_logit, a.ws.idx, a.ws.w, idx_out, a.ws.g);
}

// Kernel 3: down projections of all expert slots for a block of output rows; combine or store.
// 8 waves: wave w handles slots w%4, w%4+4, ... over half the block's rows (w/4 picks the half).
// Against 4 waves over all rows, each wave's compute after its data lands halves: decode4 15.60 ->
// 15.49, decode2 14.80 -> 14.66, decodemx 20.87 -> 20.65 us/token. The SwiGLU vectors are loaded
// once per block rather than once per wave: decode4 15.75 -> 15.61, decodemx 20.50 -> 20.20.
// The SwiGLU vectors and the expert index are requested first, from the leading arguments, which
// arrive preloaded in SGPRs; the combine coefficient is read after the parking barrier, so that the
// barrier does not wait for that load.
template <int BITS, int I, int P0, int FORM>
__global__ __launch_bounds__(2 * kBlock) void k_down(const float* __restrict__ h, const int32_t* __restrict__ idx,
                                                 int ne, int K, int H, const uint8_t* __restrict__ sdc,
                                                 const uint8_t* __restrict__ sds, const float* __restrict__ residual,
                                                 LayerArgs a, float* __restrict__ out, float* __restrict__ y) {
  using C = RowCfg<BITS, I>;
  constexpr int RB = C::RPW * P0;
  constexpr int P = P0 >= 2 ? P0 / 2 : 1;
  __shared__ float4 hs[2 * kWaves][I / 4];
  __shared__ float part[2 * kWaves][RB];
  const int t = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int sw = wave % kWaves, half = wave / kWaves;
  // Slots go in passes of kWaves: in pass q, wave w takes slot q*kWaves + w%4. The pass's SwiGLU
  // vectors are loaded once by the whole block with coalesced 16-byte loads and parked in LDS
  // (double-buffered over passes), instead of once per wave: the two halves of the block need
  // the same vectors, and a CU's time tracks the cache lines it requests.
  constexpr int N4 = I / 4;                                               // float4 per vector
  constexpr int HPER = (kWaves * N4 + 2 * kBlock - 1) / (2 * kBlock);     // float4 per thread per pass
  float4 hv0, hv1, hv2, hv3;  // HPER <= 4 (hidden rows of at most 2048 floats)
  static_assert(HPER <= 4, "SwiGLU vectors of at most 2048 floats");
  // A pass's SwiGLU vectors (past them: the last float4 again, stored again) and this wave's
  // expert index. They need only the leading arguments, which arrive preloaded in SGPRs, so pass
  // 0's requests leave first, before any kernel-argument fetch returns.
  auto request = [&](int q) __attribute__((always_inline)) {
    const int nk = min(ne - q * kWaves, kWaves);
    const float4* hsrc = reinterpret_cast<const float4*>(h + ((size_t)t * ne + q * kWaves) * I);
    hv0 = hsrc[min((int)threadIdx.x, nk * N4 - 1)];
    if constexpr (HPER > 1) hv1 = hsrc[min((int)threadIdx.x + 2 * kBlock, nk * N4 - 1)];
    if constexpr (HPER > 2) hv2 = hsrc[min((int)threadIdx.x + 4 * kBlock, nk * N4 - 1)];
    if constexpr (HPER > 3) hv3 = hsrc[min((int)threadIdx.x + 6 * kBlock, nk * N4 - 1)];
    return idx[(size_t)t * K + min(q * kWaves + sw, K - 1)];  // the shared slot reads one it ignores
  };
  int e = request(0);
  __builtin_amdgcn_sched_barrier(0);
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  const int row0 = blockIdx.x * RB + half * P * C::RPW;
  const bool combine = residual != nullptr;  // the host passes a residual exactly when out is set
  bool first = true;
  static_assert(RB <= 2 * kBlock, "one combined row per thread");
  float res = 0.0f;
  const bool active = !(P0 < 2 && half == 1);  // with one row step per block, the second half idles
  const int npass = (ne + kWaves - 1) / kWaves;
  int q = 0;
  do {  // at least one pass (ne >= 1), so pass 0's requests stay ahead of any branch
    const int k = q * kWaves + sw;
    const int nk = min(ne - q * kWaves, kWaves);  // slots in this pass
    if (q > 0) e = request(q);
    // Every wave issues its weight loads on every path (an idle wave repeats the rows of the pass's
    // last slot, a bad index reads expert 0's), so the wait before parking the vectors counts only
    // the vector loads issued before them.
    const bool work = active && k < ne;
    const int kk = min(k, ne - 1);
    // the shared slot's down rows come from preloaded arguments, so its waves request them at once;
    // a routed slot's wait for its index and the layout arguments together
    const bool routed = kk < K;
    bool valid = true;
    const uint8_t* dc = sdc;
    const uint8_t* ds = sds;
    if (routed) {
      valid = e >= 0 && e < a.E;
      const uint8_t* blob = a.experts + (size_t)(valid ? e : 0) * a.stride;
      dc = blob + a.off_codes[2];
      ds = blob + a.off_sb[2];
    }
    uint4 cw[P][C::CPL];
    uint32_t sb[P][C::CPL];
#pragma unroll
    for (int p = 0; p < P; ++p) load_row<C, FORM == 3>(dc, ds, min(row0 + p * C::RPW + rig, H - 1), lir, cw[p], sb[p]);
    __builtin_amdgcn_sched_barrier(0);
    // the residual row, behind this wave's weight loads: read at the end, it cost the combine a
    // memory round trip (decode4 13.96 -> 13.93, decodemx 19.09 -> 18.97 us/token); requested
    // first, together with the expert index, it delayed the weight loads (13.98 -> 14.50)
    if (q == 0 && combine && (int)threadIdx.x < RB && blockIdx.x * RB + threadIdx.x < H)
      res = residual[(size_t)t * H + blockIdx.x * RB + threadIdx.x];
    // the combine coefficient's address; the value is read after the barrier below, so that the
    // barrier does not wait for it
    const float* cp = routed ? a.ws.w + (size_t)t * K + kk : a.ws.g + t;
    auto park = [&](int j, const float4& hv) __attribute__((always_inline)) {
      const int i = min((int)threadIdx.x + j * 2 * kBlock, nk * N4 - 1);
      const int v = i / N4, f = i % N4;
      hs[(q & 1) * kWaves + v][xslot<C>(f / (C::CH / 4), f % (C::CH / 4))] = hv;
    };
    park(0, hv0);
    if constexpr (HPER > 1) park(1, hv1);
    if constexpr (HPER > 2) park(2, hv2);
    if constexpr (HPER > 3) park(3, hv3);
    __syncthreads();
    if (!work) continue;
    const float coef = combine ? *cp : 1.0f;
    float yv[P];
    if (valid) {
      float xr[C::XPL], S[C::CPL];
      read_act<C>(hs[(q & 1) * kWaves + sw], lir, xr, S);
#pragma unroll
      for (int p = 0; p < P; ++p) yv[p] = seg_sum<C::LPR>(row_partial<BITS, C, FORM>(cw[p], sb[p], xr, S));
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) yv[p] = NAN;
    }
    if (lir == C::LPR - 1) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int r = row0 + p * C::RPW + rig;
        if (r >= H) continue;
        if (combine) {
          const float v = coef * yv[p];
          const int i = half * P * C::RPW + p * C::RPW + rig;
          part[wave][i] = first ? v : part[wave][i] + v;
        } else {
          y[((size_t)t * ne + k) * H + r] = yv[p];
        }
      }
    }
    first = false;
  } while (++q < npass);
  if (!combine) return;
  __syncthreads();
  for (int i = threadIdx.x; i < RB; i += 2 * kBlock) {
    const int r = blockIdx.x * RB + i;
    if (r >= H) continue;
    const int hw = (i / (P * C::RPW)) * kWaves;
    float acc = res;
    for (int w = 0; w < kWaves && w < ne; ++w) acc += part[hw + w][i];
    store_through(&out[(size_t)t * H + r], acc);
  }
}

// ---- one token in two launches ---------------------------------------------------------------------
// Kernel 1 and kernel 2 above as one launch, k_front, followed by k_down. The launch has kFrontBlocks
// blocks, all resident at once (the host checks the occupancy before it takes this path). Block b
// computes router rows b and b + 256 and, after the top-K, SwiGLU outputs [4b, 4b + 4) of every
// expert slot, so it streams a 1/256 share of the router and of every selected gate/up matrix. The
// logits cross blocks inside the launch: each is stored as two 64-bit words, (tag, upper half) and
// (tag, lower half), with write-through (agent-scope) stores, and one wave per block polls the words
// themselves with agent-scope loads until every one carries this call's tag. There is no separate
// flag, fence or second round trip on that path. The tag is the call's sequence number + 1; the
// sequence word lives in the workspace's sync region and block 0 advances it at the end of the
// call, when every block has read it. The region starts zeroed, so a stale word never carries the
// current tag. The shared expert's rows need no routing and are requested at the start.
// The wait is bounded: a block that gives up writes NaN into its SwiGLU outputs (so the down kernel
// writes NaN rows) and marks the region, and every later call on it does the same until the region
// is zeroed again.
// Measured alternatives (decode4, same box): the down rows in the same launch, with the SwiGLU
// outputs handed over through per-block ready tags, 16.3-17.1 us/token against 14.1-14.4 here and
// 15.4 for the three-kernel chain (256 blocks polling the same tags and reading the same 16 KB from
// memory cost ~4 us, and the down compute then sits on the critical path); the top-K split over all
// 8 waves with a merge, 15.1 (2048 pollers contend, and the merge adds a barrier).
constexpr int kFrontBlocks = 256;
constexpr int kFrontWaves = 8;
constexpr size_t kSyncSeq = 0;       // uint32: calls completed on this workspace
constexpr size_t kSyncPoison = 128;  // uint32: nonzero once a call gave up
constexpr size_t kSyncLogits = 2048; // uint64[2 (E + 1)]: tagged halves of the fp64 logits
static_assert(kSyncLogits + 16 * (2 * kFrontBlocks + 1) <= MOE_WS_SYNC_BYTES, "sync region too small");
#ifndef BQ_SPIN_TICKS
#define BQ_SPIN_TICKS 2000000  // 20 ms of the 100 MHz real-time counter
#endif

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Repeats poll() (true once its condition holds) with a short sleep between tries, until it holds
// or about BQ_SPIN_TICKS of the 100 MHz real-time counter have passed. The counter is a scalar
// memory read, so it is read only every 64 tries.
template <class F>
__device__ __forceinline__ bool spin_poll(F poll) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 1;; ++it) {
    if (poll()) return true;
    if ((it & 63) == 0 && __builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)BQ_SPIN_TICKS) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}
__device__ __forceinline__ void store_logit(uint64_t* tl, int r, uint32_t tag, double v) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  store_through(&tl[2 * r], (uint64_t)(((uint64_t)tag << 32) | (bits >> 32)));
  store_through(&tl[2 * r + 1], (uint64_t)(((uint64_t)tag << 32) | (bits & 0xFFFFFFFFull)));
}

#ifdef BQ_TIMELINE  // measurement builds: per-block real-time stamps in the sync region's tail
#define BQ_TLT(k, th)                                                                                        \
  do {                                                                                                       \
    if (tid == (th)) reinterpret_cast<uint64_t*>(sync + 12288)[b * 10 + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define BQ_TLT(k, th) \
  do {                \
  } while (0)
#endif
#define BQ_TL(k) BQ_TLT(k, 0)

// norm: the stack's layers after the first route u = x / sqrt(mean(x^2) + eps) (unit-weight RMS
// norm), computed as in kernel 1: the logits are the fp64 dot products with x times the fp64 scale,
// and the experts read x times the scale rounded to fp32. The arguments of the first requests (x,
// the sync region, the router and shared-gate rows, E) lead the list, so they arrive preloaded in
// SGPRs and those requests leave before any kernel-argument fetch returns.
template <int BITS, int FORM, int K, int SH>
__global__ __launch_bounds__(64 * kFrontWaves) void k_front(const float* __restrict__ x, uint8_t* __restrict__ sync,
                                                            const uint16_t* __restrict__ router,
                                                            const uint16_t* __restrict__ sgate, int E, LayerArgs a,
                                                            int norm, float eps, int32_t* __restrict__ idx_out) {
  constexpr int H = 4096, I = 1024, NW = kFrontWaves, NT = 64 * NW, NE = K + SH;
  constexpr bool MX = FORM == 3;
  using Cg = RowCfg<BITS, H>;  // gate/up rows: one row per wave per step (64 lanes)
  using R = RouterCfg<H>;
  constexpr int HB = I / kFrontBlocks;  // SwiGLU outputs per block and slot
  constexpr int RCH = R::CPL / 4;       // router chunks per lane: a row over 4 waves
  constexpr int Q = Cg::CH / 4;         // float4 per gate/up chunk
  static_assert(Cg::LPR == 64 && Cg::RPW == 1 && 2 * HB == NW, "one gate or up row per wave and slot");
  static_assert(R::LPR == 64 && R::CPL % 4 == 0, "router rows over four waves");

  __shared__ float4 xs[H / 4];
  __shared__ double rpart[NW];
  __shared__ double gpart[4];
  __shared__ double psq[4];
  __shared__ float gu[NE][NW];
  __shared__ int32_t sel[MOE_MAX_TOP_K];
  __shared__ double val[MOE_MAX_TOP_K];
  __shared__ int ready, bail;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int nrows = E + SH;
  if (tid == 0) ready = bail = 0;  // read only after the first barrier below
  uint32_t* seqp = reinterpret_cast<uint32_t*>(sync + kSyncSeq);
  uint32_t* poisonp = reinterpret_cast<uint32_t*>(sync + kSyncPoison);
  uint64_t* tl = reinterpret_cast<uint64_t*>(sync + kSyncLogits);
  BQ_TL(0);

  // ---- requests that need no routing: the sequence word, x, router rows, the shared expert's rows
  const uint32_t seq = __hip_atomic_load(seqp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t poison = __hip_atomic_load(poisonp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  Stage<H, NT> st;
  st.load(x, tid);
  // router rows: waves 0-3 take row b, waves 4-7 row b + 256, each a quarter (the split of the
  // three-kernel router, so the logits are the same bit for bit); in block 0, when E = 512, waves
  // 0-3 also take the shared-gate row
  const int rrow = wave < 4 ? b : b + kFrontBlocks;
  const int piece = wave & 3;
  const bool third = SH && b == 0 && nrows > 2 * kFrontBlocks && wave < 4;
  uint4 rw[RCH], gw[RCH];
  {
    const int rr = min(rrow, nrows - 1);
    const uint16_t* row = rr < E ? router + (size_t)rr * H : sgate;
#pragma unroll
    for (int j = 0; j < RCH; ++j) rw[j] = *reinterpret_cast<const uint4*>(row + (lane + (j * 4 + piece) * 64) * 8);
    if (third) {
#pragma unroll
      for (int j = 0; j < RCH; ++j) gw[j] = *reinterpret_cast<const uint4*>(sgate + (lane + (j * 4 + piece) * 64) * 8);
    }
  }
  // gate/up rows: wave w takes matrix w / HB (gate, up), row HB*b + w % HB, in every slot
  const int gm = wave / HB;
  const int grow = b * HB + wave % HB;
  uint4 cg[NE][Cg::CPL];
  uint32_t sg[NE][Cg::CPL];
  if constexpr (SH) load_row<Cg, MX>(a.shared + a.off_codes[gm], a.shared + a.off_sb[gm], grow, lane, cg[K], sg[K]);
  __builtin_amdgcn_sched_barrier(0);
  st.template store<Cg>(xs, tid, 1.0f);
  __syncthreads();
  BQ_TL(1);
  const uint32_t tag = seq + 1u;
  auto give_up = [&]() __attribute__((always_inline)) {  // the whole block: NaN outputs, mark the region
    if (tid < NE * HB) store_through(&a.ws.h[(size_t)(tid / HB) * I + b * HB + tid % HB], (float)NAN);
    if (tid == 0) {
      store_through(poisonp, 1u);
      if (a.err != nullptr) *a.err = MOE_ETIMEOUT;
    }
  };
  if (poison != 0) {
    give_up();
    return;
  }

  // ---- router dot products in fp64 from the parked activations; the logits go out tagged
  {
    auto xchunk = [&](int c, float (&xv)[8]) __attribute__((always_inline)) {
      const float4 u = xs[xslot<Cg>((2 * c) / Q, (2 * c) % Q)], v = xs[xslot<Cg>((2 * c + 1) / Q, (2 * c + 1) % Q)];
      xv[0] = u.x; xv[1] = u.y; xv[2] = u.z; xv[3] = u.w; xv[4] = v.x; xv[5] = v.y; xv[6] = v.z; xv[7] = v.w;
    };
    auto rowdot = [&](const uint4 (&w)[RCH]) __attribute__((always_inline)) {
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int j = 0; j < RCH; ++j) {
        float xv[8];
        xchunk(lane + (j * 4 + piece) * 64, xv);
        const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[q] = fma((double)bf16_lo(ww[q]), (double)xv[2 * q], acc[q]);
          acc[q] = fma((double)bf16_hi(ww[q]), (double)xv[2 * q + 1], acc[q]);
        }
      }
      return seg_sum<64>((acc[0] + acc[1]) + (acc[2] + acc[3]));
    };
    if (norm && wave < 4) {  // waves 0-3 hold the whole vector between them, in kernel 1's order
      double ss = 0.0;
#pragma unroll
      for (int j = 0; j < RCH; ++j) {
        float xv[8];
        xchunk(lane + (j * 4 + piece) * 64, xv);
#pragma unroll
        for (int q = 0; q < 8; ++q) ss = fma((double)xv[q], (double)xv[q], ss);
      }
      ss = seg_sum<64>(ss);
      if (lane == 63) psq[wave] = ss;
    }
    const double t0 = rowdot(rw);
    if (lane == 63) rpart[wave] = t0;
    if (third) {
      const double t1 = rowdot(gw);
      if (lane == 63) gpart[wave] = t1;
    }
  }
  __syncthreads();
  const double scale = norm ? rms_inv(((psq[0] + psq[1]) + psq[2]) + psq[3], H, eps) : 1.0;
  if (lane == 0 && (wave == 0 || wave == 4)) {
    const int r = b + (wave == 4 ? kFrontBlocks : 0);
    const double v = ((rpart[wave] + rpart[wave + 1]) + rpart[wave + 2]) + rpart[wave + 3];
    if (r < nrows) store_logit(tl, r, tag, norm ? v * scale : v);
  }
  if (SH && b == 0 && nrows > 2 * kFrontBlocks && tid == 64) {
    const double v = ((gpart[0] + gpart[1]) + gpart[2]) + gpart[3];
    store_logit(tl, 2 * kFrontBlocks, tag, norm ? v * scale : v);
  }
  BQ_TL(2);

  // the shared expert's gate/up rows while the logits travel
  float xr[Cg::XPL], S[Cg::CPL];
  if (norm) read_act<Cg, true>(xs, lane, xr, S, (float)scale);
  else read_act<Cg>(xs, lane, xr, S);
  if constexpr (SH) {
    const float p = seg_sum<64>(row_partial<BITS, Cg, FORM>(cg[K], sg[K], xr, S));
    if (lane == 63) gu[K][wave] = p;
  }

  // ---- wave 0: wait for every logit, then the top-K. Each round's expert is published in LDS at
  // once (`ready` counts them, -1 if the wait gave up), and every wave requests that expert's rows
  // while the later rounds run.
  double gate_logit = 0.0;
  auto load_slot = [&](int s, int e) __attribute__((always_inline)) {
    const uint8_t* blob = a.experts + (size_t)e * a.stride;
    load_row<Cg, MX>(blob + a.off_codes[gm], blob + a.off_sb[gm], grow, lane, cg[s], sg[s]);
  };
  if (wave == 0) {
    double v[8];
    const bool done = spin_poll([&]() __attribute__((always_inline)) {
      uint32_t bad = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = lane + 64 * i;
        const int ee = min(e, E - 1);
        const uint64_t w0 = ld_agent(&tl[2 * ee]), w1 = ld_agent(&tl[2 * ee + 1]);
        bad |= (uint32_t)((w0 >> 32) != tag) | (uint32_t)((w1 >> 32) != tag);
        v[i] = e < E ? __longlong_as_double((long long)((w0 << 32) | (w1 & 0xFFFFFFFFull))) : -INFINITY;
      }
      if constexpr (SH) {
        const uint64_t w0 = ld_agent(&tl[2 * E]), w1 = ld_agent(&tl[2 * E + 1]);
        bad |= (uint32_t)((w0 >> 32) != tag) | (uint32_t)((w1 >> 32) != tag);
        gate_logit = __longlong_as_double((long long)((w0 << 32) | (w1 & 0xFFFFFFFFull)));
      }
      return __ballot(bad != 0) == 0;
    });
    BQ_TL(3);
    if (done) {
      uint64_t key[8];
      topk_keys<8>(v, E, lane, key);
      int es[K];
#pragma unroll
      for (int r = 0; r < K; ++r) {  // the values only in the block that writes the routing, afterwards
        es[r] = topk_round<8>(key, v, E, lane, r, true, sel, nullptr);
        if (lane == 0) __hip_atomic_store(&ready, r + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        load_slot(r, es[r]);
      }
      if (b == 0) {
#pragma unroll
        for (int r = 0; r < K; ++r) {
          const double wv = wave_value_at<8>(v, es[r]);
          if (lane == 0) val[r] = wv;
        }
      }
    } else if (lane == 0) {
      __hip_atomic_store(&ready, -1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  } else {
#pragma unroll
    for (int r = 0; r < K; ++r) {
      int n = 0;  // wave 0 always publishes K experts or -1; the bound is a backstop
      for (uint32_t it = 0; it < (1u << 24); ++it) {
        n = __hip_atomic_load(&ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (n > r || n < 0) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (n <= r) {  // the wait gave up (or, as a backstop, this wave did)
        if (n >= 0 && lane == 0) bail = 1;
        break;
      }
      load_slot(r, sel[r]);
    }
  }
  __syncthreads();
  if (ready != K || bail != 0) {
    give_up();
    return;
  }
  BQ_TL(4);

  // ---- the routed experts' gate/up rows, SwiGLU
  __builtin_amdgcn_sched_barrier(0);
  if (b == 0 && wave == 0)  // the routing for the down kernel, after this block's loads
    write_routing(a, 0, lane, sel, val, gate_logit, a.ws.idx, a.ws.w, idx_out, a.ws.g);
#pragma unroll
  for (int s = 0; s < K; ++s) {
    const float p = seg_sum<64>(row_partial<BITS, Cg, FORM>(cg[s], sg[s], xr, S));
    if (lane == 63) gu[s][wave] = p;
  }
  BQ_TL(5);
  __syncthreads();
  if (tid < NE * HB) {  // written through: the down kernel reads them next, mostly on other XCDs
    const int s = tid / HB, i = tid % HB;
    store_through(&a.ws.h[(size_t)s * I + b * HB + i], silu_mul(gu[s][i], gu[s][i + HB]));
  }
  if (b == 0 && tid == 0) store_through(seqp, tag);  // every block has read the sequence word by now
}

// Router-only top-K: one wave per token.
template <int PL>
__global__ __launch_bounds__(64) void k_topk(LayerArgs a, int32_t* __restrict__ idx, float* __restrict__ w,
                                             float* __restrict__ sg, double* __restrict__ logits_out,
                                             int32_t* __restrict__ idx_b) {
  __shared__ int32_t sel[MOE_MAX_TOP_K];
  __shared__ double val[MOE_MAX_TOP_K];
  const int t = blockIdx.x, lane = threadIdx.x;
  const double* lg = a.ws.logits + (size_t)t * (a.E + 1);
  double v[PL];
  load_topk_values<PL>(lg, a.E, lane, v);
  wave_topk<PL>(v, a.E, a.K, lane, -1, true, sel, val);
  if (logits_out)
    for (int e = lane; e < a.E; e += 64) logits_out[(size_t)t * a.E + e] = lg[e];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // lane 0's choices in LDS, for every lane
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  write_routing(a, t, lane, sel, val, lg[a.E], idx, w, idx_b, sg);
}

// fp64 norm of each bf16 router row (one wave per row), for the certified top-K's error bound.
__global__ __launch_bounds__(kBlock) void k_row_norms(int E, int H, const uint16_t* __restrict__ router,
                                                      double* __restrict__ rnorm) {
  const int e = blockIdx.x * kWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (e >= E) return;
  const uint16_t* row = router + (size_t)e * H;
  double ss = 0.0;
  for (int c = lane; c < H / 8; c += 64) {
    const uint4 w = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = bf16_lo(ww[q]), hi = bf16_hi(ww[q]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
  }
  ss = readlane_f64(seg_sum<64>(ss), 63);
  if (lane == 0) rnorm[e] = sqrt(ss);
}

// fp64 dot products of NR bf16 rows with the token's activations held in registers (chunk
// lane + 64j, 8 values each). The rows' loads are issued together; every lane returns the totals.
template <int H, int NR>
__device__ __forceinline__ void wave_rows_dot(const uint16_t* const (&rows)[NR],
                                              const float4 (&xr)[(H / 8 + 63) / 64][2], int lane, double (&out)[NR]) {
  constexpr int NCH = H / 8, XC = (NCH + 63) / 64;
  double acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.0;
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int ch = lane + 64 * j;
    if (NCH % 64 != 0 && ch >= NCH) continue;
    const float xv[8] = {xr[j][0].x, xr[j][0].y, xr[j][0].z, xr[j][0].w,
                         xr[j][1].x, xr[j][1].y, xr[j][1].z, xr[j][1].w};
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint4 w = *reinterpret_cast<const uint4*>(rows[r] + ch * 8);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[r] = fma((double)bf16_lo(ww[q]), (double)xv[2 * q], acc[r]);
        acc[r] = fma((double)bf16_hi(ww[q]), (double)xv[2 * q + 1], acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) out[r] = readlane_f64(seg_sum<64>(acc[r]), 63);
}

__device__ __forceinline__ double wave_min_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmin(v, __shfl_xor(v, m));
  return v;
}

// Certified top-K from approximate logits (one wave per token). ws.logits holds approximations
// l~_e with |l~_e - l_e| <= b_e = kc * |r_e| * |x| + (|r_e| + 1) * 2^-100 (Cauchy-Schwarz on the
// approximation's error bound, with the row norms |r_e| from k_row_norms). With A the K rows of
// largest l~ and LB = min over A of (l~_a - b_a), every a in A has l_a >= LB, so a row with
// l~_i + b_i < LB lies strictly below K rows and cannot be chosen. The other rows (A itself and
// any row the bound cannot separate) are recomputed exactly in fp64 and the top-K is taken over
// them: the same choice as a top-K over every row's fp64 logit. A non-finite approximation or
// bound makes every row a candidate. The shared-gate logit (row id E in the list) is computed in
// fp64 with A's rows.
constexpr int kCertBatch = 4;  // rows recomputed together
template <int PL, int H>
__global__ __launch_bounds__(kBlock) void k_topk_certified(LayerArgs a, const float* __restrict__ x,
                                                           const double* __restrict__ rnorm, double kc, int T,
                                                           int32_t* __restrict__ idx, float* __restrict__ w,
                                                           float* __restrict__ sg, int32_t* __restrict__ idx_b) {
  constexpr int NCH = H / 8, XC = (NCH + 63) / 64;
  constexpr int kList = 64 * PL + MOE_MAX_TOP_K + 1;  // every row, the gate row, and room for A twice
  __shared__ int32_t sel[kWaves][MOE_MAX_TOP_K];
  __shared__ double val[kWaves][MOE_MAX_TOP_K];
  __shared__ int32_t list[kWaves][kList];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * kWaves + wave;
  if (t >= T) return;  // wave-uniform; the kernel has no block barrier
  const double* lg = a.ws.logits + (size_t)t * (a.E + 1);
  double la[PL], rn[PL];
  load_topk_values<PL>(lg, a.E, lane, la);
#pragma unroll
  for (int i = 0; i < PL; ++i) rn[i] = rnorm[min(lane + 64 * i, a.E - 1)];
  float4 xr[XC][2];
  double xx = 0.0;
#pragma unroll
  for (int j = 0; j < XC; ++j) {
    const int ch = min(lane + 64 * j, NCH - 1);
    const float4* p = reinterpret_cast<const float4*>(x + (size_t)t * H + ch * 8);
    xr[j][0] = p[0];
    xr[j][1] = p[1];
    if (NCH % 64 != 0 && lane + 64 * j >= NCH) continue;
    const float xv[8] = {xr[j][0].x, xr[j][0].y, xr[j][0].z, xr[j][0].w,
                         xr[j][1].x, xr[j][1].y, xr[j][1].z, xr[j][1].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) xx = fma((double)xv[q], (double)xv[q], xx);
  }
  const double xn = sqrt(readlane_f64(seg_sum<64>(xx), 63));
  double bnd[PL];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    bnd[i] = kc * rn[i] * xn + (rn[i] + 1.0) * 0x1p-100;
    if (lane + 64 * i < a.E && !(__builtin_isfinite(la[i]) && __builtin_isfinite(bnd[i]))) bad = true;
  }
  // The list of rows to recompute: A (or, after a non-finite value, every row), the gate row
  // (id E), then the rows the bound cannot separate from A.
  int32_t* lst = list[wave];
  int n = 0;
  bool extra[PL];
  if (__ballot(bad) == 0) {
    double v[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) v[i] = la[i];
    wave_topk<PL>(v, a.E, a.K, lane, -1, true, sel[wave], val[wave]);  // the K best become -inf
    // lane 0 recorded the choices in LDS; the other lanes read them below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double lb = INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (lane + 64 * i < a.E && v[i] == -INFINITY) lb = fmin(lb, la[i] - bnd[i]);
    lb = wave_min_f64(lb);
#pragma unroll
    for (int i = 0; i < PL; ++i) extra[i] = lane + 64 * i < a.E && v[i] != -INFINITY && la[i] + bnd[i] >= lb;
    if (lane < a.K) lst[lane] = sel[wave][lane];
    n = a.K;
  } else {
#pragma unroll
    for (int i = 0; i < PL; ++i) extra[i] = lane + 64 * i < a.E;
  }
  if (a.has_shared) {  // the shared-gate row
    if (lane == 0) lst[n] = a.E;
    n += 1;
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint64_t m = __ballot(extra[i]);
    if (extra[i]) lst[n + __popcll(m & ((1ull << lane) - 1))] = lane + 64 * i;
    n += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double ex[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) ex[i] = -INFINITY;
  double gl = 0.0;
  for (int b = 0; b < n; b += kCertBatch) {
    int id[kCertBatch];
    const uint16_t* rows[kCertBatch];
#pragma unroll
    for (int q = 0; q < kCertBatch; ++q) {
      id[q] = lst[min(b + q, n - 1)];  // past the end: the last row again, its result unused
      rows[q] = id[q] < a.E ? a.router + (size_t)id[q] * H : a.sgate;  // id E only with a shared gate
    }
    double d[kCertBatch];
    wave_rows_dot<H, kCertBatch>(rows, xr, lane, d);
#pragma unroll
    for (int q = 0; q < kCertBatch; ++q) {
      if (id[q] == a.E) {
        gl = d[q];
        continue;
      }
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (id[q] == lane + 64 * i) ex[i] = d[q];
    }
  }
  wave_topk<PL>(ex, a.E, a.K, lane, -1, true, sel[wave], val[wave]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // lane 0's choices in LDS, for every lane
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  write_routing(a, t, lane, sel[wave], val[wave], gl, idx, w, idx_b, sg);
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

// MXFP4: w = e2m1(q) * 2^(e - 127), exact in fp32 for the E8M0 range of normal floats.
__global__ void k_dequant_mx(int rows, int cols, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ sc,
                             int out_dtype, void* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * cols) return;
  const int64_t r = i / cols, c = i % cols;
  const uint32_t byte = codes[(r * cols + c) / 2];
  const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
  const float v = (c & 1 ? v2[1] : v2[0]) * e8m0_value(sc[r * (cols / 32) + c / 32]);
  if (out_dtype == 0) {
    static_cast<float*>(out)[i] = v;
  } else {
    uint32_t b = __float_as_uint(v);
    b += 0x7FFFu + ((b >> 16) & 1u);  // round to nearest even (finite values)
    static_cast<uint16_t*>(out)[i] = (uint16_t)(b >> 16);
  }
}

__global__ void k_zero16(int64_t n, uint4* __restrict__ p) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void k_pack_e8m0(int64_t n, const uint16_t* __restrict__ s, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = (uint8_t)s[i];
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
#define BQ_FOR_I(X) X(64) X(128) X(256) X(512) X(1024) X(2048)

// Row steps per down wave: enough for 16 output rows per block (so hidden 4096 gives 256 blocks,
// one per CU), at most BQ_P3 (the bytes each wave has in flight, tuned on MI355X for the 4096/1024
// 4-bit shape). A 2-bit row of 1024 is 16 lanes wide, so its waves take 4 steps of 4 rows. With more
// expert slots than waves (top-6 + shared), each wave takes two slots in turn, and blocks of 8 rows
// (two per CU) measured 5% faster per token.
#ifndef BQ_P3
#define BQ_P3 8
#endif
#ifndef BQ_ROUTER_STEPS
#define BQ_ROUTER_STEPS 1
#endif
template <int RPW, int ROWS>
constexpr int down_steps() { return ROWS / RPW < 1 ? 1 : (ROWS / RPW > BQ_P3 ? BQ_P3 : ROWS / RPW); }
// Tokens per block of the multi-token router (k_router_group).
#ifndef BQ_ROUTER_GROUP
#define BQ_ROUTER_GROUP 4
#endif
#ifndef BQ_ROUTER_GROUP_MIN_TOKENS
#define BQ_ROUTER_GROUP_MIN_TOKENS BQ_ROUTER_GROUP
#endif
constexpr int kRouterGroup = BQ_ROUTER_GROUP;

// A launch that, when events are given, has the dispatch itself record its start and end time
// (the same timestamps a kernel-trace profiler reports), not separate event packets around it.
template <typename F, typename... Args>
hipError_t launch_timed(F kernel, dim3 grid, dim3 block, hipStream_t s, const KernelEvents& ev, Args... args) {
  if (ev.start != nullptr || ev.stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

template <int BITS, int H>
hipError_t router_phase_impl(const LayerArgs& a, const float* x, const float* norm_src, float eps, int T,
                             hipStream_t s, const KernelEvents& ev) {
  using R = RouterCfg<H>;
  const int router_steps = BQ_ROUTER_STEPS;
  const int nrows = a.E + a.has_shared;
  constexpr int SPLIT = (R::CPL % BQ_ROUTER_SPLIT == 0) ? BQ_ROUTER_SPLIT : 1;
  const int rows_per_block = kWaves / SPLIT * router_steps * R::RPW;
  const int nrb = (nrows + rows_per_block - 1) / rows_per_block;
  if (norm_src == nullptr && T >= BQ_ROUTER_GROUP_MIN_TOKENS && router_steps == 1) {  // one read per token group
    return launch_timed(k_router_group<H, kRouterGroup>, dim3(nrb, (T + kRouterGroup - 1) / kRouterGroup),
                        dim3(kBlock), s, ev, x, (const uint16_t*)a.router, (const uint16_t*)a.sgate, a.E,
                        a.E + a.has_shared, T, a);
  }
  return launch_timed(k_router_phase<H>, dim3(nrb, T), dim3(kBlock), s, ev, norm_src != nullptr ? norm_src : x,
                      (const uint16_t*)a.router, (const uint16_t*)a.sgate, a.E, a.E + a.has_shared, router_steps, a,
                      x, norm_src, eps);
}

// Waves per gate/up block: 8 (two per SIMD, so one computes while the other waits), except where a
// row's registers would not fit two waves per SIMD (hidden 8192) or a block would hold fewer rows than
// waves' worth of lanes (hidden 256).
#ifndef BQ_GATEUP_WAVES
#define BQ_GATEUP_WAVES 8
#endif
template <int BITS, int H>
hipError_t gateup_impl(const LayerArgs& a, const float* x, int T, const int32_t* idx_in, int32_t* idx_out,
                       bool with_shared, hipStream_t s, const KernelEvents& ev) {
  constexpr int NW = (H >= 64 * BQ_GATEUP_WAVES && H <= 4096) ? BQ_GATEUP_WAVES : 4;
  const int slots = a.K + ((with_shared && a.has_shared) ? 1 : 0);
  const dim3 grid(a.I / kSlice, slots, T), block(64 * NW);
#define BQ_GU(PL, F) \
  launch_timed(k_gateup<BITS, H, F, PL, NW>, grid, block, s, ev, (const double*)a.ws.logits, x, idx_in, a.E, a.K, a, \
               idx_out)
  if constexpr (BITS == 4) {
    if (a.form == 3) return a.E <= 512 ? BQ_GU(8, 3) : BQ_GU(16, 3);
  }
  if (a.E <= 512) return a.form == 1 ? BQ_GU(8, 1) : a.form == 2 ? BQ_GU(8, 2) : BQ_GU(8, 0);
  return a.form == 1 ? BQ_GU(16, 1) : a.form == 2 ? BQ_GU(16, 2) : BQ_GU(16, 0);
#undef BQ_GU
}

template <int BITS, int I>
hipError_t down_impl(const LayerArgs& a, int T, const int32_t* idx, const float* residual, float* out, float* y,
                     hipStream_t s, const KernelEvents& ev) {
  using C = RowCfg<BITS, I>;
  constexpr int P16 = down_steps<C::RPW, 16>(), P8 = down_steps<C::RPW, 8>();
  const bool two_rounds = a.NE > kWaves;
  const int RB = C::RPW * (two_rounds ? P8 : P16);
  const int nb = (a.H + RB - 1) / RB;
#define BQ_DN(P, F) launch_timed(k_down<BITS, I, P, F>, dim3(nb, T), dim3(2 * kBlock), s, ev, (const float*)a.ws.h, idx, a.NE, a.K, a.H, \
                                        (const uint8_t*)a.shared + a.off_codes[2], (const uint8_t*)a.shared + a.off_sb[2], \
                                        residual, a, out, y)
  if constexpr (BITS == 4) {
    if (a.form == 3) return two_rounds ? BQ_DN(P8, 3) : BQ_DN(P16, 3);
  }
  if (two_rounds) return a.form == 1 ? BQ_DN(P8, 1) : a.form == 2 ? BQ_DN(P8, 2) : BQ_DN(P8, 0);
  return a.form == 1 ? BQ_DN(P16, 1) : a.form == 2 ? BQ_DN(P16, 2) : BQ_DN(P16, 0);
#undef BQ_DN
}


// The two-launch decode's first kernel: 4-bit and 2-bit affine top-3 and MXFP4 top-6 layers, with a
// shared expert, H 4096, I 1024.
template <int BITS, int FORM, int K>
constexpr auto front_kernel() { return k_front<BITS, FORM, K, 1>; }

// Whether every block of k_front (kFrontBlocks blocks of 512 threads) can be resident at once on
// the current device: the occupancy per CU times the CU count, looked up once per device.
template <int BITS, int FORM, int K>
bool front_resident() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static signed char known[kMaxDevices] = {};  // 0 unknown, 1 yes, -1 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    int cus = 0, per_cu = 0;
    const bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, front_kernel<BITS, FORM, K>(), 64 * kFrontWaves, 0) ==
                        hipSuccess &&
                    (long)cus * per_cu >= kFrontBlocks;
    known[dev] = ok ? 1 : -1;
  }
  return known[dev] > 0;
}
}  // namespace

hipError_t launch_router_phase(const Geometry& g, const LayerPtrs& p, const float* x, const float* norm_src,
                               float eps, int T, const Workspace& ws, hipStream_t s, const KernelEvents& ev) {
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(HV)                                                                                  \
  case HV:                                                                                           \
    return g.bits == 4 ? router_phase_impl<4, HV>(a, x, norm_src, eps, T, s, ev)                     \
                       : router_phase_impl<2, HV>(a, x, norm_src, eps, T, s, ev);
  switch (g.H) { BQ_FOR_H(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_gateup(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                         const int32_t* idx_in, int32_t* idx_out, bool with_shared, int32_t* err, hipStream_t s,
                         const KernelEvents& ev) {
  LayerArgs a = make_args(g, p, ws);
  a.err = err;
#define BQ_CASE(HV)                                                                              \
  case HV:                                                                                       \
    return g.bits == 4 ? gateup_impl<4, HV>(a, x, T, idx_in, idx_out, with_shared, s, ev)        \
                       : gateup_impl<2, HV>(a, x, T, idx_in, idx_out, with_shared, s, ev);
  switch (g.H) { BQ_FOR_H(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_down(const Geometry& g, const LayerPtrs& p, int T, const Workspace& ws, const int32_t* idx,
                       const float* residual, float* out, float* y, hipStream_t s, const KernelEvents& ev) {
  if ((residual == nullptr) != (out == nullptr)) return hipErrorInvalidValue;  // k_down combines iff residual
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(IV)                                                                        \
  case IV:                                                                                 \
    return g.bits == 4 ? down_impl<4, IV>(a, T, idx, residual, out, y, s, ev)              \
                       : down_impl<2, IV>(a, T, idx, residual, out, y, s, ev);
  switch (g.I) { BQ_FOR_I(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

bool pair_supported(const Geometry& g) {
  if (g.H != 4096 || g.I != 1024 || g.E > 2 * kFrontBlocks || !g.has_shared || g.chain) return false;
  if (g.form == 0 && g.K == 3 && g.G == 64)
    return g.bits == 4 ? front_resident<4, 0, 3>() : g.bits == 2 ? front_resident<2, 0, 3>() : false;
  if (g.form == 3 && g.K == 6) return front_resident<4, 3, 6>();
  return false;
}

hipError_t launch_pair(const Geometry& g, const LayerPtrs& p, const float* x, const float* norm_src, float eps,
                       const float* residual, float* out, int32_t* idx_out, const Workspace& ws, uint8_t* sync,
                       int32_t* err, hipStream_t s, const KernelEvents& ev_front, const KernelEvents& ev_down) {
  LayerArgs a = make_args(g, p, ws);
  a.err = err;
  const dim3 grid(kFrontBlocks), block(64 * kFrontWaves);
  const float* in = norm_src != nullptr ? norm_src : x;
  const int norm = norm_src != nullptr;
  hipError_t e;
  if (g.form == 3)
    e = launch_timed(front_kernel<4, 3, 6>(), grid, block, s, ev_front, in, sync, p.router, p.sgate, g.E, a, norm,
                     eps, idx_out);
  else if (g.bits == 4)
    e = launch_timed(front_kernel<4, 0, 3>(), grid, block, s, ev_front, in, sync, p.router, p.sgate, g.E, a, norm,
                     eps, idx_out);
  else
    e = launch_timed(front_kernel<2, 0, 3>(), grid, block, s, ev_front, in, sync, p.router, p.sgate, g.E, a, norm,
                     eps, idx_out);
  if (e != hipSuccess) return e;
  return launch_down(g, p, 1, ws, ws.idx, residual, out, nullptr, s, ev_down);
}

hipError_t launch_topk(const Geometry& g, int T, const Workspace& ws, int32_t* idx, float* w, float* sg,
                       double* logits_out, int32_t* idx_b, hipStream_t s) {
  LayerPtrs p{};
  const LayerArgs a = make_args(g, p, ws);
  if (g.E <= 512)
    hipLaunchKernelGGL(k_topk<8>, dim3(T), dim3(64), 0, s, a, idx, w, sg, logits_out, idx_b);
  else
    hipLaunchKernelGGL(k_topk<16>, dim3(T), dim3(64), 0, s, a, idx, w, sg, logits_out, idx_b);
  return hipGetLastError();
}

hipError_t launch_topk_certified(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                 double kc, int32_t* idx, float* w, float* sg, int32_t* idx_b, hipStream_t s) {
  const LayerArgs a = make_args(g, p, ws);
  hipLaunchKernelGGL(k_row_norms, dim3((g.E + kWaves - 1) / kWaves), dim3(kBlock), 0, s, g.E, g.H, p.router, ws.rnorm);
  const dim3 grid((T + kWaves - 1) / kWaves);
#define BQ_CASE(HV)                                                                                              \
  case HV:                                                                                                       \
    if (g.E <= 512)                                                                                              \
      hipLaunchKernelGGL((k_topk_certified<8, HV>), grid, dim3(kBlock), 0, s, a, x, ws.rnorm, kc, T, idx, w, sg, idx_b); \
    else                                                                                                         \
      hipLaunchKernelGGL((k_topk_certified<16, HV>), grid, dim3(kBlock), 0, s, a, x, ws.rnorm, kc, T, idx, w, sg, idx_b); \
    return hipGetLastError();
  switch (g.H) { BQ_FOR_H(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
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
  if (g.form == 3) {
    hipLaunchKernelGGL(k_dequant_mx, dim3(blocks_for(n, 256)), dim3(256), 0, s, rows, cols, blob + g.off_codes[matrix],
                       blob + g.off_sb[matrix], out_dtype, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_dequant, dim3(blocks_for(n, 256)), dim3(256), 0, s, rows, cols, g.bits,
                     blob + g.off_codes[matrix], reinterpret_cast<const uint32_t*>(blob + g.off_sb[matrix]), out_dtype,
                     out);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t n, hipStream_t s) {
  const int64_t n4 = (int64_t)(n / 16);
  hipLaunchKernelGGL(k_zero16, dim3(blocks_for(n4, 256)), dim3(256), 0, s, n4, static_cast<uint4*>(p));
  return hipGetLastError();
}

hipError_t launch_pack(int H, int I, int bits, int G, const moe_expert_arrays_t* arr, uint8_t* blob, hipStream_t s) {
  const int64_t code_bytes = (int64_t)I * H * bits / 8;
  const int64_t ngroups = (int64_t)I * H / G;
  for (int m = 0; m < 3; ++m) {
    hipLaunchKernelGGL(k_pack_codes, dim3(blocks_for(code_bytes, 256)), dim3(256), 0, s, code_bytes, bits, arr->q[m],
                       blob + m * code_bytes);
    if (G == 32) {  // MXFP4: one E8M0 byte per block
      hipLaunchKernelGGL(k_pack_e8m0, dim3(blocks_for(ngroups, 256)), dim3(256), 0, s, ngroups, arr->scale[m],
                         blob + 3 * code_bytes + m * ngroups);
      continue;
    }
    hipLaunchKernelGGL(k_pack_sb, dim3(blocks_for(ngroups, 256)), dim3(256), 0, s, ngroups, arr->scale[m],
                       arr->bias[m], reinterpret_cast<uint32_t*>(blob + 3 * code_bytes + m * ngroups * 4));
  }
  return hipGetLastError();
}

}  // namespace bqmoe

// Workspace of moe_layer_forward_noalloc: a fixed device array, one copy per GPU, held until the
// process ends. Host code must not pass `scratch` itself to a kernel (in host code the name is a
// stand-in, not a device address); noalloc_scratch looks up each device's address once.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace bqmoe {

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace bqmoe
