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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

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
template <class C>
__device__ __forceinline__ void read_act(const float4* __restrict__ xs, int lir, float (&xr)[C::XPL],
                                         float (&S)[C::CPL]) {
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    const int chunk = lir + j * C::LPR;
#pragma unroll
    for (int q = 0; q < C::CH / 4; ++q) {
      const float4 t = xs[xslot<C>(chunk, q)];
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

struct LayerArgs {
  int H, I, E, K, NE, has_shared, form;
  uint64_t off_codes[3], off_sb[3];
  const uint8_t* experts;
  uint64_t stride;
  const uint8_t* shared;
  const uint16_t* router;
  const uint16_t* sgate;
  Workspace ws;
};

// Cross-layer prefetch: the grid reads the two regions (as one concatenated range, split evenly over
// the blocks, 4 KiB per block pass) so that their lines are filled into the memory-side cache, and
// discards the data. 8 loads per thread are in flight at a time.
__global__ __launch_bounds__(kBlock) void k_prefetch(Prefetch pf) {
  const uint64_t total = pf.bytes[0] + pf.bytes[1];
  const uint64_t per = ((total + gridDim.x - 1) / gridDim.x + 4095) & ~(uint64_t)4095;
  const uint64_t lo = (uint64_t)blockIdx.x * per, hi = lo + per < total ? lo + per : total;
  uint32_t acc = 0;
  for (uint64_t base = lo; base < hi; base += 8 * 4096) {
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint64_t off = base + (uint64_t)i * 4096 + threadIdx.x * 16;
      if (off + 16 > hi) off = lo;  // past the range: re-read its first line
      const uint8_t* src = off < pf.bytes[0] ? pf.ptr[0] + off : pf.ptr[1] + (off - pf.bytes[0]);
      v[i] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v[i].x ^ v[i].w;
  }
  asm volatile("" ::"v"(acc));  // keeps the loads
}

LayerArgs make_args(const Geometry& g, const LayerPtrs& p, const Workspace& ws) {
  LayerArgs a;
  a.H = g.H; a.I = g.I; a.E = g.E; a.K = g.K; a.NE = g.NE; a.has_shared = g.has_shared; a.form = g.form;
  for (int m = 0; m < 3; ++m) { a.off_codes[m] = g.off_codes[m]; a.off_sb[m] = g.off_sb[m]; }
  a.experts = p.experts; a.stride = p.stride; a.shared = p.shared; a.router = p.router; a.sgate = p.sgate;
  a.ws = ws;
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

// Softmax of the K chosen logits (the full softmax over E renormalised over the chosen set reduces to
// this), written with the choices and the shared gate for token t. One lane calls this.
__device__ __forceinline__ void write_routing(const LayerArgs& a, int t, const int32_t* __restrict__ sel,
                                              const double* __restrict__ val, const double* __restrict__ lg,
                                              int32_t* __restrict__ idx_a, float* __restrict__ w_a,
                                              int32_t* __restrict__ idx_b, float* __restrict__ g_out) {
  double z = 0.0;
  for (int k = 0; k < a.K; ++k) z += exp(val[k] - val[0]);
  for (int k = 0; k < a.K; ++k) {
    idx_a[(size_t)t * a.K + k] = sel[k];
    w_a[(size_t)t * a.K + k] = (float)(exp(val[k] - val[0]) / z);
    if (idx_b) idx_b[(size_t)t * a.K + k] = sel[k];
  }
  if (g_out && a.has_shared) g_out[t] = (float)(1.0 / (1.0 + exp(-lg[a.E])));
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

// gate/up/SwiGLU for P row steps of one expert, for a whole block: weight loads go out first,
// then the staged activations are parked in LDS (one barrier) and read back per lane.
template <int BITS, int H, int P, int FORM>
__device__ __forceinline__ void gateup_block(const LayerArgs& a, const uint8_t* __restrict__ blob,
                                             const Stage<H, kBlock>& st, float scale, float4* __restrict__ xs,
                                             int step0, int lir, int rig, float* __restrict__ h) {
  using C = RowCfg<BITS, H>;
  const uint8_t* gc = blob + a.off_codes[0];
  const uint8_t* uc = blob + a.off_codes[1];
  const uint8_t* gs = blob + a.off_sb[0];
  const uint8_t* us = blob + a.off_sb[1];
  uint4 cg[P][C::CPL], cu[P][C::CPL];
  uint32_t sg[P][C::CPL], su[P][C::CPL];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = min((step0 + p) * C::RPW + rig, a.I - 1);  // rows past the end re-read the last row
    load_row<C, FORM == 3>(gc, gs, r, lir, cg[p], sg[p]);
    load_row<C, FORM == 3>(uc, us, r, lir, cu[p], su[p]);
  }
  __builtin_amdgcn_sched_barrier(0);
  st.template store<C>(xs, threadIdx.x, scale);
  __syncthreads();
  float xr[C::XPL], S[C::CPL];
  read_act<C>(xs, lir, xr, S);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int r = (step0 + p) * C::RPW + rig;
    const float ga = seg_sum<C::LPR>(row_partial<BITS, C, FORM>(cg[p], sg[p], xr, S));
    const float ua = seg_sum<C::LPR>(row_partial<BITS, C, FORM>(cu[p], su[p], xr, S));
    if (lir == C::LPR - 1 && r < a.I) h[r] = silu_mul(ga, ua);
  }
}

// ---------------------------------------------------------------------------------------------
// Kernel 1: router logits and the shared-gate logit (row E), accumulated in fp64. In a stack the
// input is RMS-normalised first, and the blocks together store the normalised vector for kernel 2.
#ifndef BQ_ROUTER_SPLIT
#define BQ_ROUTER_SPLIT 4
#endif
template <int H>
__global__ __launch_bounds__(kBlock) void k_router_phase(LayerArgs a, const float* __restrict__ x,
                                                         const float* __restrict__ norm_src, float eps,
                                                         int router_steps) {
  using R = RouterCfg<H>;
  constexpr int SPLIT = (R::CPL % BQ_ROUTER_SPLIT == 0) ? BQ_ROUTER_SPLIT : 1;  // waves per row
  constexpr int CPW = R::CPL / SPLIT;                                            // chunks per lane
  __shared__ double part[kWaves];
  __shared__ double psq[kWaves];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % R::LPR, rig = lane / R::LPR;
  const int nrows = a.E + a.has_shared;
  const int piece = wave % SPLIT;
  auto row_of = [&](int s) {
    const int base = ((blockIdx.x * (kWaves / SPLIT) + wave / SPLIT) * router_steps + s) * R::RPW;
    return base + rig;
  };
  auto load_w = [&](int s, uint4 (&w)[CPW]) {
    const int rr = min(row_of(s), nrows - 1);
    const uint16_t* row = (rr < a.E) ? a.router + (size_t)rr * H : a.sgate;
#pragma unroll
    for (int j = 0; j < CPW; ++j) w[j] = *reinterpret_cast<const uint4*>(row + (lir + (j * SPLIT + piece) * R::LPR) * 8);
  };
  // The norm's scale is a scalar, so a row's dot product with the raw input is taken first and
  // scaled at the end: sum_j R[e][j] (s h_j) = s sum_j R[e][j] h_j, with every product exact in fp64.
  const bool norm = norm_src != nullptr;
  const float* src = (norm ? norm_src : x) + (size_t)t * H;
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
      if (lir == R::LPR - 1 && r < nrows) a.ws.logits[(size_t)t * (a.E + 1) + r] = norm ? tot * scale : tot;
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
        a.ws.logits[(size_t)t * (a.E + 1) + r] = norm ? v * scale : v;
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
// traffic drops, from T reads of the router to T / TG.
template <int H, int TG>
__global__ __launch_bounds__(kBlock) void k_router_group(LayerArgs a, const float* __restrict__ x, int T) {
  using R = RouterCfg<H>;
  constexpr int SPLIT = (R::CPL % BQ_ROUTER_SPLIT == 0) ? BQ_ROUTER_SPLIT : 1;  // waves per row
  constexpr int CPW = R::CPL / SPLIT;                                            // chunks per lane
  __shared__ double part[TG][kWaves];
  const int t0 = blockIdx.y * TG;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % R::LPR, rig = lane / R::LPR;
  const int nrows = a.E + a.has_shared;
  const int piece = wave % SPLIT;
  const int r = (blockIdx.x * (kWaves / SPLIT) + wave / SPLIT) * R::RPW + rig;  // one row step per block
  uint4 w[CPW];
  {
    const int rr = min(r, nrows - 1);
    const uint16_t* row = (rr < a.E) ? a.router + (size_t)rr * H : a.sgate;
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
        if (t0 + g < T) a.ws.logits[(size_t)(t0 + g) * (a.E + 1) + r] = tot[g];
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
        a.ws.logits[(size_t)(t0 + g) * (a.E + 1) + r] = v;
      }
    }
  }
}

// Kernel 2: gate/up/SwiGLU of the routed experts (blockIdx.y = slot) and, as slot K, of the shared
// expert. The shared slot needs no routing, so its blocks stream weights while the routed blocks are
// still picking their experts.
template <int BITS, int H, int P, int PL, int FORM>
__global__ __launch_bounds__(kBlock) void k_gateup(LayerArgs a, const float* __restrict__ x,
                                                   const int32_t* __restrict__ idx_in, int32_t* __restrict__ idx_out) {
  using C = RowCfg<BITS, H>;
  __shared__ float4 xs[H / 4];
  __shared__ int32_t sel[MOE_MAX_TOP_K];
  __shared__ double val[MOE_MAX_TOP_K];
  // Dispatch order of the routed slots. Slot s needs top-K rounds 0..s. With many routed experts
  // (K > 4) the slots go in reverse, so the ones with the most rounds start first; with few, in
  // order. Measured: top-6 40.7k -> 43.9k tokens/s reversed; top-3 64.7k in order against 63.7k.
  // The first slot dispatched records the routing; the shared expert's slot K stays last.
  const int t = blockIdx.z;
  const bool reversed = a.K > 4;
  const int slot = reversed && (int)blockIdx.y < a.K ? a.K - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  const int step0 = (blockIdx.x * kWaves + wave) * P;
  const uint8_t* blob = a.shared;
  Stage<H, kBlock> st;
  // One wave records the choices (LDS) and writes the routing for the next kernel after its block's
  // gate/up work: written before it, the softmax's fp64 exps and the gate logit's load would hold
  // back this block's weight loads, and the block's barrier the other waves'.
  bool writer = false;
  if (slot < a.K) {
    int e;
    if (idx_in != nullptr) {
      e = idx_in[(size_t)t * a.K + slot];
      st.load(x + (size_t)t * H, threadIdx.x);
    } else {
      const double* lg = a.ws.logits + (size_t)t * (a.E + 1);
      // the logits are requested first, so waiting for them never waits for the activations
      double v[PL];
      load_topk_values<PL>(lg, a.E, lane, v);
      st.load(x + (size_t)t * H, threadIdx.x);
      writer = blockIdx.x == 0 && blockIdx.y == 0 && wave == 0;  // the first routed slot dispatched
      // slot s needs rounds 0..s only; the writer takes all K to record the routing
      e = wave_topk<PL>(v, a.E, writer ? a.K : slot + 1, lane, slot, writer, sel, val);
    }
    if (e < 0 || e >= a.E) {  // never read outside the pool: mark the slot's output as invalid
      for (int p = 0; p < P; ++p) {
        const int r = (step0 + p) * C::RPW + rig;
        if (r < a.I && lir == C::LPR - 1) a.ws.h[((size_t)t * a.NE + slot) * a.I + r] = NAN;
      }
      return;  // the whole block takes this branch (slot is per block)
    }
    blob = a.experts + (size_t)e * a.stride;
  } else {
    st.load(x + (size_t)t * H, threadIdx.x);
  }
  gateup_block<BITS, H, P, FORM>(a, blob, st, 1.0f, xs, step0, lir, rig, a.ws.h + ((size_t)t * a.NE + slot) * a.I);
  if (writer && lane == 0)
    write_routing(a, t, sel, val, a.ws.logits + (size_t)t * (a.E + 1), a.ws.idx, a.ws.w, idx_out, a.ws.g);
}

// Kernel 3: down projections of all expert slots for a block of output rows; combine or store.
// Wave w handles slots w, w+4, ...; each stages its slot's SwiGLU vector through its own LDS region.
template <int BITS, int I, int P, int FORM>
__global__ __launch_bounds__(kBlock) void k_down(LayerArgs a, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ residual, float* __restrict__ out,
                                                 float* __restrict__ y) {
  using C = RowCfg<BITS, I>;
  constexpr int RB = C::RPW * P;
  __shared__ float4 hs[kWaves][I / 4];
  __shared__ float part[kWaves][RB];
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lir = lane % C::LPR, rig = lane / C::LPR;
  const int row0 = blockIdx.x * RB;
  const bool combine = out != nullptr;
  bool first = true;
  for (int k = wave; k < a.NE; k += kWaves) {
    const uint8_t* blob = a.shared;
    bool valid = true;
    float coef = 1.0f;
    if (k < a.K) {
      const int e = idx[(size_t)t * a.K + k];
      valid = (e >= 0 && e < a.E);
      blob = a.experts + (size_t)(valid ? e : 0) * a.stride;
      if (combine) coef = a.ws.w[(size_t)t * a.K + k];
    } else if (combine) {
      coef = a.ws.g[t];
    }
    Stage<I, 64> st;
    st.load(a.ws.h + ((size_t)t * a.NE + k) * I, lane);
    float yv[P];
    if (valid) {
      const uint8_t* dc = blob + a.off_codes[2];
      const uint8_t* ds = blob + a.off_sb[2];
      uint4 cw[P][C::CPL];
      uint32_t sb[P][C::CPL];
#pragma unroll
      for (int p = 0; p < P; ++p)
        load_row<C, FORM == 3>(dc, ds, min(row0 + p * C::RPW + rig, a.H - 1), lir, cw[p], sb[p]);
      __builtin_amdgcn_sched_barrier(0);
      st.template store<C>(hs[wave], lane, 1.0f);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float xr[C::XPL], S[C::CPL];
      read_act<C>(hs[wave], lir, xr, S);
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
    __builtin_amdgcn_wave_barrier();  // the next slot reuses this wave's LDS region
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
  if (lane == 0) write_routing(a, t, sel, val, lg, idx, w, idx_b, sg);
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
  if (lane == 0) {
    write_routing(a, t, sel[wave], val[wave], nullptr, idx, w, idx_b, nullptr);
    if (sg && a.has_shared) sg[t] = (float)(1.0 / (1.0 + exp(-gl)));
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

// Row steps per wave (the bytes each wave has in flight), tuned on MI355X for the 4096/1024 shape.
#ifndef BQ_P2
#define BQ_P2 1
#endif
#ifndef BQ_P3
#define BQ_P3 8
#endif
#ifndef BQ_ROUTER_STEPS
#define BQ_ROUTER_STEPS 1
#endif
constexpr int kP2 = BQ_P2;  // gate/up
constexpr int kP3 = BQ_P3;  // down
// With several tokens per launch the grid holds a block set per token; from BQ_WIDE_MIN_TOKENS
// tokens, gate/up waves take BQ_P2_WIDE row pairs each (fewer, longer blocks). Measured on the
// 512-expert top-3 layer: 56.0 against 65.2 us at 8 tokens, 234 against 283 us at 40, while one
// row pair stays best for single tokens.
#ifndef BQ_P2_WIDE
#define BQ_P2_WIDE 4
#endif
#ifndef BQ_WIDE_MIN_TOKENS
#define BQ_WIDE_MIN_TOKENS 4
#endif
constexpr int kP2Wide = BQ_P2_WIDE;
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
                        dim3(kBlock), s, ev, a, x, T);
  }
  return launch_timed(k_router_phase<H>, dim3(nrb, T), dim3(kBlock), s, ev, a, x, norm_src, eps, router_steps);
}

template <int BITS, int H>
hipError_t gateup_impl(const LayerArgs& a, const float* x, int T, const int32_t* idx_in, int32_t* idx_out,
                       bool with_shared, hipStream_t s, const KernelEvents& ev) {
  using C = RowCfg<BITS, H>;
  const bool wide = T >= BQ_WIDE_MIN_TOKENS && (a.form == 0 || a.form == 3);
  const int rows_per_block = kWaves * (wide ? kP2Wide : kP2) * C::RPW;
  const int nb = (a.I + rows_per_block - 1) / rows_per_block;
  const int slots = a.K + ((with_shared && a.has_shared) ? 1 : 0);
  const dim3 grid(nb, slots, T);
#define BQ_GU(P, PL, F) launch_timed(k_gateup<BITS, H, P, PL, F>, grid, dim3(kBlock), s, ev, a, x, idx_in, idx_out)
  if (wide) {
    if constexpr (BITS == 4) {
      if (a.form == 3) return a.E <= 512 ? BQ_GU(kP2Wide, 8, 3) : BQ_GU(kP2Wide, 16, 3);
    }
    return a.E <= 512 ? BQ_GU(kP2Wide, 8, 0) : BQ_GU(kP2Wide, 16, 0);
  }
  if constexpr (BITS == 4) {
    if (a.form == 3) return a.E <= 512 ? BQ_GU(kP2, 8, 3) : BQ_GU(kP2, 16, 3);
  }
  if (a.E <= 512) return a.form == 1 ? BQ_GU(kP2, 8, 1) : a.form == 2 ? BQ_GU(kP2, 8, 2) : BQ_GU(kP2, 8, 0);
  return a.form == 1 ? BQ_GU(kP2, 16, 1) : a.form == 2 ? BQ_GU(kP2, 16, 2) : BQ_GU(kP2, 16, 0);
#undef BQ_GU
}

template <int BITS, int I>
hipError_t down_impl(const LayerArgs& a, int T, const int32_t* idx, const float* residual, float* out, float* y,
                     hipStream_t s, const KernelEvents& ev) {
  using C = RowCfg<BITS, I>;
  constexpr int RB = C::RPW * kP3;
  const int nb = (a.H + RB - 1) / RB;
#define BQ_DN(F) launch_timed(k_down<BITS, I, kP3, F>, dim3(nb, T), dim3(kBlock), s, ev, a, idx, residual, out, y)
  if constexpr (BITS == 4) {
    if (a.form == 3) return BQ_DN(3);
  }
  return a.form == 1 ? BQ_DN(1) : a.form == 2 ? BQ_DN(2) : BQ_DN(0);
#undef BQ_DN
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
                         const int32_t* idx_in, int32_t* idx_out, bool with_shared, hipStream_t s,
                         const KernelEvents& ev) {
  const LayerArgs a = make_args(g, p, ws);
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
  const LayerArgs a = make_args(g, p, ws);
#define BQ_CASE(IV)                                                                        \
  case IV:                                                                                 \
    return g.bits == 4 ? down_impl<4, IV>(a, T, idx, residual, out, y, s, ev)              \
                       : down_impl<2, IV>(a, T, idx, residual, out, y, s, ev);
  switch (g.I) { BQ_FOR_I(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefetch(const Prefetch& pf, int blocks, hipStream_t s) {
  if (pf.bytes[0] + pf.bytes[1] == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefetch, dim3(blocks), dim3(kBlock), 0, s, pf);
  return hipGetLastError();
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
