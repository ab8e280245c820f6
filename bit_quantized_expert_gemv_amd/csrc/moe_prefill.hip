// Prefill path of the quantised MoE layer for MI355X (gfx950): many tokens through one layer,
// grouped by expert so that each expert's weights are streamed once per tile of tokens.
//
//   1. prep: activations to fp16 (each 8-block stored in the order 0,2,4,6,1,3,5,7, the order in
//      which the code widening below produces weights) and per-64-group sums of the fp16 values;
//   2. router: logits = X . [R; gate]^T as an fp64 tiled GEMM, so the top-K decision is exact
//      up to fp64 rounding, then the top-K and weights per token (the decode top-K kernel); or,
//      from MOE_ROUTER_CERTIFIED_MIN_TOKENS tokens, approximate logits on bf16 MFMAs with an error
//      bound, and fp64 only for the rows the bound cannot rule out (the same choice);
//   3. grouping: per-expert counts, exclusive scan and a stable permutation by token index,
//      built from per-chunk histograms so that the result is deterministic;
//   4. gate/up: an MFMA grouped GEMM per expert tile with SwiGLU in the epilogue; the routed
//      experts and the shared expert (all tokens) are separate launches;
//   5. down: the same grouped GEMM on the SwiGLU outputs;
//   6. combine: out[t] = residual[t] + sum_k w[t][k] y[pos(t,k)] + g[t] y_shared[t] (gather).
// HN thread "Flash-MoE: Running a 397B Parameter Model on a Laptop": the router's choice decides
// which experts are read. p4 "300b on 32gb MoE-streaming findings": even short prompts touch most
// experts, which is why prefill streams the whole pool once.
//
// Exact weights. A dequantised weight is s*q + b ("Kernel de dequantización optimizado con FMA").
// It needs up to 15 significant bits, so rounding the weights to a 16-bit type would lose
// accuracy. Instead the MFMA's weight operand is the raw code q itself, exact in fp16: a 4-bit code
// in a byte is the e4m3 value q * 2^-9, and a 2-bit code in a nibble is the e2m1 value q / 2.
// v_cvt_scalef32_pk_f16_fp8 / _fp4 widen them two at a time, with the scale folded in, to exactly q.
// Per 64-wide group the fp32 MFMA result D = sum q x is finished in the epilogue as
//   s * D + b * S,   S = sum x over the group (of the fp16 activations the MFMA sees).
// The activations are rounded to fp16 once (relative 2^-11), which keeps the layer output well
// inside its error bound. Before the cast they are scaled by a power of two, so that fp16's range
// (largest 65504, normal down to 2^-14) never clips them: x per token, the SwiGLU outputs per token
// and 64-row group. The scale is exact and is undone in the fp32 epilogues.
//
// MFMA: v_mfma_f32_16x16x32_f16 with A = activations (16 tokens x 32 k) and B = codes (32 k x 16
// weight rows); lane l holds k slice l/16 of token or row l%16 (layout checked on the device). Every
// MFMA stays inside one scale group: lane swaps regroup each lane's 16-byte code load so that the
// 32 k of one MFMA share a scale, and the activation operand is read in the same k order (details
// at k_grouped).
#include <hip/hip_runtime.h>
#include <type_traits>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "moe_internal.h"

namespace bqmoe {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// silu(a) * c = a / (1 + e^-a) * c, with e^-a as the hardware 2^x of -a log2(e) and the hardware
// reciprocal (about 1 ulp each, far inside the layer's tolerance). Limits: a -> -inf gives 2^x = inf,
// a reciprocal of 0 and a product of -0; a -> +inf gives a.
__device__ __forceinline__ float silu_mul_fast(float a, float c) {
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.44269504088896341f)) * c;
}

// Stored position of element e (0..7) of an 8-block: the order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ int perm8(int e) { return (e >> 1) + 4 * (e & 1); }

// ---- 1. activation prep -------------------------------------------------------------------------
// Exponent e of the power of two that brings a largest magnitude m into [2^14, 2^15), inside fp16's
// range with room to spare (0 for a zero, infinite or NaN m; clamped so that 2^e and 2^-e are
// normal floats).
__device__ __forceinline__ int fp16_exponent(float m) {
  if (!(m > 0.0f) || !(m < INFINITY)) return 0;
  int k;
  (void)frexpf(m, &k);  // m in [2^(k-1), 2^k)
  return min(max(15 - k, -100), 100);
}

// One block per token: the token's values times 2^e (e from its largest magnitude), as fp16 with
// each 8-block stored in the order 0,2,4,6,1,3,5,7, the per-64-group sums of those fp16 values,
// and xu[t] = 2^-e. Thread i takes 8-blocks i, i + 256, ...; the 8 threads of a group add their
// sums with 3 butterfly steps, in a fixed order.
constexpr int kPrepPer = 4;  // 8-blocks per thread: hidden <= 8192
__global__ __launch_bounds__(kThreads) void k_prep(int H, const float* __restrict__ x, _Float16* __restrict__ xq,
                                                   float* __restrict__ xs, float* __restrict__ xu) {
  __shared__ float red[kThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, nb = H / 8;
  const float4* src = reinterpret_cast<const float4*>(x + (size_t)t * H);
  float4 v[kPrepPer][2];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kPrepPer; ++j) {
    const int i = tid + j * kThreads;
    const int ib = i < nb ? i : 0;
    v[j][0] = src[2 * ib];
    v[j][1] = src[2 * ib + 1];
    if (i < nb) {
      const float4 a = v[j][0], b = v[j][1];
      m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                         fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w)))));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = fp16_exponent(m);
  const float up = ldexpf(1.0f, e);
  if (tid == 0) xu[t] = ldexpf(1.0f, -e);
#pragma unroll
  for (int j = 0; j < kPrepPer; ++j) {
    const int i = tid + j * kThreads;
    const bool live = i < nb;  // nb and 256 are multiples of 8, so a group's 8 threads agree
    const float4 a = v[j][0], b = v[j][1];
    const _Float16 h[8] = {(_Float16)(a.x * up), (_Float16)(a.y * up), (_Float16)(a.z * up), (_Float16)(a.w * up),
                           (_Float16)(b.x * up), (_Float16)(b.y * up), (_Float16)(b.z * up), (_Float16)(b.w * up)};
    if (live) {
      f16x8_t o;
#pragma unroll
      for (int q = 0; q < 8; ++q) o[perm8(q)] = h[q];
      reinterpret_cast<f16x8_t*>(xq + (size_t)t * H)[i] = o;
    }
    float sum = (((float)h[0] + (float)h[1]) + ((float)h[2] + (float)h[3])) +
                (((float)h[4] + (float)h[5]) + ((float)h[6] + (float)h[7]));
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) sum += __shfl_xor(sum, msk, 8);
    if (live && (i & 7) == 0) xs[(size_t)t * (H / 64) + (i >> 3)] = sum;
  }
}

// ---- 2. router GEMM (fp64 MFMA) ---------------------------------------------------------------------
// logits[t][e] = sum_j R[e][j] x[t][j] for e < E, and the shared-gate vector as row E, on
// v_mfma_f64_16x16x4_f64: every bf16 x fp32 product is exact in fp64 and the sums are fp64, so the
// top-K decision is exact up to fp64 rounding. Lane layout (checked on the device): A[i][k] in lane
// i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane j + 16*(i%4), element i/4.
// Each wave owns 32 tokens x 32 rows as 2 x 2 tiles over a quarter of K; the four waves of a block split
// K and add their parts in a fixed order (((q0 + q1) + q2) + q3). There is no LDS staging: within each
// 32-wide K slice, MFMA step s of lane (i, kk) takes k = 8*kk + s instead of 4*s + kk (both operands
// use the same order, so every product is still paired), so a lane's operands are 8 contiguous
// elements of its token or row: two 16-byte loads of x, one of the router row. Three register stages
// keep two slices in flight during the MFMAs; the bf16 and fp32 values widen to fp64 exactly, one
// step at a time.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kRW = 32;      // tokens and rows per wave
#ifndef BQ_ROUTER_SPLITK
#define BQ_ROUTER_SPLITK 4
#endif
constexpr int kRSplit = BQ_ROUTER_SPLITK;  // waves per block, each with 1/kRSplit of K
constexpr int kRSlice = 32;  // K per slice
#ifndef BQ_APPROX_QUAD
#define BQ_APPROX_QUAD 1
#endif
#ifndef BQ_ROUTER_GEMM_MIN
#define BQ_ROUTER_GEMM_MIN MOE_ROUTER_BATCH_MIN_TOKENS
#endif
constexpr int kRouterGemmMinTokens = BQ_ROUTER_GEMM_MIN;
#ifndef BQ_ROUTER_CERTIFIED_MIN
#define BQ_ROUTER_CERTIFIED_MIN MOE_ROUTER_CERTIFIED_MIN_TOKENS
#endif
constexpr int kRouterCertifiedMinTokens = BQ_ROUTER_CERTIFIED_MIN;

struct RouterRaw {
  float4 x[2][2];  // [token tile][half]: 8 consecutive x of the lane's token
  uint4 r[2];      // [row tile]: 8 consecutive bf16 of the lane's row
};

__global__ __launch_bounds__(64 * kRSplit) void k_router_gemm(int T, int H, int E, int has_shared,
                                                              const float* __restrict__ x,
                                                              const uint16_t* __restrict__ router,
                                                              const uint16_t* __restrict__ sgate,
                                                              double* __restrict__ logits) {
  __shared__ f64x4_t part[kRSplit - 1][2][2][64];  // the partial tiles of waves 1..kRSplit-1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kk = lane >> 4;
  const int t0 = blockIdx.y * kRW, e0 = blockIdx.x * kRW;
  const int nrows = E + has_shared;
  const int kh = H / kRSplit;
  const int kbeg = wave * kh + 8 * kk;
  // operand rows of this lane (clamped ones are computed and never stored)
  const float* xp[2];
  const uint16_t* rp[2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) xp[ti] = x + (size_t)min(t0 + 16 * ti + c, T - 1) * H + kbeg;
#pragma unroll
  for (int rj = 0; rj < 2; ++rj) {
    const int e = min(e0 + 16 * rj + c, nrows - 1);
    rp[rj] = (e < E ? router + (size_t)e * H : sgate) + kbeg;
  }
  const int nsl = kh / kRSlice;
  auto load = [&](RouterRaw& R, int sl) __attribute__((always_inline)) {
    const int off = sl * kRSlice;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int h = 0; h < 2; ++h) R.x[ti][h] = *reinterpret_cast<const float4*>(xp[ti] + off + 4 * h);
#pragma unroll
    for (int rj = 0; rj < 2; ++rj) R.r[rj] = *reinterpret_cast<const uint4*>(rp[rj] + off);
  };
  f64x4_t acc[2][2];
#pragma unroll
  for (int ti = 0; ti < 2; ++ti)
#pragma unroll
    for (int rj = 0; rj < 2; ++rj) acc[ti][rj] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  auto compute = [&](const RouterRaw& R) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      double a[2], b[2];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const float4 v = R.x[ti][st >> 2];
        const int e = st & 3;
        a[ti] = (double)(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
      }
#pragma unroll
      for (int rj = 0; rj < 2; ++rj) {
        const uint4 w = R.r[rj];
        const uint32_t d = (st >> 1) == 0 ? w.x : (st >> 1) == 1 ? w.y : (st >> 1) == 2 ? w.z : w.w;
        b[rj] = (double)__uint_as_float((st & 1) ? (d & 0xFFFF0000u) : (d << 16));
      }
#pragma unroll
      for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int rj = 0; rj < 2; ++rj) acc[ti][rj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ti], b[rj], acc[ti][rj], 0, 0, 0);
    }
  };
  RouterRaw r0, r1, r2;
  load(r0, 0);
  load(r1, min(1, nsl - 1));
#pragma unroll 1
  for (int sl = 0; sl < nsl; sl += 3) {
    // every load is issued on every path (clamped past the end), so the wait counts stay exact
    load(r2, min(sl + 2, nsl - 1));
    compute(r0);
    load(r0, min(sl + 3, nsl - 1));
    if (sl + 1 < nsl) compute(r1);
    load(r1, min(sl + 4, nsl - 1));
    if (sl + 2 < nsl) compute(r2);
  }
  if (wave > 0) {
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int rj = 0; rj < 2; ++rj) part[wave - 1][ti][rj][lane] = acc[ti][rj];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < kRSplit - 1; ++w)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
      for (int rj = 0; rj < 2; ++rj) acc[ti][rj] += part[w][ti][rj][lane];
  // element q of tile (ti, rj) in lane (c, kk): token t0 + 16ti + kk + 4q, row e0 + 16rj + c
#pragma unroll
  for (int rj = 0; rj < 2; ++rj) {
    const int e = e0 + 16 * rj + c;
    if (e >= nrows) continue;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 16 * ti + kk + 4 * q;
        if (t < T) logits[(size_t)t * (E + 1) + e] = acc[ti][rj][q];
      }
    }
  }
}

// ---- 2b. certified router: approximate logits on bf16 MFMAs -------------------------------------
// For a top-K alone the fp64 GEMM above does far more exact work than the decision needs. Here the
// logits are first approximated on bf16 MFMAs, then a per-token kernel recomputes in fp64 only the
// rows that the approximation's error bound cannot rule out. Each x is split into two bf16 values,
// x = hi + lo + d with |d| <= 2^-16 |x| (round to nearest even twice), so the MFMAs see products
// that are exact in fp32; the only other error is the fp32 accumulation inside the MFMA chain.
// D = A B with A = router rows (16 x 32 bf16) and B = activations (32 x 16). A[i][k] sits in lane
// i + 16*(k/8), element k%8; B[k][j] in lane j + 16*(k/8), element k%8; D[i][j] in lane
// j + 16*(i/4), element i%4. A block computes 16 RT rows x 32 tokens; its kASplit waves take equal
// slices of K, and their partial tiles are added in fp64 in wave order.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Row tiles of 16 per wave (RT = 2, 4 or 8). The approximation is latency-bound per block, so the
// launch takes the smallest tile whose grid still fits one block per CU: a grid past 256 blocks
// puts two blocks on some CUs, and those finish last.
#ifndef BQ_ROUTER_APPROX_RT
#define BQ_ROUTER_APPROX_RT 0  // 0: chosen per launch
#endif
constexpr int kAT = 32;     // tokens per block (2 token tiles)
#ifndef BQ_ROUTER_APPROX_SPLITK
#define BQ_ROUTER_APPROX_SPLITK 4
#endif
constexpr int kASplit = BQ_ROUTER_APPROX_SPLITK;  // waves per block, each with 1/kASplit of K

template <int RT>
struct ApproxRaw {
  uint4 r[RT];     // [row tile]: 8 consecutive bf16 of the lane's row
  float4 x[2][2];  // [token tile][half]: 8 consecutive x of the lane's token
};

__device__ __forceinline__ void split_bf16(const float4& a, const float4& b, bf16x8_t& hi, bf16x8_t& lo) {
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)v[i];  // round to nearest even
    hi[i] = h;
    lo[i] = (__bf16)(v[i] - (float)h);  // the difference is exact in fp32
  }
}

template <int RT>
__global__ __launch_bounds__(64 * kASplit) void k_router_approx(int T, int H, int E, const float* __restrict__ x,
                                                                const uint16_t* __restrict__ router,
                                                                double* __restrict__ logits) {
  constexpr int kAR = 16 * RT;  // router rows per block
  __shared__ f32x4_t part[kASplit - 1][RT][2][64];  // the partial tiles of waves 1..kASplit-1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, kk = lane >> 4;
  // XCD-aware order: blocks are dealt to the 8 XCDs in turn, so when the count allows, the blocks
  // of one XCD take consecutive tiles (a few token tiles, every row tile) and share them in its L2.
  const int nbx = gridDim.x, total = gridDim.x * gridDim.y;
  int id = blockIdx.x + nbx * blockIdx.y;
  if (total % 8 == 0) id = (id & 7) * (total / 8) + (id >> 3);
  const int e0 = (id % nbx) * kAR, t0 = (id / nbx) * kAT;
  // Loads: each group of 4 lanes reads 64 (router) or 128 (x) contiguous bytes of one row, lane
  // 4r + j taking chunk j of row r; the compute moves chunk kk of row c to lane c + 16 kk, the MFMA
  // operand layout, with ds_bpermute. Loading in the operand layout directly (16 rows per 4-lane
  // group of 16-byte reads) halves what L2 delivers per cycle.
  const int lr = BQ_APPROX_QUAD ? (lane >> 2) : c, lk = BQ_APPROX_QUAD ? (lane & 3) : kk;
  const int kh = H / kASplit;
  const int kbeg = wave * kh + 8 * lk;
  const uint16_t* rp[RT];
  const float* xp[2];
#pragma unroll
  for (int i = 0; i < RT; ++i) rp[i] = router + (size_t)min(e0 + 16 * i + lr, E - 1) * H + kbeg;
#pragma unroll
  for (int j = 0; j < 2; ++j) xp[j] = x + (size_t)min(t0 + 16 * j + lr, T - 1) * H + kbeg;
  const int src = (4 * c + kk) << 2;  // the lane that loaded this lane's operand chunk
  auto move4 = [&](uint4 v) __attribute__((always_inline)) {
    if constexpr (BQ_APPROX_QUAD) {
      v.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.x);
      v.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.y);
      v.z = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.z);
      v.w = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.w);
    }
    return v;
  };
  const int nst = kh / 32;
  auto load = [&](ApproxRaw<RT>& R, int st) __attribute__((always_inline)) {
    const int off = st * 32;
#pragma unroll
    for (int i = 0; i < RT; ++i) R.r[i] = *reinterpret_cast<const uint4*>(rp[i] + off);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) R.x[j][h] = *reinterpret_cast<const float4*>(xp[j] + off + 4 * h);
  };
  f32x4_t acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const ApproxRaw<RT>& R) __attribute__((always_inline)) {
    bf16x8_t hi[2], lo[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      split_bf16(__builtin_bit_cast(float4, move4(__builtin_bit_cast(uint4, R.x[j][0]))),
                 __builtin_bit_cast(float4, move4(__builtin_bit_cast(uint4, R.x[j][1]))), hi[j], lo[j]);
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, move4(R.r[i]));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, hi[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, lo[j], acc[i][j], 0, 0, 0);
      }
    }
  };
  ApproxRaw<RT> r0, r1, r2;
  load(r0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(r1, min(1, nst - 1));
  __builtin_amdgcn_sched_barrier(0);
  // The scheduling barriers keep each stage's loads where they are written: left to itself, the
  // scheduler sinks them into the MFMA stream of the previous stage, and each stage then waits for
  // loads issued just before it.
#pragma unroll 1
  for (int st = 0; st < nst; st += 3) {
    // every load is issued on every path (clamped past the end), so the wait counts stay exact
    load(r2, min(st + 2, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(r0);
    __builtin_amdgcn_sched_barrier(0);
    load(r0, min(st + 3, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < nst) compute(r1);
    __builtin_amdgcn_sched_barrier(0);
    load(r1, min(st + 4, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    if (st + 2 < nst) compute(r2);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) part[wave - 1][i][j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave > 0) return;
  // element q of tile (i, j) in lane (c, kk): row e0 + 16i + 4kk + q, token t0 + 16j + c
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = t0 + 16 * j + c;
    if (t >= T) continue;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      double v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (double)acc[i][j][q];
#pragma unroll
      for (int w = 0; w < kASplit - 1; ++w) {
        const f32x4_t p = part[w][i][j][lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += (double)p[q];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 16 * i + 4 * kk + q;
        if (e < E) logits[(size_t)t * (E + 1) + e] = v[q];
      }
    }
  }
}

// ---- 3. grouping by expert --------------------------------------------------------------------------
// Entries i = t*K + k (token t, slot k) carry expert idx[i]. Chunks of 256 entries. A caller's index
// outside [0, E) is grouped with expert 0, so that every position stays inside the buffers; the
// output kernel writes NaN for such an entry instead of the expert 0 result computed for it.
constexpr int kChunk = 256;
__device__ __forceinline__ int valid_expert(int e, int E) { return (e >= 0 && e < E) ? e : 0; }

__global__ __launch_bounds__(kChunk) void k_group_hist(int N, int E, const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  if (i < N) atomicAdd(&cnt[valid_expert(idx[i], E)], 1);  // counts do not depend on the order of the adds
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) hist[(size_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive prefix sum of v over the block (1024 threads, wave64), in a fixed order; *total gets the
// sum. wsum: 16 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* __restrict__ wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(inc, d, 64);
    if (lane >= d) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {  // 16 waves in a 1024-thread block
    const int t = wsum[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// One block of 1024 threads, thread e for expert e: per-expert prefix over chunks (in place),
// counts, offsets and the tile list (tiles of BM entries per expert; those above BM/2 first). The chunk
// column is read eight loads at a time, and the expert scans are block-wide.
__global__ __launch_bounds__(1024) void k_group_scan(int nchunks, int E, int BM, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_first,
                                                     int32_t* __restrict__ ntiles) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;  // E <= MOE_MAX_EXPERTS == 1024 == blockDim.x
  int run = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (c0 + i < nchunks) ? hist[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (c0 + i < nchunks) hist[(size_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
    counts[e] = run;
  }
  // Tiles with more than BM/2 tokens run both token halves and take longer, so they go first (a
  // stable partition, each class in expert order): the launch then ends on the light tiles.
  const int full = (e < E) ? run / BM : 0, rem = (e < E) ? run % BM : 0;
  const int heavy = full + (rem > BM / 2 ? 1 : 0), light = (rem > 0 && rem <= BM / 2) ? 1 : 0;
  int total_entries, total_heavy, total_light;
  const int off = block_exclusive_scan(e < E ? run : 0, wsum, &total_entries);
  const int h0 = block_exclusive_scan(heavy, wsum, &total_heavy);
  const int l0 = block_exclusive_scan(light, wsum, &total_light);
  if (e < E) {
    offsets[e] = off;
    for (int j = 0; j < heavy; ++j) {  // the full tiles, then a partial one above BM/2
      tile_e[h0 + j] = e;
      tile_first[h0 + j] = off + j * BM;
    }
    if (light) {
      tile_e[total_heavy + l0] = e;
      tile_first[total_heavy + l0] = off + full * BM;
    }
  }
  if (e == 0) {
    offsets[E] = total_entries;
    *ntiles = total_heavy + total_light;
  }
}

// Position of every entry: offsets[e] + (entries of e in earlier chunks) + (earlier entries of e in
// this chunk). Stable by token index; perm is its inverse.
__global__ __launch_bounds__(kChunk) void k_group_place(int N, int E, const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ hist,
                                                        const int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ pos, int32_t* __restrict__ perm) {
  __shared__ int32_t ex[kChunk];
  const int i = blockIdx.x * kChunk + threadIdx.x;
  const int e = (i < N) ? valid_expert(idx[i], E) : -1;
  ex[threadIdx.x] = e;
  __syncthreads();
  if (i >= N) return;
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += (ex[j] == e);
  const int p = offsets[e] + hist[(size_t)blockIdx.x * E + e] + rank;
  pos[i] = p;
  perm[p] = i;
}

// ---- 4/5. grouped GEMM on MFMA ---------------------------------------------------------------------
struct GroupArgs {
  const uint8_t* experts;
  uint64_t stride;
  const uint8_t* shared;
  uint64_t off_codes[2], off_sb[2];  // (gate, up) or (down, unused)
  const _Float16* a;                 // activations [rows][KDIM], fp16, 8-blocks permuted
  const float* as;                   // their group sums [rows][KDIM/64]
  const float* ascale;               // powers of two undoing their scaling: gate/up [T], down [rows][KDIM/64]
  const int32_t* perm;               // routed: position -> entry (t*K + k)
  int K;
  const int32_t* tile_e;
  const int32_t* tile_first;
  const int32_t* ntiles;
  const int32_t* offsets;
  int shared_base;  // output row of the shared expert's token 0 (= T*K)
  int T;
  _Float16* oh;  // gate/up: SwiGLU outputs [rows][nout] (fp16, 8-blocks permuted), group sums os [rows][nout/64]
  float* os;
  float* oscale;  // gate/up: [rows][nout/64] powers of two undoing the scaling of oh
  float* oy;  // down: [rows][nout]
  int nout;
  // MXFP4 layers: activations as kMxTerms planes of E4M3 bytes [rows][KDIM] (a_plane bytes apart)
  // with E8M0 scales [rows][KDIM/32] (sc_plane bytes apart); gate/up writes fp32 SwiGLU outputs
  const uint8_t* a8;
  const uint8_t* asc;
  uint64_t a_plane, sc_plane;
  float* oh32;
};

constexpr int kTileM = 32;  // token rows per tile
// Word 3 of a raw buffer descriptor on gfx9 (32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;

// One MFMA's B operand: 8 codes (one dword at 4-bit, one 16-bit half at 2-bit) widened to fp16 q,
// in the element order 0,2,4,6,1,3,5,7.
template <int BITS>
__device__ __forceinline__ f16x8_t codes_f16(uint32_t w, int half) {
  f16x2_t p0, p1, p2, p3;
  if constexpr (BITS == 4) {
    const uint32_t u = w & 0x0F0F0F0Fu;         // bytes: codes 0, 2, 4, 6
    const uint32_t v = (w >> 4) & 0x0F0F0F0Fu;  // bytes: codes 1, 3, 5, 7
    p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 512.0f, false);
    p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 512.0f, true);
    p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 512.0f, false);
    p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 512.0f, true);
  } else {
    const uint32_t u = w & 0x33333333u;         // nibble n: code 2n
    const uint32_t v = (w >> 2) & 0x33333333u;  // nibble n: code 2n + 1
    if (half == 0) {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 2.0f, 0);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 2.0f, 1);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 0);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 1);
    } else {
      p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 2.0f, 2);
      p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(u, 2.0f, 3);
      p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 2);
      p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 3);
    }
  }
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Per-lane registers of one pipeline step: NI 16-byte code loads per row block (see k_grouped), the
// (scale, bias) words of a step pair, and the tile's activations.
template <int NI>
struct GCodes {
  u32x4_t v[2][NI];  // [row block][load]
};
struct GWords {
  uint32_t w[4];
};
struct GWordsX {
  uint32_t w[2][2][4];  // [step of the pair][row block][group of the step]
};
template <int U>
struct GAct {
  u32x4_t v[U];
};

#ifndef BQ_LB_GU
#define BQ_LB_GU 2
#endif
#ifndef BQ_LB_DOWN
#define BQ_LB_DOWN 2
#endif
#ifndef BQ_GROUP_SCHED_BARRIER
#define BQ_GROUP_SCHED_BARRIER 1
#endif
#ifndef BQ_U_LINE
#define BQ_U_LINE 1
#endif
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 8-element block of group G that K slice q of MFMA half h reads (the codes' order after the lane
// swaps of k_grouped; the activations are read in the same order)
template <int BITS>
__device__ __forceinline__ int kblock(int q, int h) {
  return BITS == 4 ? 4 * (q & 1) + 2 * (q >> 1) + h : 2 * q + h;
}

// Block: 4 waves, one tile of up to 32 tokens, all rows of the weight matrices. Each wave owns 32
// rows (two 16-row blocks) of one matrix in every slab: for down, waves 0..3 take rows 32w..32w+31
// of a 128-row slab; for gate/up, waves 0, 1 take 32 rows of gate and waves 2, 3 the same rows of
// up, in a 64-row slab, and the SwiGLU pairs meet through LDS at the end of the slab. The block
// walks the slabs one after the other, and the pipeline runs over the flattened (slab, step)
// sequence, so it fills once per block rather than once per slab.
//
// Arithmetic on v_mfma_f32_16x16x32_f16 (A = 16 tokens x 32 k, B = 32 k x 16 rows; lane l holds
// k slice l/16 of token / row l%16): the tile is one or two halves of 16 tokens, so a tile of at
// most 16 tokens (most routed tiles) costs half the matrix work and half the epilogue. The codes
// of one MFMA must lie in one group (one scale): a lane loads 16 contiguous bytes of its row, and
// lane swaps regroup them (4-bit: two groups per load, the lower 32 lanes and the upper 32 lanes
// exchange half their dwords; 2-bit: four groups per load, a 4 x 4 transpose over the four 16-lane
// rows). The bias term sum_g bias[r][g] * S[t][g] runs as an fp32 16x16x4 MFMA per row block and
// step (A = group sums S, B = biases), so the vector ALUs only apply the scales.
//
// Pipeline, per step s of U groups: the tile's activations for step s+2 are loaded into one of
// two register sets (16 bytes per thread and group), then the wave's codes for step s+2, and on
// even steps the (scale, bias) words of steps s+2 and s+3; step s is computed from registers
// (weights) and an LDS ring (activations); the activations of step s+1, loaded a step earlier,
// are parked in the ring and one barrier closes the step. Every load has two steps to land
// before it is waited for.
#ifndef BQ_CODE_STAGES
#define BQ_CODE_STAGES 4
#endif
// Code register stages of the k_grouped pipeline: 4 keep three steps of weight loads in flight per
// wave (12 KB), at 250 VGPRs for the 4-bit gate/up, still two waves per SIMD; against 3 stages the
// prefill4 grouped GEMMs measured 1099 -> 1040 us per step.
constexpr int kStagesMax = BQ_CODE_STAGES;
template <int BITS, int KDIM, int UMAX, bool GATEUP, bool SHARED>
__global__ __launch_bounds__(kThreads, GATEUP ? BQ_LB_GU : BQ_LB_DOWN) void k_grouped(GroupArgs g, int sgroups) {
  // short gate/up rows (hidden 256, 512) keep three stages: their fourth spilled registers
  constexpr int kStages = GATEUP && KDIM <= 512 ? 3 : kStagesMax;
  constexpr int NG = KDIM / 64;
  constexpr int U = NG >= UMAX ? UMAX : NG;  // groups per pipeline step
  static_assert(U <= 4, "a step holds at most four groups");
  constexpr int NSTEP = NG / U;               // steps per slab
  constexpr int ROWB = KDIM * BITS / 8;
  constexpr int GB = 64 * BITS / 8;           // code bytes per row and group
  constexpr int NI = (U * GB + 63) / 64;      // 16-byte code loads per lane, row block and step
  constexpr int ROWS_B = GATEUP ? 64 : 128;   // rows per matrix per slab
  constexpr int AS = U * 8;                   // 16-byte activation slots per row and step
  constexpr int ASW = AS >= 16 ? 15 : AS - 1; // slot swizzle: 16 consecutive rows hit distinct banks
  // Down projections (K <= 1024) keep the tile's whole activation rows in LDS (64 KiB at K = 1024),
  // loaded once per block: the steps then issue only weight loads and need no barrier.
  constexpr bool RESIDENT = !GATEUP && KDIM <= 1024;
  constexpr int RS = KDIM / 8;                // 16-byte slots per resident row
  constexpr int RSW = RS >= 16 ? 15 : RS - 1; // its slot swizzle stays inside the row (RS is 8 at K = 64)
  using Codes = GCodes<NI>;
  using Act = GAct<U>;
  __shared__ float s_lds[NG * kTileM];             // group sums of the tile's activations, [group][row]
  __shared__ u32x4_t a_lds[RESIDENT ? kTileM * RS : 2 * kTileM * AS];  // resident rows, or a ring
                                                   // [step parity][row][slot ^ swizzle]
  __shared__ float x_lds[GATEUP ? 2 : 1][GATEUP ? 16 : 1][64];  // gate/up: gate results for the up waves
  __shared__ float h_lds[GATEUP ? 2 : 1][kTileM];  // gate/up: per-wave sums of the fp16 SwiGLU outputs
  __shared__ float hm_lds[GATEUP ? 2 : 1][kTileM]; // gate/up: per-wave largest |SwiGLU output|
  // powers of two undoing the activations' scaling: gate/up per token row, down per [group][row]
  __shared__ float u_lds[GATEUP ? kTileM : NG * kTileM];

  // the wave index through readfirstlane: the compiler then knows it is uniform, so the buffer
  // descriptors built from it (a matrix per wave in gate/up) stay in scalar registers; derived from
  // threadIdx alone it counts as divergent, and every buffer load became a waterfall loop
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c16 = lane & 15, q = lane >> 4;        // MFMA lane: token / row within 16, k slice
  const int mi = GATEUP ? (wave >> 1) : 0;         // matrix of this wave (gate 0, up 1)
  const int wrow = (GATEUP ? (wave & 1) : wave) * 32;  // first row of this wave in a slab
  // Block b works on tile tau, slab group gy. Blocks go to the 8 XCDs round-robin, so a run of
  // 8 * sgroups consecutive blocks holds 8 tiles, one per XCD, each with all its slab groups on that
  // XCD: they start together and stream the same activation rows, which then come from its L2.
  const int b8 = 8 * sgroups;
  const int tau = (int)(blockIdx.x / b8) * 8 + (int)(blockIdx.x & 7);
  const int gy = (int)(blockIdx.x % b8) >> 3;
  int first, count;
  const uint8_t* blob;
  if constexpr (SHARED) {
    first = tau * kTileM;
    if (first >= g.T) return;  // uniform per block
    count = min(kTileM, g.T - first);
    blob = g.shared;
  } else {
    if (tau >= *g.ntiles) return;  // uniform per block
    const int e = g.tile_e[tau];
    first = g.tile_first[tau];
    count = min(kTileM, g.offsets[e + 1] - first);
    blob = g.experts + (size_t)e * g.stride;
  }
  const int nh = count > 16 ? 2 : 1;  // token halves (uniform per block)
  // activation row of token slot m (clamped into the tile) and output row
  auto arow = [&](int m) -> int {
    const int mm = first + min(m, count - 1);
    if constexpr (SHARED) return GATEUP ? mm : g.shared_base + mm;
    else return GATEUP ? g.perm[mm] / g.K : mm;
  };
  auto orow = [&](int m) -> int { return SHARED ? g.shared_base + first + m : first + m; };

  for (int i = tid; i < NG * kTileM; i += kThreads) {
    const int m = i % kTileM, gi = i / kTileM;
    s_lds[i] = g.as[(size_t)arow(m) * NG + gi];
    if constexpr (!GATEUP) u_lds[i] = g.ascale[(size_t)arow(m) * NG + gi];
  }
  if constexpr (GATEUP) {
    if (tid < kTileM) u_lds[tid] = g.ascale[arow(tid)];
  }
  // this thread's 16-byte activation slot: row tid/8, slot tid%8 of every group
  const int a_row = tid >> 3, a_slot = tid & 7;
  const u32x4_t* a_src = reinterpret_cast<const u32x4_t*>(g.a + (size_t)arow(a_row) * KDIM) + a_slot;
  auto load_act = [&](Act& r, int s) {  // s: flattened step; the activations depend on its step in the slab only
    const int k = s % NSTEP;
#pragma unroll
    for (int u = 0; u < U; ++u) r.v[u] = a_src[(k * U + u) * 8];
  };
  auto park_act = [&](const Act& r, int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) a_lds[(s & 1) * kTileM * AS + a_row * AS + ((u * 8 + a_slot) ^ (a_row & ASW))] = r.v[u];
  };
  if constexpr (RESIDENT) {
    // whole rows, 16-byte slot j of row m at slot j ^ (m & RSW): 16 consecutive rows of a fragment read
    // hit distinct banks (a row of 256 bytes or more starts at bank 0)
    constexpr int PER = kTileM * RS / kThreads;
    u32x4_t v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * kThreads, m = idx / RS, j = idx % RS;
      v[i] = reinterpret_cast<const u32x4_t*>(g.a + (size_t)arow(m) * KDIM)[j];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * kThreads, m = idx / RS, j = idx % RS;
      a_lds[m * RS + (j ^ (m & RSW))] = v[i];
    }
  }

  // this block's slabs: range gy of sgroups equal ranges
  const int nslab = (g.nout + ROWS_B - 1) / ROWS_B;
  const int spb = (nslab + sgroups - 1) / sgroups;
  const int slab0 = gy * spb;
  const int ntot = (min(nslab, slab0 + spb) - slab0) * NSTEP;  // flattened steps
  if (ntot <= 0) return;  // uniform per block
  // Weights through buffer loads: a descriptor per section (scalar registers), a 32-bit lane
  // offset, and the step's offset as a scalar. Rows past nout are clamped; so are steps past the
  // end (they re-read the last step, from cache): every load is issued on every path, because a
  // load skipped on some path would make the compiler's wait counts conservative and drain the
  // loads in flight. A load that runs past a row (U below 4) reads bytes that are never used, or
  // zeros past the end of the section.
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_codes[mi]), (short)0, g.nout * ROWB, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_sb[mi]), (short)0, g.nout * NG * 4, kRsrcWord3);
  // codes: lane (c16, q) reads 16 bytes at byte 16q of each 64-byte span of its row's step
  auto load_codes = [&](Codes& st, int s) {
    const int slab = slab0 + s / NSTEP, k = s % NSTEP;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = min(slab * ROWS_B + wrow + 16 * rb + c16, g.nout - 1);
      const int voff = row * ROWB + 16 * q;
#pragma unroll
      for (int c = 0; c < NI; ++c) st.v[rb][c] = __builtin_amdgcn_raw_buffer_load_b128(crs, voff, k * U * GB + 64 * c, 0);
    }
  };
  // (scale, bias) words of steps 2p and 2p+1: the 16-lane row q loads those of row block q & 1 and
  // step 2p + q/2 (4 groups), so one instruction serves two steps; split_words then gives every
  // lane both row blocks' words of both steps.
  auto load_words = [&](GWords& r, int p) {
    const int t = min(2 * p + (q >> 1), ntot - 1);
    const int slab = slab0 + t / NSTEP, k = t % NSTEP;
    const int row = min(slab * ROWS_B + wrow + 16 * (q & 1) + c16, g.nout - 1);
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(srs, row * (NG * 4) + k * U * 4, 0, 0);
    r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
  };
  auto split_words = [&](const GWords& r, GWordsX& x) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // 16-lane rows [0,0,2,2] (row block 0) and [1,1,3,3] (row block 1), then halves
      const auto a = __builtin_amdgcn_permlane16_swap(r.w[u], r.w[u], false, false);
      const auto b0 = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
      const auto b1 = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
      x.w[0][0][u] = b0[0]; x.w[1][0][u] = b0[1];
      x.w[0][1][u] = b1[0]; x.w[1][1][u] = b1[1];
    }
  };

  f32x4_t acc[2][2], accb[2][2];  // [token half][row block]: scaled code sums; bias terms
#pragma unroll
  for (int th = 0; th < 2; ++th)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[th][rb][e] = accb[th][rb][e] = 0.0f;

  auto a_frag = [&](int s, int th, int G, int h) __attribute__((always_inline)) {
    const int row = 16 * th + c16;
    if constexpr (RESIDENT) {
      const int j = ((s % NSTEP) * U + G) * 8 + kblock<BITS>(q, h);
      return __builtin_bit_cast(f16x8_t, a_lds[row * RS + (j ^ (row & RSW))]);
    } else {
      return __builtin_bit_cast(f16x8_t, a_lds[(s & 1) * kTileM * AS + row * AS + ((G * 8 + kblock<BITS>(q, h)) ^ (row & ASW))]);
    }
  };
  // One step: regroup the codes, then per group the MFMAs of every token half and row block and the
  // scale epilogue; the bias MFMAs first.
  auto compute = [&](Codes& st, const uint32_t (&sw)[2][4], int s) __attribute__((always_inline)) {
    const int k = s % NSTEP;
    // bias terms: A = S[token][group k*U + q], B = bias[row][group k*U + q] (K = the step's groups)
    {
      // lane row q takes word q of its row block: two 16-lane swaps give rows [w0, w1, w0, w1] and
      // [w2, w3, w2, w3], a 32-lane swap joins their halves
      uint32_t bw[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const auto t01 = __builtin_amdgcn_permlane16_swap(sw[rb][0], sw[rb][1], false, false);
        const auto t23 = __builtin_amdgcn_permlane16_swap(sw[rb][2], sw[rb][3], false, false);
        bw[rb] = __builtin_amdgcn_permlane32_swap(t01[0], t23[0], false, false)[0];
      }
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        if (th < nh) {
          const float a = q < U ? s_lds[(k * U + q) * kTileM + 16 * th + c16] : 0.0f;
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            const float b = q < U ? __builtin_bit_cast(float, bw[rb] & 0xFFFF0000u) : 0.0f;
            accb[th][rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, accb[th][rb], 0, 0, 0);
          }
        }
      }
    }
    // B dwords per row block, group and MFMA half
    uint32_t bd[2][4][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if constexpr (BITS == 4) {
#pragma unroll
        for (int c = 0; c < NI; ++c) {
          const u32x4_t v = st.v[rb][c];
          const auto p = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
          const auto r = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
          bd[rb][2 * c][0] = p[0]; bd[rb][2 * c + 1][0] = p[1];
          bd[rb][2 * c][1] = r[0]; bd[rb][2 * c + 1][1] = r[1];
        }
      } else {
        const u32x4_t v = st.v[rb][0];
        const auto x02 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
        const auto y01 = __builtin_amdgcn_permlane16_swap(x02[0], x13[0], false, false);
        const auto y23 = __builtin_amdgcn_permlane16_swap(x02[1], x13[1], false, false);
        const uint32_t t4[4] = {y01[0], y01[1], y23[0], y23[1]};
#pragma unroll
        for (int G = 0; G < 4; ++G) bd[rb][G][0] = bd[rb][G][1] = t4[G];
      }
    }
#pragma unroll
    for (int G = 0; G < U; ++G) {
      f16x8_t b[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) b[rb][h] = codes_f16<BITS>(bd[rb][G][h], h);
      float sc[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sc[rb] = bf16_val((uint16_t)(sw[rb][G] & 0xFFFFu));
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        if (th < nh) {
          const f16x8_t a0 = a_frag(s, th, G, 0), a1 = a_frag(s, th, G, 1);
          // down: the group's unscale factors of tokens 16 th + 4 q + e (gate/up undoes its
          // per-token factor once, in the epilogue)
          f32x4_t u = {1.0f, 1.0f, 1.0f, 1.0f};
          if constexpr (!GATEUP) u = *reinterpret_cast<const f32x4_t*>(&u_lds[(k * U + G) * kTileM + 16 * th + 4 * q]);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) {
            f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b[rb][0], d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b[rb][1], d, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (GATEUP) acc[th][rb][e] = fmaf(sc[rb], d[e], acc[th][rb][e]);
              else acc[th][rb][e] = fmaf(sc[rb] * u[e], d[e], acc[th][rb][e]);
            }
          }
        }
      }
#if BQ_GROUP_SCHED_BARRIER
      // one group at a time: keeps the scheduler from widening every group of the step up front
      // (without it the down GEMMs measured 295 -> 384 us at prefill4; gate/up the same within noise)
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
  };

  // End of a slab: write its outputs and clear the accumulators. Element e of acc[th][rb] holds
  // token 16*th + 4*q + e and weight row slab*ROWS_B + wrow + 16*rb + c16. (Block-uniform; holds
  // barriers.)
  auto finish_slab = [&](int slab) __attribute__((always_inline)) {
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[th][rb][e] += accb[th][rb][e];
          accb[th][rb][e] = 0.0f;
        }
    if constexpr (GATEUP) {
      // the gate waves hand their results to the up waves that hold the same rows
      if (mi == 0) {
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) x_lds[wave][8 * th + 4 * rb + e][lane] = acc[th][rb][e];
      }
      __syncthreads();
      // The up waves finish the SwiGLU in fp32 (undoing the token's activation scaling first), then
      // cast to fp16 with a power of two per token from the largest |h| over the slab's 64 rows
      // (both up waves), and keep that factor's inverse for the down projection.
      const bool active = slab * ROWS_B + wrow < g.nout;  // wave-uniform
      float hv[2][2][4];
      if (mi == 1) {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          float mx[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float u = u_lds[16 * th + 4 * q + e];
              const float a = x_lds[wave - 2][8 * th + 4 * rb + e][lane] * u, c = acc[th][rb][e] * u;
              hv[th][rb][e] = silu_mul_fast(a, c);
              if (active && th < nh) mx[e] = fmaxf(mx[e], fabsf(hv[th][rb][e]));
            }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int msk = 8; msk >= 1; msk >>= 1) mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], msk, 16));
          }
          if (c16 == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) hm_lds[wave - 2][16 * th + 4 * q + e] = mx[e];
          }
        }
      }
      __syncthreads();
      if (mi == 1) {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
          if (th < nh) {
            float up[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 16 * th + 4 * q + e;
              up[e] = ldexpf(1.0f, fp16_exponent(fmaxf(hm_lds[0][m], hm_lds[1][m])));
            }
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const int row = slab * ROWS_B + wrow + 16 * rb + c16;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = 16 * th + 4 * q + e;
                const _Float16 h = (_Float16)(hv[th][rb][e] * up[e]);
                if (active && m < count) g.oh[(size_t)orow(m) * g.nout + (row & ~7) + perm8(row & 7)] = h;
                part[e] += active ? (float)h : 0.0f;
              }
            }
          }
          // sum over the 32 rows of this wave (2 row blocks in-lane, 16 lanes), then over the two up
          // waves: the slab's 64 rows are one group of the down projection's input
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int msk = 8; msk >= 1; msk >>= 1) part[e] += __shfl_xor(part[e], msk, 16);
          }
          if (c16 == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) h_lds[wave - 2][16 * th + 4 * q + e] = part[e];
          }
        }
      }
      __syncthreads();
      const int col0 = slab * ROWS_B;
      if (tid < kTileM && tid < count && col0 < g.nout) {
        const float down = ldexpf(1.0f, -fp16_exponent(fmaxf(hm_lds[0][tid], hm_lds[1][tid])));
        const size_t o = (size_t)orow(tid) * (g.nout / 64) + col0 / 64;
        g.os[o] = (h_lds[0][tid] + h_lds[1][tid]) * down;
        g.oscale[o] = down;
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = slab * ROWS_B + wrow + 16 * rb + c16;
        if (row < g.nout) {
#pragma unroll
          for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 16 * th + 4 * q + e;
              if (m < count) g.oy[(size_t)orow(m) * g.nout + row] = acc[th][rb][e];
            }
        }
      }
    }
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[th][rb][e] = 0.0f;
  };

  // kStages code stages (step s computes stage s % kStages while the next kStages - 1 are in flight),
  // two activation register sets (step s loads set s % 2 with the activations of step s + 2 and
  // parks the other set, which holds step s + 1), and the (scale, bias) words of a step pair: wp is
  // loaded two steps ahead and split at the pair's first step into wx. The steps run in an unrolled
  // period of lcm(kStages, 2) so that every register set has a fixed name. Past the end a step
  // re-reads the last one, so every path issues the same loads.
  constexpr int kAhead = kStages - 1;
  Codes cst[kStages];
  Act a0, a1;
  GWords wp;
  GWordsX wx;
  auto body = [&](auto ci, auto ai, int s) __attribute__((always_inline)) {
    constexpr int CI = decltype(ci)::value, AI = decltype(ai)::value;
    Codes& cur = cst[CI];
    Codes& ahead = cst[(CI + kAhead) % kStages];  // stage (s + kAhead) % kStages
    Act& aload = AI == 0 ? a0 : a1;
    Act& apark = AI == 0 ? a1 : a0;
    if constexpr (AI == 0) split_words(wp, wx);
    if constexpr (!RESIDENT) load_act(aload, min(s + 2, ntot - 1));
    load_codes(ahead, min(s + kAhead, ntot - 1));
    if constexpr (AI == 0) load_words(wp, s / 2 + 1);
    if (s < ntot) {  // uniform per block
      compute(cur, wx.w[AI], s);
      if (s % NSTEP == NSTEP - 1) finish_slab(slab0 + s / NSTEP);
    }
    if constexpr (!RESIDENT) {
      park_act(apark, s + 1);
      __syncthreads();
    }
  };
  if constexpr (!RESIDENT) {
    load_act(a0, 0);
    load_act(a1, min(1, ntot - 1));
  }
  load_codes(cst[0], 0);
  load_words(wp, 0);
#pragma unroll
  for (int i = 1; i < kAhead; ++i) load_codes(cst[i], min(i, ntot - 1));
  if constexpr (!RESIDENT) park_act(a0, 0);
  __syncthreads();
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  static_assert(kStages == 3 || kStages == 4, "3 or 4 code stages");
  if constexpr (kStages == 3) {
#pragma unroll 1
    for (int s = 0; s < ntot; s += 6) {
      body(I0{}, I0{}, s);
      body(I1{}, I1{}, s + 1);
      body(I2{}, I0{}, s + 2);
      body(I0{}, I1{}, s + 3);
      body(I1{}, I0{}, s + 4);
      body(I2{}, I1{}, s + 5);
    }
  } else {
#pragma unroll 1
    for (int s = 0; s < ntot; s += 4) {
      body(I0{}, I0{}, s);
      body(I1{}, I1{}, s + 1);
      body(I2{}, I0{}, s + 2);
      body(I3{}, I1{}, s + 3);
    }
  }
}


// ---- MXFP4 experts on the scaled MX MFMA ------------------------------------------------------------
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = E4M3 activations and B = E2M1 codes, block scales
// applied by the matrix core (lane layout checked on the device): B lane j + 16q holds block q
// (32 codes = 16 bytes, lower nibble first) of column j with that block's scale; A lane i + 16q
// holds K = 16q..16q+15 (bytes 0-15) and K = 64+16q..64+16q+15 (bytes 16-31) of row i, with the
// scale of block q; D as for the other 16 x 16 MFMAs.
constexpr int kMxTerms = 3;

// 3-term MXFP8 expansion of fp32 rows (E4M3 values, one E8M0 scale per block of 32):
// x = sum_t q_t * 2^(e_t - 127) + r. Term t quantises what terms 0..t-1 left, with the block scale
// chosen so that the block's largest magnitude falls in [128, 256) (no E4M3 saturation); the
// residual is exact in fp32, and after three terms |r| is about 2^-12 of each element (less
// than fp16's rounding). A thread takes 8 consecutive elements (two 16-byte loads, one 8-byte store
// per term); 4 threads hold one block and share its maximum in 2 butterfly steps.
__global__ __launch_bounds__(kThreads) void k_prep_mx(int64_t nblk, const float* __restrict__ x, uint8_t* __restrict__ q8,
                                                      uint8_t* __restrict__ sc, uint64_t q_plane, uint64_t sc_plane) {
  const int64_t i8 = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // 8-element chunk
  const bool live = i8 < nblk * 4;  // a block's 4 threads agree (kThreads is a multiple of 4)
  const int64_t ib = live ? i8 : 0;
  const float4* src = reinterpret_cast<const float4*>(x) + 2 * ib;
  const float4 p0 = src[0], p1 = src[1];
  float r[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
  for (int t = 0; t < kMxTerms; ++t) {
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(r[k]));
    a = fmaxf(a, __shfl_xor(a, 1, 4));
    a = fmaxf(a, __shfl_xor(a, 2, 4));
    const int e = a > 0.0f ? max(-127, min(127, ilogbf(a) - 7)) : -127;
    const float down = ldexpf(1.0f, -e), up = ldexpf(1.0f, e);
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // y = r * 2^-e is exact, |y| < 256; bytes in element order
      w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[4 * h] * down, r[4 * h + 1] * down, 0, false);
      w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r[4 * h + 2] * down, r[4 * h + 3] * down, (int)w[h], true);
    }
    if (live) {
      *reinterpret_cast<uint2*>(q8 + t * q_plane + 8 * ib) = make_uint2(w[0], w[1]);
      if ((i8 & 3) == 0) sc[t * sc_plane + (ib >> 2)] = (uint8_t)(e + 127);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the residual, exact
      r[4 * h] -= __builtin_amdgcn_cvt_f32_fp8((int)w[h], 0) * up;
      r[4 * h + 1] -= __builtin_amdgcn_cvt_f32_fp8((int)w[h], 1) * up;
      r[4 * h + 2] -= __builtin_amdgcn_cvt_f32_fp8((int)w[h], 2) * up;
      r[4 * h + 3] -= __builtin_amdgcn_cvt_f32_fp8((int)w[h], 3) * up;
    }
  }
}

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x4m_t __attribute__((ext_vector_type(4)));

// KB MX K-blocks of 128 per step (KB = 2 wherever K allows): per row block KB code loads of 16 bytes
// and KB scale dwords in one load.
template <int KB>
struct MxCodes {
  u32x4_t v[2][KB];   // [row block][K-block]: 16 code bytes (block q of the K-block for lane q)
  uint32_t sc[2][KB]; // [row block][K-block]: the 4 E8M0 bytes of the lane's row
};
template <int KB>
struct MxAct {
  u32x4_t v[kMxTerms][KB];  // 16 bytes of each term: row tid/(8KB) + (32/KB)h, slot tid%(8KB)
};

template <int KB>
__device__ __forceinline__ void mx_load_scales(uint32_t (&d)[KB], __amdgpu_buffer_rsrc_t rs, int voff, int soff) {
  if constexpr (KB == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    d[0] = v[0];
    d[1] = v[1];
  } else {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
  }
}

// Block: as k_grouped (4 waves, a tile of up to 32 tokens as one or two 16-token halves, each wave
// 32 rows of one matrix per slab, slabs walked in order, XCD-aware tile placement). Step: K = 128 KB,
// i.e. 4 KB MX blocks: per row block KB 16-byte code loads (a whole 128-byte line of the row when
// KB = 2) and one scale load; the tile's three activation terms (12 KiB per K-block) through an LDS ring.
// The activations' E8M0 scales (3 KiB per 1024 of K) sit in LDS for the whole block.
// No dequantisation on the VALU: the MFMA consumes the packed codes and both scale sets.
template <int KDIM, bool GATEUP, bool SHARED>
__global__ __launch_bounds__(kThreads, GATEUP ? BQ_LB_GU : BQ_LB_DOWN) void k_grouped_mx(GroupArgs g, int sgroups) {
  static_assert(KDIM % 128 == 0, "K steps of 128");
  constexpr int KB = (KDIM % 256 == 0) ? 2 : 1;  // K-blocks per step
  constexpr int SLOTS = 8 * KB;                  // 16-byte activation slots per row and step
  constexpr int NSTEP = KDIM / (128 * KB);       // steps per slab
  constexpr int ROWB = KDIM / 2;                 // code bytes per row
  constexpr int NB = KDIM / 32;                  // scale bytes per row
  constexpr int ROWS_B = GATEUP ? 64 : 128;      // rows per matrix per slab
  __shared__ u32x4_t a_lds[2][kMxTerms][kTileM][SLOTS];  // [parity][term][row][16-byte slot ^ swizzle]
  // every activation scale of the tile, loaded once; rows padded by a dword so that the 16 rows of a
  // fragment read hit distinct banks
  __shared__ uint32_t sc_lds[kMxTerms][kTileM][NB / 4 + 1];
  __shared__ float x_lds[GATEUP ? 2 : 1][16][64];

  // the wave index through readfirstlane: the compiler then knows it is uniform, so the buffer
  // descriptors built from it (a matrix per wave in gate/up) stay in scalar registers; derived from
  // threadIdx alone it counts as divergent, and every buffer load became a waterfall loop
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c16 = lane & 15, q = lane >> 4;
  const int mi = GATEUP ? (wave >> 1) : 0;
  const int wrow = (GATEUP ? (wave & 1) : wave) * 32;
  const int b8 = 8 * sgroups;
  const int tau = (int)(blockIdx.x / b8) * 8 + (int)(blockIdx.x & 7);
  const int gy = (int)(blockIdx.x % b8) >> 3;
  int first, count;
  const uint8_t* blob;
  if constexpr (SHARED) {
    first = tau * kTileM;
    if (first >= g.T) return;  // uniform per block
    count = min(kTileM, g.T - first);
    blob = g.shared;
  } else {
    if (tau >= *g.ntiles) return;  // uniform per block
    const int e = g.tile_e[tau];
    first = g.tile_first[tau];
    count = min(kTileM, g.offsets[e + 1] - first);
    blob = g.experts + (size_t)e * g.stride;
  }
  const int nh = count > 16 ? 2 : 1;
  auto arow = [&](int m) -> int {
    const int mm = first + min(m, count - 1);
    if constexpr (SHARED) return GATEUP ? mm : g.shared_base + mm;
    else return GATEUP ? g.perm[mm] / g.K : mm;
  };
  auto orow = [&](int m) -> int { return SHARED ? g.shared_base + first + m : first + m; };
  // LDS slot swizzle: the 16 rows of a fragment read (and of a 16-lane write) hit distinct banks.
  // Rows of 128 bytes (KB = 1) alternate bank halves; rows of 256 bytes all start at bank 0.
  auto swz = [](int row, int slot) -> int { return KB == 2 ? (slot ^ (row & 15)) : (slot ^ ((row >> 1) & 7)); };

  // activation loads: row tid/SLOTS + (32/KB)h, slot tid%SLOTS of each term; the scales of (term, row)
  const int a_row = tid / SLOTS, a_slot = tid % SLOTS;
  // buffer loads: the planes' base in scalar registers, a 32-bit offset per lane, term and step as
  // scalar offsets (the host keeps the three planes under 2^31 bytes)
  const __amdgpu_buffer_rsrc_t ars =
      __builtin_amdgcn_make_buffer_rsrc((void*)g.a8, (short)0, (int)(kMxTerms * g.a_plane), kRsrcWord3);
  int a_off[KB];
#pragma unroll
  for (int h = 0; h < KB; ++h) a_off[h] = arow(a_row + (32 / KB) * h) * KDIM + a_slot * 16;
  // the tile's activation scales are the same for every slab: all of them go to LDS once
  {
    constexpr int NW = kMxTerms * kTileM * (NB / 4);
    for (int i = tid; i < NW; i += kThreads) {
      const int t = i / (kTileM * (NB / 4)), m = (i / (NB / 4)) % kTileM, d = i % (NB / 4);
      sc_lds[t][m][d] = *reinterpret_cast<const uint32_t*>(g.asc + t * g.sc_plane + (size_t)arow(m) * NB + 4 * d);
    }
  }
  auto load_act = [&](MxAct<KB>& r, int s) __attribute__((always_inline)) {
    const int k = s % NSTEP;
#pragma unroll
    for (int t = 0; t < kMxTerms; ++t)
#pragma unroll
      for (int h = 0; h < KB; ++h)
        r.v[t][h] = __builtin_amdgcn_raw_buffer_load_b128(ars, a_off[h], (int)(t * g.a_plane) + k * 128 * KB, 0);
  };
  auto park_act = [&](const MxAct<KB>& r, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kMxTerms; ++t)
#pragma unroll
      for (int h = 0; h < KB; ++h) {
        const int row = a_row + (32 / KB) * h;
        a_lds[s & 1][t][row][swz(row, a_slot)] = r.v[t][h];
      }
  };

  const int nslab = (g.nout + ROWS_B - 1) / ROWS_B;
  const int spb = (nslab + sgroups - 1) / sgroups;
  const int slab0 = gy * spb;
  const int ntot = (min(nslab, slab0 + spb) - slab0) * NSTEP;
  if (ntot <= 0) return;  // uniform per block
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_codes[mi]), (short)0, g.nout * ROWB, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_sb[mi]), (short)0, g.nout * NB, kRsrcWord3);
  // clamped rows and steps: every path issues the same loads (exact wait counts)
  auto load_codes = [&](MxCodes<KB>& st, int s) __attribute__((always_inline)) {
    const int slab = slab0 + s / NSTEP, k = s % NSTEP;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int row = min(slab * ROWS_B + wrow + 16 * rb + c16, g.nout - 1);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        st.v[rb][kb] = __builtin_amdgcn_raw_buffer_load_b128(crs, row * ROWB + 16 * q, (k * KB + kb) * 64, 0);
      mx_load_scales<KB>(st.sc[rb], srs, row * NB, k * 4 * KB);
    }
  };

  f32x4m_t acc[2][2];
#pragma unroll
  for (int th = 0; th < 2; ++th)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[th][rb] = f32x4m_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const MxCodes<KB>& st, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      v8i_t b[2];
      int sb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        b[rb] = v8i_t{(int)st.v[rb][kb][0], (int)st.v[rb][kb][1], (int)st.v[rb][kb][2], (int)st.v[rb][kb][3], 0, 0, 0, 0};
        sb[rb] = (int)((st.sc[rb][kb] >> (8 * q)) & 0xFFu);
      }
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        if (th < nh) {
          const int row = 16 * th + c16;
#pragma unroll
          for (int t = 0; t < kMxTerms; ++t) {
            const u32x4_t lo = a_lds[s & 1][t][row][swz(row, 8 * kb + q)];
            const u32x4_t hi = a_lds[s & 1][t][row][swz(row, 8 * kb + 4 + q)];
            const v8i_t a = v8i_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int sa = (int)((sc_lds[t][row][(s % NSTEP) * KB + kb] >> (8 * q)) & 0xFFu);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
              acc[th][rb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[rb], acc[th][rb], 0, 4, 0, sa, 0, sb[rb]);
          }
        }
      }
    }
  };

  // End of a slab: element e of acc[th][rb] is token 16*th + 4*q + e, row slab*ROWS_B + wrow + 16*rb + c16.
  auto finish_slab = [&](int slab) __attribute__((always_inline)) {
    if constexpr (GATEUP) {
      if (mi == 0) {
#pragma unroll
        for (int th = 0; th < 2; ++th)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) x_lds[wave][8 * th + 4 * rb + e][lane] = acc[th][rb][e];
      }
      __syncthreads();
      if (mi == 1 && slab * ROWS_B + wrow < g.nout) {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          if (th < nh) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
              const int row = slab * ROWS_B + wrow + 16 * rb + c16;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int m = 16 * th + 4 * q + e;
                const float a = x_lds[wave - 2][8 * th + 4 * rb + e][lane], c = acc[th][rb][e];
                if (m < count) g.oh32[(size_t)orow(m) * g.nout + row] = silu_mul_fast(a, c);
              }
            }
          }
        }
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = slab * ROWS_B + wrow + 16 * rb + c16;
        if (row < g.nout) {
#pragma unroll
          for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 16 * th + 4 * q + e;
              if (m < count) g.oy[(size_t)orow(m) * g.nout + row] = acc[th][rb][e];
            }
        }
      }
    }
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[th][rb] = f32x4m_t{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // Codes: three register stages, loaded two steps ahead. Activations: one register set, loaded at
  // the start of a step and parked at its end (loads retire in order, so parking waits for the
  // activations and not for the codes issued after them).
  MxCodes<KB> c0, c1, c2;
  MxAct<KB> act;
  auto body = [&](auto ci, int s) __attribute__((always_inline)) {
    constexpr int CI = decltype(ci)::value;
    MxCodes<KB>& cur = CI == 0 ? c0 : (CI == 1 ? c1 : c2);
    MxCodes<KB>& ahead = CI == 0 ? c2 : (CI == 1 ? c0 : c1);
    load_act(act, min(s + 1, ntot - 1));
    load_codes(ahead, min(s + 2, ntot - 1));
    if (s < ntot) {  // uniform per block
      compute(cur, s);
      if (s % NSTEP == NSTEP - 1) finish_slab(slab0 + s / NSTEP);
    }
    park_act(act, s + 1);
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  load_act(act, 0);
  load_codes(c0, 0);
  load_codes(c1, min(1, ntot - 1));
  park_act(act, 0);
  __syncthreads();
#pragma unroll 1
  for (int s = 0; s < ntot; s += 3) {
    body(I0{}, s);
    body(I1{}, s + 1);
    body(I2{}, s + 2);
  }
}

// ---- 6. combine (gather) / scatter ------------------------------------------------------------------
// out[t][r] = residual[t][r] + sum_k w[t][k] * y[pos[t*K+k]][r] + g[t] * y[T*K + t][r]   (combine)
// y_out[t][k][r] = y[pos[t*K+k]][r], y_out[t][K][r] = y[T*K + t][r]                       (scatter)
__global__ __launch_bounds__(kThreads) void k_prefill_out(int T, int H, int K, int E, int has_shared,
                                                          const int32_t* __restrict__ idx, int32_t* __restrict__ err,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ y, const float* __restrict__ w,
                                                          const float* __restrict__ sg,
                                                          const float* __restrict__ residual,
                                                          float* __restrict__ out, float* __restrict__ y_out) {
  // 4 consecutive rows per thread (H is a multiple of 64): 16-byte loads of y (workspace) and
  // stores of out and y_out (16-byte aligned by the entry points' checks); the residual, which
  // carries no alignment requirement, is read as 4 floats
  const int t = blockIdx.y;
  const int r = 4 * (blockIdx.x * kThreads + threadIdx.x);
  if (r >= H) return;
  const int NE = K + has_shared;
  auto row4 = [&](size_t row) { return *reinterpret_cast<const float4*>(y + row * H + r); };
  if (out != nullptr) {
    const float* rs = residual + (size_t)t * H + r;
    float4 acc = make_float4(rs[0], rs[1], rs[2], rs[3]);
    for (int k = 0; k < K; ++k) {
      const float wk = w[(size_t)t * K + k];
      const float4 v = row4((size_t)pos[(size_t)t * K + k]);
      acc.x += wk * v.x; acc.y += wk * v.y; acc.z += wk * v.z; acc.w += wk * v.w;
    }
    if (has_shared) {
      const float gs = sg[t];
      const float4 v = row4((size_t)T * K + t);
      acc.x += gs * v.x; acc.y += gs * v.y; acc.z += gs * v.z; acc.w += gs * v.w;
    }
    *reinterpret_cast<float4*>(out + (size_t)t * H + r) = acc;
  } else {
    for (int k = 0; k < K; ++k) {
      const int e = idx[(size_t)t * K + k];
      float4 v = make_float4(NAN, NAN, NAN, NAN);
      if (e >= 0 && e < E) v = row4((size_t)pos[(size_t)t * K + k]);
      else if (err != nullptr && r == 0) *err = MOE_EINVAL;
      *reinterpret_cast<float4*>(y_out + ((size_t)t * NE + k) * H + r) = v;
    }
    if (has_shared) *reinterpret_cast<float4*>(y_out + ((size_t)t * NE + K) * H + r) = row4((size_t)T * K + t);
  }
}

unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

template <int BITS>
constexpr int kULine = BQ_U_LINE * 4;

// Blocks: one per tile, times enough slab groups that a launch has about BQ_GROUP_TARGET working
// blocks. `tiles` is the number expected to hold tokens: for the routed experts at most one per
// routed entry. Measured at 2048 tokens (704 tile slots for the routed experts):
//  - routed: at least 4 slab groups per tile (BQ_ROUTED_MIN_GROUPS) balance the launch's tail
//    better than one block per tile: gate/up 670-690 -> 607-622 us, down 307 -> 287 us; 5 groups
//    measured the same, 8 slower for gate/up; prefillmx (896 tile slots) 1.83 -> 1.54 ms per step
//    with 4 groups, 1.58 with 3;
//  - shared (64 tiles): 512, two blocks per CU with two slabs each, so the pipeline fills half as
//    often as with 1024 (gate/up 97 -> 93 us, down 52 -> 43 us; 256 and 2048 were slower).
#ifndef BQ_GROUP_TARGET
#define BQ_GROUP_TARGET 3072
#endif
#ifndef BQ_SHARED_GROUP_TARGET
#define BQ_SHARED_GROUP_TARGET 512
#endif
#ifndef BQ_ROUTED_MIN_GROUPS
#define BQ_ROUTED_MIN_GROUPS 4
#endif
int slab_groups(int tiles, int nout, int rows_per_slab, int target, int min_groups) {
  const int nslab = (nout + rows_per_slab - 1) / rows_per_slab;
  return std::max(1, std::min(nslab, std::max(min_groups, target / std::max(1, tiles))));
}
// 1-D grid for `tiles` tile slots with `sg` slab groups each, in runs of 8 tiles (see k_grouped).
unsigned grouped_grid(int tiles, int sg) { return cdiv(tiles, 8) * 8u * (unsigned)sg; }

template <int BITS, int KDIM, bool GATEUP>
hipError_t launch_grouped(const GroupArgs& ga, int nout, int T, int N, int E, bool routed, bool has_shared,
                          hipStream_t s) {
  constexpr int UM = kULine<BITS>;
  constexpr int RS = GATEUP ? 64 : 128;  // rows per matrix per slab
  const dim3 block(kThreads);
  const int max_tiles = E + (int)cdiv(N, kTileM);
  const int rg = slab_groups(std::min(max_tiles, N), nout, RS, BQ_GROUP_TARGET, BQ_ROUTED_MIN_GROUPS);
  if (routed)
    hipLaunchKernelGGL((k_grouped<BITS, KDIM, UM, GATEUP, false>), dim3(grouped_grid(max_tiles, rg)), block, 0, s,
                       ga, rg);
  if (has_shared) {
    const int st = (int)cdiv(T, kTileM);
    const int sg = slab_groups(st, nout, RS, BQ_SHARED_GROUP_TARGET, 1);
    hipLaunchKernelGGL((k_grouped<BITS, KDIM, UM, GATEUP, true>), dim3(grouped_grid(st, sg)), block, 0, s, ga,
                       sg);
  }
  return hipGetLastError();
}

template <int KDIM, bool GATEUP>
hipError_t launch_grouped_mx(const GroupArgs& ga, int nout, int T, int N, int E, bool routed, bool has_shared,
                             hipStream_t s) {
  constexpr int RS = GATEUP ? 64 : 128;
  const dim3 block(kThreads);
  const int max_tiles = E + (int)cdiv(N, kTileM);
  const int rg = slab_groups(std::min(max_tiles, N), nout, RS, BQ_GROUP_TARGET, BQ_ROUTED_MIN_GROUPS);
  if (routed)
    hipLaunchKernelGGL((k_grouped_mx<KDIM, GATEUP, false>), dim3(grouped_grid(max_tiles, rg)), block, 0, s, ga, rg);
  if (has_shared) {
    const int st = (int)cdiv(T, kTileM);
    const int sg = slab_groups(st, nout, RS, BQ_SHARED_GROUP_TARGET, 1);
    hipLaunchKernelGGL((k_grouped_mx<KDIM, GATEUP, true>), dim3(grouped_grid(st, sg)), block, 0, s, ga, sg);
  }
  return hipGetLastError();
}

#define BQ_FOR_KDIM_GU(X) X(256) X(512) X(1024) X(2048) X(4096) X(8192)
#define BQ_FOR_KDIM_DN(X) X(64) X(128) X(256) X(512) X(1024) X(2048)

#define BQ_FOR_KDIM_MX(X) X(128) X(256) X(512) X(1024) X(2048) X(4096) X(8192)
hipError_t dispatch_mx(bool gateup, int kdim, const GroupArgs& ga, int nout, int T, int N, int E, bool routed, bool hs,
                       hipStream_t s) {
#define BQ_CASE(KV)                                                                        \
  case KV:                                                                                 \
    return gateup ? launch_grouped_mx<KV, true>(ga, nout, T, N, E, routed, hs, s)          \
                  : launch_grouped_mx<KV, false>(ga, nout, T, N, E, routed, hs, s);
  switch (kdim) { BQ_FOR_KDIM_MX(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

// Rows [row0, row0 + nrows) of a [rows][cols] array into planes of rows * cols codes and
// rows * cols / 32 scales.
hipError_t launch_prep_mx(int rows, int row0, int nrows, int cols, const float* x, uint8_t* q8, uint8_t* sc,
                          hipStream_t s) {
  const int64_t nblk = (int64_t)nrows * cols / 32, off = (int64_t)row0 * cols;
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prep_mx, dim3(cdiv(nblk * 4, kThreads)), dim3(kThreads), 0, s, nblk, x + off, q8 + off,
                     sc + off / 32, (uint64_t)rows * cols, (uint64_t)rows * cols / 32);
  return hipGetLastError();
}

hipError_t dispatch_gateup(int bits, int H, const GroupArgs& ga, int I, int T, int N, int E, bool routed, bool hs,
                           hipStream_t s) {
#define BQ_CASE(KV)                                                                   \
  case KV:                                                                            \
    return bits == 4 ? launch_grouped<4, KV, true>(ga, I, T, N, E, routed, hs, s)     \
                     : launch_grouped<2, KV, true>(ga, I, T, N, E, routed, hs, s);
  switch (H) { BQ_FOR_KDIM_GU(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t dispatch_down(int bits, int I, const GroupArgs& ga, int H, int T, int N, int E, bool routed, bool hs,
                         hipStream_t s) {
#define BQ_CASE(KV)                                                                   \
  case KV:                                                                            \
    return bits == 4 ? launch_grouped<4, KV, false>(ga, H, T, N, E, routed, hs, s)    \
                     : launch_grouped<2, KV, false>(ga, H, T, N, E, routed, hs, s);
  switch (I) { BQ_FOR_KDIM_DN(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_router_gemm(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_router_gemm, dim3(cdiv(g.E + g.has_shared, kRW), cdiv(T, kRW)), dim3(64 * kRSplit), 0, s, T,
                     g.H, g.E, g.has_shared, x, p.router, p.sgate, ws.logits);
  return hipGetLastError();
}

hipError_t launch_router_tokens(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                hipStream_t s) {
  // the fp64 GEMM fills the chip only for many tokens; below that, per-token router rows win
  if (T >= kRouterGemmMinTokens) return launch_router_gemm(g, p, x, T, ws, s);
  return launch_router_phase(g, p, x, nullptr, 0.0f, T, ws, s);
}

hipError_t launch_router_approx(const Geometry& g, const LayerPtrs& p, const float* x, int T, double* logits,
                                double* kc_out, hipStream_t s) {
  int rt = BQ_ROUTER_APPROX_RT;
  if (rt == 0) {  // the smallest tile whose grid fits one block per CU (256), else the largest
    rt = 8;
    for (int c : {2, 4})
      if (cdiv(g.E, 16 * c) * cdiv(T, kAT) <= 256) {
        rt = c;
        break;
      }
  }
  const dim3 ag(cdiv(g.E, 16 * rt), cdiv(T, kAT)), ab(64 * kASplit);
  if (rt == 8)
    hipLaunchKernelGGL(k_router_approx<8>, ag, ab, 0, s, T, g.H, g.E, x, p.router, logits);
  else if (rt == 4)
    hipLaunchKernelGGL(k_router_approx<4>, ag, ab, 0, s, T, g.H, g.E, x, p.router, logits);
  else
    hipLaunchKernelGGL(k_router_approx<2>, ag, ab, 0, s, T, g.H, g.E, x, p.router, logits);
  // Error bound of the approximate logits, relative to |r_e| |x_t|:
  //  - splitting x into two bf16 values leaves |d| <= 2^-16 |x|, and |hi| + |lo| <= 1.01 |x|;
  //  - one MFMA adds 32 exact products to its accumulator with an error of at most 34 * 2^-23 times
  //    the sum of the magnitudes it adds (per-addition rounding, to nearest or toward zero, or
  //    operands aligned and truncated to fp32 precision);
  //  - a wave chains n = 2 H / (32 * kASplit) MFMAs (hi and lo parts), so its error is at most
  //    34 * 2^-23 * n * (1 + 34 * 2^-23 * n) times its sum of |r| (|hi| + |lo|);
  //  - the sum of |r_j| |x_j| is at most |r| |x| (Cauchy-Schwarz), and the fp64 sums around
  //    this (the waves' partial sums, the norms, the exact recomputation) are far below it.
  // The factor 1.25 is a safety margin on all of it; the errors measured on the 2048-token
  // workloads stay far inside the bound (a test asserts below a quarter of it).
  const double n = 2.0 * g.H / (32.0 * kASplit);
  const double u = std::ldexp(1.0, -23);
  *kc_out = 1.25 * (std::ldexp(1.0, -16) * 1.01 + 34.0 * u * n * (1.0 + 34.0 * u * n) * 1.01);
  return hipGetLastError();
}

hipError_t launch_router_select(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                int32_t* idx, float* w, float* sg, double* logits_out, int32_t* idx_b,
                                hipStream_t s) {
  if (logits_out != nullptr || T < kRouterCertifiedMinTokens) {
    hipError_t e = launch_router_tokens(g, p, x, T, ws, s);
    return e == hipSuccess ? launch_topk(g, T, ws, idx, w, sg, logits_out, idx_b, s) : e;
  }
  double kc = 0.0;
  hipError_t e = launch_router_approx(g, p, x, T, ws.logits, &kc, s);
  if (e != hipSuccess) return e;
  return launch_topk_certified(g, p, x, T, ws, kc, idx, w, sg, idx_b, s);
}

hipError_t launch_prefill(const Geometry& g, const LayerPtrs& p, const float* x, const float* residual, int T,
                          const PrefillWorkspace& w, const int32_t* idx_in, int32_t* idx_out, float* out,
                          float* y_out, int32_t* err, hipStream_t s) {
  const int H = g.H, I = g.I, E = g.E, K = g.K;
  const int N = T * K;
  const int nchunks = (int)cdiv(N, kChunk);
  const bool mx = g.form == 3;
  const int R = N + (g.has_shared ? T : 0);  // SwiGLU rows: the routed entries, then the shared expert's
  if (mx) {
    hipError_t e = launch_prep_mx(T, 0, T, H, x, w.x8, w.xsc, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(k_prep, dim3(T), dim3(kThreads), 0, s, H, x, reinterpret_cast<_Float16*>(w.xq), w.xs, w.xu);
  }
  const bool shared_here = g.has_shared != 0;
  const int32_t* idx = idx_in;
  if (idx_in == nullptr) {
    hipError_t e = launch_router_select(g, p, x, T, w.layer, w.layer.idx, w.layer.w, w.layer.g, nullptr, idx_out, s);
    if (e != hipSuccess) return e;
    idx = w.layer.idx;
  }
  hipLaunchKernelGGL(k_group_hist, dim3(nchunks), dim3(kChunk), E * sizeof(int32_t), s, N, E, idx, w.hist);
  hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, s, nchunks, E, kTileM, w.hist, w.counts,
                     w.offsets, w.tile_e, w.tile_first, w.ntiles);
  hipLaunchKernelGGL(k_group_place, dim3(nchunks), dim3(kChunk), 0, s, N, E, idx, w.hist, w.offsets, w.pos, w.perm);
  GroupArgs ga{};
  ga.experts = p.experts; ga.stride = p.stride; ga.shared = p.shared;
  ga.perm = w.perm; ga.K = K; ga.tile_e = w.tile_e; ga.tile_first = w.tile_first; ga.ntiles = w.ntiles;
  ga.offsets = w.offsets; ga.shared_base = N; ga.T = T;
  // gate/up + SwiGLU
  ga.off_codes[0] = g.off_codes[0]; ga.off_codes[1] = g.off_codes[1];
  ga.off_sb[0] = g.off_sb[0]; ga.off_sb[1] = g.off_sb[1];
  if (mx) {
    ga.a8 = w.x8; ga.asc = w.xsc; ga.a_plane = (uint64_t)T * H; ga.sc_plane = (uint64_t)T * H / 32;
    ga.oh32 = w.h32; ga.nout = I;
    hipError_t e = dispatch_mx(true, H, ga, I, T, N, E, true, shared_here, s);
    if (e == hipSuccess) e = launch_prep_mx(R, 0, shared_here ? R : N, I, w.h32, w.h8, w.hsc, s);
    if (e != hipSuccess) return e;
    ga.off_codes[0] = g.off_codes[2]; ga.off_sb[0] = g.off_sb[2];
    ga.a8 = w.h8; ga.asc = w.hsc; ga.a_plane = (uint64_t)R * I; ga.sc_plane = (uint64_t)R * I / 32;
    ga.oy = w.y; ga.nout = H;
    e = dispatch_mx(false, I, ga, H, T, N, E, true, shared_here, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_prefill_out, dim3(cdiv(H / 4, kThreads), T), dim3(kThreads), 0, s, T, H, K, E, g.has_shared,
                       idx, err, w.pos, w.y, w.layer.w, w.layer.g, residual, out, y_out);
    return hipGetLastError();
  }
  ga.a = reinterpret_cast<const _Float16*>(w.xq); ga.as = w.xs; ga.ascale = w.xu;
  ga.oh = reinterpret_cast<_Float16*>(w.hq); ga.os = w.hs; ga.oscale = w.hu; ga.nout = I;
  hipError_t e = dispatch_gateup(g.bits, H, ga, I, T, N, E, true, shared_here, s);
  if (e != hipSuccess) return e;
  // down
  ga.off_codes[0] = g.off_codes[2]; ga.off_sb[0] = g.off_sb[2];
  ga.a = reinterpret_cast<const _Float16*>(w.hq); ga.as = w.hs; ga.ascale = w.hu;
  ga.oy = w.y; ga.nout = H;
  e = dispatch_down(g.bits, I, ga, H, T, N, E, true, shared_here, s);
  if (e != hipSuccess) return e;
  // combine or scatter
  hipLaunchKernelGGL(k_prefill_out, dim3(cdiv(H / 4, kThreads), T), dim3(kThreads), 0, s, T, H, K, E, g.has_shared,
                     idx, err, w.pos, w.y, w.layer.w, w.layer.g, residual, out, y_out);
  return hipGetLastError();
}

}  // namespace bqmoe
