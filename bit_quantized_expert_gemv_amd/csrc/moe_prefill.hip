// Prefill path of the quantised MoE layer for MI355X (gfx950): many tokens through one layer,
// grouped by expert so that each expert's weights are streamed once per tile of tokens.
//
//   1. prep: activations to fp16 (each 8-block stored in the order 0,2,4,6,1,3,5,7, the order in
//      which the code widening below produces weights) and per-64-group sums of the fp16 values;
//   2. router: logits = X . [R; gate]^T as an fp64 tiled GEMM, so the top-K decision is exact
//      up to fp64 rounding; then the top-K and weights per token (the decode top-K kernel);
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
// inside its error bound.
//
// MFMA: v_mfma_f32_32x32x16_f16 with A = activations (32 token rows) and B = codes (32 weight
// rows). A[i][k] sits in lane i + 32*(k/8), element k%8; B[k][j] in lane j + 32*(k/8), element k%8;
// D[i][j] in lane j + 32*((i/4)%2), element (i/8)*4 + i%4 (checked on the device). The sum over k is
// order-free, so a lane's 16-byte code load (32 codes of one row, half a 4-bit group) supplies
// MFMAs m = 0..3 with codes 8m..8m+7. Lanes 32..63 hold the other half of the same group, so every
// MFMA stays inside one scale group, and the activation operand is read in the same k order.
#include <hip/hip_runtime.h>

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

// Stored position of element e (0..7) of an 8-block: the order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ int perm8(int e) { return (e >> 1) + 4 * (e & 1); }

// ---- 1. activation prep -------------------------------------------------------------------------
// One block per token: fp16 copy (8-blocks permuted) and per-64-group sums of the fp16 values.
__global__ __launch_bounds__(kThreads) void k_prep(int H, const float* __restrict__ x, _Float16* __restrict__ xq,
                                                   float* __restrict__ xs) {
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * H;
  const int ng = H / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int gi = wave; gi < ng; gi += kThreads / 64) {
    const int j = gi * 64 + lane;
    const _Float16 q = (_Float16)xr[j];
    xq[(size_t)t * H + (j & ~7) + perm8(j & 7)] = q;
    float v = (float)q;
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) xs[(size_t)t * ng + gi] = v;
  }
}

// ---- 2. router GEMM (fp64 MFMA) ---------------------------------------------------------------------
// logits[t][e] = sum_j R[e][j] x[t][j] for e < E, and the shared-gate vector as row E, on
// v_mfma_f64_16x16x4_f64: every bf16 x fp32 product is exact in fp64 and the sums are fp64, so the
// top-K decision is exact up to fp64 rounding. Lane layout (checked on the device): A[i][k] in lane
// i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane j + 16*(i%4), element i/4.
// Block: 4 waves, 64 tokens x 32 rows; wave (wt, wr) owns tokens 32wt..32wt+31 x rows 16wr..16wr+15
// as two 16 x 16 tiles that share the row operand. Operands are staged in LDS as fp64, token- or
// row-major with a 34-double stride: a fragment read (16 rows x 4 consecutive k per 32-lane pass)
// and the 16-byte staging writes both touch distinct banks. The next k-slice is in flight during
// the MFMAs.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef double f64x2_t __attribute__((ext_vector_type(2)));
constexpr int kRTok = 64, kRRow = 32, kRK = 32, kRS = kRK + 2;
#ifndef BQ_ROUTER_GEMM_MIN
#define BQ_ROUTER_GEMM_MIN 256
#endif
constexpr int kRouterGemmMinTokens = BQ_ROUTER_GEMM_MIN;
__global__ __launch_bounds__(kThreads) void k_router_gemm(int T, int H, int E, int has_shared,
                                                          const float* __restrict__ x,
                                                          const uint16_t* __restrict__ router,
                                                          const uint16_t* __restrict__ sgate,
                                                          double* __restrict__ logits) {
  __shared__ double xs[kRTok][kRS];
  __shared__ double rs[kRRow][kRS];
  const int t0 = blockIdx.y * kRTok, e0 = blockIdx.x * kRRow;
  const int nrows = E + has_shared;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, kk = lane >> 4;
  const int wt = wave >> 1, wr = wave & 1;
  // staging: x as (token tid/4, k 8*(tid%4) .. +7); R as (row tid/8, k 4*(tid%8) .. +3)
  const int xt = tid >> 2, xk = (tid & 3) * 8;
  const int rr = tid >> 3, rk = (tid & 7) * 4;
  const float* xp = x + (size_t)min(t0 + xt, T - 1) * H + xk;
  const int er = min(e0 + rr, nrows - 1);
  const uint16_t* rp = ((er < E) ? router + (size_t)er * H : sgate) + rk;
  float4 xv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) xv[q] = *reinterpret_cast<const float4*>(xp + 4 * q);
  uint2 rv = *reinterpret_cast<const uint2*>(rp);
  f64x4_t acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    f64x2_t* xw = reinterpret_cast<f64x2_t*>(&xs[xt][xk]);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      xw[2 * q] = f64x2_t{(double)xv[q].x, (double)xv[q].y};
      xw[2 * q + 1] = f64x2_t{(double)xv[q].z, (double)xv[q].w};
    }
    f64x2_t* rw = reinterpret_cast<f64x2_t*>(&rs[rr][rk]);
    const uint32_t rw32[2] = {rv.x, rv.y};
#pragma unroll
    for (int q = 0; q < 2; ++q)
      rw[q] = f64x2_t{(double)bf16_val((uint16_t)(rw32[q] & 0xFFFFu)), (double)bf16_val((uint16_t)(rw32[q] >> 16))};
    __syncthreads();
    if (k0 + kRK < H) {  // next slice in flight during the MFMAs
#pragma unroll
      for (int q = 0; q < 2; ++q) xv[q] = *reinterpret_cast<const float4*>(xp + k0 + kRK + 4 * q);
      rv = *reinterpret_cast<const uint2*>(rp + k0 + kRK);
    }
#pragma unroll
    for (int s4 = 0; s4 < kRK / 4; ++s4) {
      const double bv = rs[wr * 16 + c][4 * s4 + kk];
      const double a0 = xs[wt * 32 + c][4 * s4 + kk];
      const double a1 = xs[wt * 32 + 16 + c][4 * s4 + kk];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, bv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, bv, acc1, 0, 0, 0);
    }
    __syncthreads();
  }
  const int e = e0 + wr * 16 + c;
  if (e >= nrows) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ta = t0 + wt * 32 + kk + 4 * q;
    if (ta < T) logits[(size_t)ta * (E + 1) + e] = acc0[q];
    if (ta + 16 < T) logits[(size_t)(ta + 16) * (E + 1) + e] = acc1[q];
  }
}

// ---- 3. grouping by expert --------------------------------------------------------------------------
// Entries i = t*K + k (token t, slot k) carry expert idx[i]. Chunks of 256 entries.
constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void k_group_hist(int N, int E, const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kChunk + threadIdx.x;
  if (i < N) atomicAdd(&cnt[idx[i]], 1);  // counts do not depend on the order of the adds
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
// counts, offsets and the tile list (tiles of BM entries per expert, in expert order). The chunk
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
  const int nt = (e < E) ? (run + BM - 1) / BM : 0;
  int total_entries, total_tiles;
  const int off = block_exclusive_scan(e < E ? run : 0, wsum, &total_entries);
  const int t0 = block_exclusive_scan(nt, wsum, &total_tiles);
  if (e < E) {
    offsets[e] = off;
    for (int j = 0; j < nt; ++j) {
      tile_e[t0 + j] = e;
      tile_first[t0 + j] = off + j * BM;
    }
  }
  if (e == 0) {
    offsets[E] = total_entries;
    *ntiles = total_tiles;
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
  const int e = (i < N) ? idx[i] : -1;
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
  float* oy;  // down: [rows][nout]
  int nout;
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

// Per-lane registers of U groups of weights: codes and (scale, bias) words.
template <int BITS, int NTILE, int U>
struct GStage {
  static constexpr int CW = BITS == 4 ? 4 : 2;  // code dwords per lane per group
  uint32_t c[U][NTILE][CW];
  uint32_t sb[U][NTILE];
};

#ifndef BQ_LB_GU
#define BQ_LB_GU 3
#endif
#ifndef BQ_LB_DOWN
#define BQ_LB_DOWN 3
#endif
#ifndef BQ_GROUP_SCHED_BARRIER
#define BQ_GROUP_SCHED_BARRIER 1
#endif
#ifndef BQ_U_LINE
#define BQ_U_LINE 1
#endif
#ifndef BQ_ST_GU
#define BQ_ST_GU 2
#endif
#ifndef BQ_ST_DOWN
#define BQ_ST_DOWN 2
#endif
// Groups per pipeline step (by default one 128-byte line of every row: 4 groups at 4-bit, 8 at
// 2-bit, so that no line is fetched twice) and weight stages in flight + 1.
// Block: 4 waves, one tile of up to 32 token rows, all rows of the weight matrices. Each wave owns
// one 32-row tile of one matrix in every slab: for down, waves 0..3 take rows 32w..32w+31 of a
// 128-row slab; for gate/up, waves 0, 1 take 32-row tiles of gate and waves 2, 3 the same rows of
// up, in a 64-row slab, and the SwiGLU pairs meet through LDS at the end of the slab. One tile
// per wave keeps a wave's registers low enough for three waves per SIMD. The block walks the
// slabs one after the other, and the pipeline runs over the flattened (slab, step) sequence, so
// it fills once per block rather than once per slab; there are about as many blocks as tiles.
//
// Pipeline, per step of U groups: the tile's activations for the next step are loaded (16 bytes
// per thread and group), then each wave's weights for the step STAGES-1 ahead; this step is
// computed from registers (weights) and an LDS ring (activations); the next step's activations are
// parked in the ring and one barrier closes the step. Loads retire in order, so the activations are
// requested before the weights: waiting for them never waits for the weights in flight.
template <int BITS, int KDIM, int UMAX, int STAGES, bool GATEUP, bool SHARED>
__global__ __launch_bounds__(kThreads, GATEUP ? BQ_LB_GU : BQ_LB_DOWN) void k_grouped(GroupArgs g) {
  constexpr int NG = KDIM / 64;
  constexpr int U = NG >= UMAX ? UMAX : NG;  // groups per pipeline step
  constexpr int NSTEP = NG / U;               // steps per slab
  constexpr int ROWB = KDIM * BITS / 8;
  constexpr int GB = 64 * BITS / 8;  // code bytes per row and group
  constexpr int LB = GB / 2;         // per lane half
  constexpr int ROWS_B = GATEUP ? 64 : 128;  // rows per matrix per slab
  constexpr int AS = U * 8;          // 16-byte activation slots per row and step
  constexpr int ASW = AS >= 16 ? 15 : AS - 1;  // slot swizzle: 16 consecutive rows hit distinct banks
  using Stage = GStage<BITS, 1, U>;
  __shared__ float s_lds[NG * kTileM];             // group sums of the tile's activations, [group][row]
  __shared__ u32x4_t a_lds[2][kTileM * AS];        // activation ring: [step parity][row][slot ^ swizzle]
  __shared__ float x_lds[GATEUP ? 2 : 1][16][64];  // gate/up: gate results handed to the up waves
  __shared__ float h_lds[GATEUP ? 2 : 1][kTileM];  // gate/up: per-wave sums of the fp16 SwiGLU outputs

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hk = lane >> 5;
  const int mi = GATEUP ? (wave >> 1) : 0;         // matrix of this wave (gate 0, up 1)
  const int wrow = (GATEUP ? (wave & 1) : wave) * 32;  // first row of this wave in a slab
  const int tau = blockIdx.x;
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
  }
  // this thread's 16-byte activation slot: row tid/8, slot tid%8 of every group
  const int a_row = tid >> 3, a_slot = tid & 7;
  const u32x4_t* a_src = reinterpret_cast<const u32x4_t*>(g.a + (size_t)arow(a_row) * KDIM) + a_slot;
  u32x4_t a_reg[U];
  auto load_act = [&](int s) {  // s: flattened step; the activations depend on its step in the slab only
    const int k = s % NSTEP;
#pragma unroll
    for (int u = 0; u < U; ++u) a_reg[u] = a_src[(k * U + u) * 8];
  };
  auto park_act = [&](int s) {
#pragma unroll
    for (int u = 0; u < U; ++u) a_lds[s & 1][a_row * AS + ((u * 8 + a_slot) ^ (a_row & ASW))] = a_reg[u];
  };

  // this block's slabs: blockIdx.y of gridDim.y equal ranges (more blocks when there are few tiles)
  const int nslab = (g.nout + ROWS_B - 1) / ROWS_B;
  const int spb = (nslab + gridDim.y - 1) / gridDim.y;
  const int slab0 = blockIdx.y * spb;
  const int ntot = (min(nslab, slab0 + spb) - slab0) * NSTEP;  // flattened steps
  if (ntot <= 0) return;  // uniform per block
  // Weights through buffer loads: a descriptor per section (scalar registers), a 32-bit lane
  // offset, and the step's group offset as a scalar. Rows past nout are clamped.
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_codes[mi]), (short)0, g.nout * ROWB, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(blob + g.off_sb[mi]), (short)0, g.nout * NG * 4, kRsrcWord3);
  // unconditional (past the end, a clamped step is re-read): a load skipped on some path would
  // make the compiler's wait counts conservative and drain the prefetch
  auto load_w = [&](Stage& st, int s) {
    const int slab = slab0 + s / NSTEP, k = s % NSTEP;
    const int row = min(slab * ROWS_B + wrow + j, g.nout - 1);
    const int voff = row * ROWB + hk * LB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (BITS == 4) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(crs, voff, (k * U + u) * GB, 0);
        st.c[u][0][0] = v[0]; st.c[u][0][1] = v[1]; st.c[u][0][2] = v[2]; st.c[u][0][3] = v[3];
      } else {
        const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(crs, voff, (k * U + u) * GB, 0);
        st.c[u][0][0] = v[0]; st.c[u][0][1] = v[1];
      }
    }
    const int soff = row * (NG * 4);
#pragma unroll
    for (int u4 = 0; u4 < U; u4 += 4) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(srs, soff, (k * U + u4) * 4, 0);
#pragma unroll
      for (int q = 0; q < 4 && u4 + q < U; ++q) st.sb[u4 + q][0] = v[q];
    }
  };

  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;

  auto compute = [&](const Stage& st, int s) {
    const int k = s % NSTEP;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = k * U + u;
      f32x16_t d;
#pragma unroll
      for (int v = 0; v < 16; ++v) d[v] = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f16x8_t af = __builtin_bit_cast(f16x8_t, a_lds[s & 1][j * AS + ((u * 8 + 4 * hk + m) ^ (j & ASW))]);
        const uint32_t w = BITS == 4 ? st.c[u][0][m] : st.c[u][0][m >> 1];
        d = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, codes_f16<BITS>(w, m & 1), d, 0, 0, 0);
      }
      const uint32_t p = st.sb[u][0];
      const float sc = bf16_val((uint16_t)(p & 0xFFFFu)), bi = bf16_val((uint16_t)(p >> 16));
      // group sums of this lane's 16 token rows: rows 8a + 4*hk + b for element 4a + b
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 S = *reinterpret_cast<const float4*>(&s_lds[gi * kTileM + 8 * a4 + 4 * hk]);
        acc[4 * a4 + 0] = fmaf(sc, d[4 * a4 + 0], fmaf(bi, S.x, acc[4 * a4 + 0]));
        acc[4 * a4 + 1] = fmaf(sc, d[4 * a4 + 1], fmaf(bi, S.y, acc[4 * a4 + 1]));
        acc[4 * a4 + 2] = fmaf(sc, d[4 * a4 + 2], fmaf(bi, S.z, acc[4 * a4 + 2]));
        acc[4 * a4 + 3] = fmaf(sc, d[4 * a4 + 3], fmaf(bi, S.w, acc[4 * a4 + 3]));
      }
#if BQ_GROUP_SCHED_BARRIER
      // one group at a time: stops the scheduler from widening every group of the step up front,
      // which would cost the registers of a third wave per SIMD
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
  };

  // End of a slab: write its outputs and clear the accumulators. Element v of acc holds token row
  // 8*(v/4) + 4*hk + v%4 and weight row slab*ROWS_B + wrow + j. (Block-uniform; holds barriers.)
  auto finish_slab = [&](int slab) {
    const int row = slab * ROWS_B + wrow + j;
    if constexpr (GATEUP) {
      // the gate waves hand their results to the up waves that hold the same rows
      if (mi == 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) x_lds[wave][v][lane] = acc[v];
      }
      __syncthreads();
      if (mi == 1) {
        const bool active = slab * ROWS_B + wrow < g.nout;  // wave-uniform
        float part[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 8 * (v >> 2) + 4 * hk + (v & 3);
          const float a = x_lds[wave - 2][v][lane], c = acc[v];
          const _Float16 h = (_Float16)(a / (1.0f + expf(-a)) * c);
          if (active && m < count) g.oh[(size_t)orow(m) * g.nout + (row & ~7) + perm8(row & 7)] = h;
          part[v] = active ? (float)h : 0.0f;
        }
        // sum over the 32 rows of this wave (the 32 lanes of each half), then over the two up waves:
        // the slab's 64 rows are one group of the down projection's input
#pragma unroll
        for (int v = 0; v < 16; ++v) {
#pragma unroll
          for (int msk = 16; msk >= 1; msk >>= 1) part[v] += __shfl_xor(part[v], msk, 32);
        }
        if (j == 0) {
#pragma unroll
          for (int v = 0; v < 16; ++v) h_lds[wave - 2][8 * (v >> 2) + 4 * hk + (v & 3)] = part[v];
        }
      }
      __syncthreads();
      const int col0 = slab * ROWS_B;
      if (tid < kTileM && tid < count && col0 < g.nout)
        g.os[(size_t)orow(tid) * (g.nout / 64) + col0 / 64] = h_lds[0][tid] + h_lds[1][tid];
    } else {
      if (row < g.nout) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = 8 * (v >> 2) + 4 * hk + (v & 3);
          if (m < count) g.oy[(size_t)orow(m) * g.nout + row] = acc[v];
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  };

  // STAGES weight stages in a ring: step s computes stage s % STAGES while the next STAGES - 1
  // steps' loads are in flight. The activations of step s+1 are requested before the weights of
  // step s + STAGES - 1, so parking them at the end of step s waits only for loads that step s+1
  // needs anyway. Every load is issued on every path (past the end it re-reads the last step, from
  // cache), so that the compiler's wait counts stay exact and never drain the loads in flight.
  auto body = [&](const Stage& cur, Stage& ahead, int s) {
    load_act(min(s + 1, ntot - 1));
    load_w(ahead, min(s + STAGES - 1, ntot - 1));
    if (s < ntot) {
      compute(cur, s);
      if (s % NSTEP == NSTEP - 1) finish_slab(slab0 + s / NSTEP);
    }
    park_act(s + 1);
    __syncthreads();
  };
  Stage s0, s1;
  load_act(0);
  load_w(s0, 0);
  park_act(0);
  if constexpr (STAGES == 2) {
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s < ntot; s += 2) {
      body(s0, s1, s);
      body(s1, s0, s + 1);
    }
  } else {
    Stage s2;
    load_w(s1, min(1, ntot - 1));
    __syncthreads();
#pragma unroll 1
    for (int s = 0; s < ntot; s += 3) {
      body(s0, s2, s);
      body(s1, s0, s + 1);
      body(s2, s1, s + 2);
    }
  }
}

// ---- 6. combine (gather) / scatter ------------------------------------------------------------------
// out[t][r] = residual[t][r] + sum_k w[t][k] * y[pos[t*K+k]][r] + g[t] * y[T*K + t][r]   (combine)
// y_out[t][k][r] = y[pos[t*K+k]][r], y_out[t][K][r] = y[T*K + t][r]                       (scatter)
__global__ __launch_bounds__(kThreads) void k_prefill_out(int T, int H, int K, int has_shared,
                                                          const int32_t* __restrict__ pos,
                                                          const float* __restrict__ y, const float* __restrict__ w,
                                                          const float* __restrict__ sg,
                                                          const float* __restrict__ residual,
                                                          float* __restrict__ out, float* __restrict__ y_out) {
  const int t = blockIdx.y;
  const int r = blockIdx.x * kThreads + threadIdx.x;
  if (r >= H) return;
  const int NE = K + has_shared;
  if (out != nullptr) {
    float acc = residual[(size_t)t * H + r];
    for (int k = 0; k < K; ++k) acc += w[(size_t)t * K + k] * y[(size_t)pos[(size_t)t * K + k] * H + r];
    if (has_shared) acc += sg[t] * y[((size_t)T * K + t) * H + r];
    out[(size_t)t * H + r] = acc;
  } else {
    for (int k = 0; k < K; ++k) y_out[((size_t)t * NE + k) * H + r] = y[(size_t)pos[(size_t)t * K + k] * H + r];
    if (has_shared) y_out[((size_t)t * NE + K) * H + r] = y[((size_t)T * K + t) * H + r];
  }
}

__global__ void k_copy_i32(int n, const int32_t* __restrict__ src, int32_t* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

constexpr int kStGateUp = BQ_ST_GU;
constexpr int kStDown = BQ_ST_DOWN;
template <int BITS>
constexpr int kULine = BQ_U_LINE * (BITS == 4 ? 4 : 8);

// Blocks: one per tile, times enough slab groups that a launch has about 1024 working blocks when
// tiles are few (the shared expert's 64 tiles at 2048 tokens; small batches). `tiles` is the number
// expected to hold tokens: for the routed experts at most one per routed entry.
unsigned slab_groups(int tiles, int nout, int rows_per_slab) {
  const int nslab = (nout + rows_per_slab - 1) / rows_per_slab;
  return (unsigned)std::max(1, std::min(nslab, 1024 / std::max(1, tiles)));
}

template <int BITS, int KDIM, bool GATEUP>
hipError_t launch_grouped(const GroupArgs& ga, int nout, int T, int N, int E, bool has_shared, hipStream_t s) {
  constexpr int UM = kULine<BITS>;
  constexpr int ST = GATEUP ? kStGateUp : kStDown;
  constexpr int RS = GATEUP ? 64 : 128;  // rows per matrix per slab
  const dim3 block(kThreads);
  const int max_tiles = E + (int)cdiv(N, kTileM);
  hipLaunchKernelGGL((k_grouped<BITS, KDIM, UM, ST, GATEUP, false>),
                     dim3(max_tiles, slab_groups(std::min(max_tiles, N), nout, RS)), block, 0, s, ga);
  if (has_shared) {
    const int st = (int)cdiv(T, kTileM);
    hipLaunchKernelGGL((k_grouped<BITS, KDIM, UM, ST, GATEUP, true>), dim3(st, slab_groups(st, nout, RS)), block, 0,
                       s, ga);
  }
  return hipGetLastError();
}

#define BQ_FOR_KDIM_GU(X) X(256) X(512) X(1024) X(2048) X(4096) X(8192)
#define BQ_FOR_KDIM_DN(X) X(64) X(128) X(256) X(512) X(1024) X(2048)

hipError_t dispatch_gateup(int bits, int H, const GroupArgs& ga, int I, int T, int N, int E, bool hs, hipStream_t s) {
#define BQ_CASE(KV)                                                                   \
  case KV:                                                                            \
    return bits == 4 ? launch_grouped<4, KV, true>(ga, I, T, N, E, hs, s)             \
                     : launch_grouped<2, KV, true>(ga, I, T, N, E, hs, s);
  switch (H) { BQ_FOR_KDIM_GU(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

hipError_t dispatch_down(int bits, int I, const GroupArgs& ga, int H, int T, int N, int E, bool hs, hipStream_t s) {
#define BQ_CASE(KV)                                                                   \
  case KV:                                                                            \
    return bits == 4 ? launch_grouped<4, KV, false>(ga, H, T, N, E, hs, s)            \
                     : launch_grouped<2, KV, false>(ga, H, T, N, E, hs, s);
  switch (I) { BQ_FOR_KDIM_DN(BQ_CASE) }
#undef BQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_router_gemm(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_router_gemm, dim3(cdiv(g.E + g.has_shared, kRRow), cdiv(T, kRTok)), dim3(kThreads), 0, s, T, g.H,
                     g.E, g.has_shared, x, p.router, p.sgate, ws.logits);
  return hipGetLastError();
}

hipError_t launch_router_tokens(const Geometry& g, const LayerPtrs& p, const float* x, int T, const Workspace& ws,
                                hipStream_t s) {
  // the fp64 GEMM fills the chip only for many tokens; below that, per-token router rows win
  if (T >= kRouterGemmMinTokens) return launch_router_gemm(g, p, x, T, ws, s);
  return launch_router_phase(g, p, x, nullptr, nullptr, 0, 0.0f, T, ws, s);
}

hipError_t launch_prefill(const Geometry& g, const LayerPtrs& p, const float* x, const float* residual, int T,
                          const PrefillWorkspace& w, const int32_t* idx_in, int32_t* idx_out, float* out,
                          float* y_out, hipStream_t s) {
  const int H = g.H, I = g.I, E = g.E, K = g.K;
  const int N = T * K;
  const int nchunks = (int)cdiv(N, kChunk);
  hipLaunchKernelGGL(k_prep, dim3(T), dim3(kThreads), 0, s, H, x, reinterpret_cast<_Float16*>(w.xq), w.xs);
  const int32_t* idx = idx_in;
  if (idx_in == nullptr) {
    // the fp64 GEMM fills the chip only for many tokens; below that, per-token router rows win
    hipError_t e = launch_router_tokens(g, p, x, T, w.layer, s);
    if (e == hipSuccess) e = launch_topk(g, T, w.layer, w.layer.idx, w.layer.w, w.layer.g, nullptr, s);
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
  ga.a = reinterpret_cast<const _Float16*>(w.xq); ga.as = w.xs;
  ga.oh = reinterpret_cast<_Float16*>(w.hq); ga.os = w.hs; ga.nout = I;
  hipError_t e = dispatch_gateup(g.bits, H, ga, I, T, N, E, g.has_shared != 0, s);
  if (e != hipSuccess) return e;
  // down
  ga.off_codes[0] = g.off_codes[2]; ga.off_sb[0] = g.off_sb[2];
  ga.a = reinterpret_cast<const _Float16*>(w.hq); ga.as = w.hs;
  ga.oy = w.y; ga.nout = H;
  e = dispatch_down(g.bits, I, ga, H, T, N, E, g.has_shared != 0, s);
  if (e != hipSuccess) return e;
  // combine or scatter
  if (idx_out && idx_in == nullptr)
    hipLaunchKernelGGL(k_copy_i32, dim3(cdiv(N, kThreads)), dim3(kThreads), 0, s, N, w.layer.idx, idx_out);
  hipLaunchKernelGGL(k_prefill_out, dim3(cdiv(H, kThreads), T), dim3(kThreads), 0, s, T, H, K, g.has_shared, w.pos,
                     w.y, w.layer.w, w.layer.g, residual, out, y_out);
  return hipGetLastError();
}

}  // namespace bqmoe
