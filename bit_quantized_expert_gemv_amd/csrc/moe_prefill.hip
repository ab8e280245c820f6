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
// Block: 4 waves, 32 tokens x 32 rows; wave w owns the 16 x 16 output tile (w/2, w%2). Tiles this
// small keep the fp64 MFMA pipes of all SIMDs evenly loaded. Operands are staged in LDS as fp64,
// [k][token or row], rows padded to 48 doubles so that two 16-lane halves never share banks.
typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kRT = 32, kRK = 32, kRP = 48;
__global__ __launch_bounds__(kThreads) void k_router_gemm(int T, int H, int E, int has_shared,
                                                          const float* __restrict__ x,
                                                          const uint16_t* __restrict__ router,
                                                          const uint16_t* __restrict__ sgate,
                                                          double* __restrict__ logits) {
  __shared__ double xs[kRK][kRP];
  __shared__ double rs[kRK][kRP];
  const int t0 = blockIdx.y * kRT, e0 = blockIdx.x * kRT;
  const int nrows = E + has_shared;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, kk = lane >> 4;
  const int ti = wave >> 1, ej = wave & 1;
  // staging: thread -> (row tid/8, k 4*(tid%8) .. +3) of the 32 x 32 tiles
  const int sr = tid >> 3, sk = (tid & 7) * 4;
  const float* xp = x + (size_t)min(t0 + sr, T - 1) * H + sk;
  const int er = min(e0 + sr, nrows - 1);
  const uint16_t* rp = ((er < E) ? router + (size_t)er * H : sgate) + sk;
  float4 xv = *reinterpret_cast<const float4*>(xp);
  uint2 rv = *reinterpret_cast<const uint2*>(rp);
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    xs[sk + 0][sr] = (double)xv.x; xs[sk + 1][sr] = (double)xv.y;
    xs[sk + 2][sr] = (double)xv.z; xs[sk + 3][sr] = (double)xv.w;
    rs[sk + 0][sr] = (double)bf16_val((uint16_t)(rv.x & 0xFFFFu));
    rs[sk + 1][sr] = (double)bf16_val((uint16_t)(rv.x >> 16));
    rs[sk + 2][sr] = (double)bf16_val((uint16_t)(rv.y & 0xFFFFu));
    rs[sk + 3][sr] = (double)bf16_val((uint16_t)(rv.y >> 16));
    __syncthreads();
    if (k0 + kRK < H) {  // next tile in flight during the MFMAs
      xv = *reinterpret_cast<const float4*>(xp + k0 + kRK);
      rv = *reinterpret_cast<const uint2*>(rp + k0 + kRK);
    }
#pragma unroll
    for (int s4 = 0; s4 < kRK / 4; ++s4) {
      const double av = xs[4 * s4 + kk][ti * 16 + c];
      const double bv = rs[4 * s4 + kk][ej * 16 + c];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int e = e0 + ej * 16 + c;
  if (e >= nrows) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = t0 + ti * 16 + kk + 4 * q;
    if (t < T) logits[(size_t)t * (E + 1) + e] = acc[q];
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

// One block: per-expert prefix over chunks (in place), counts, offsets and the tile list
// (tiles of BM entries per expert, in expert order).
__global__ __launch_bounds__(1024) void k_group_scan(int nchunks, int E, int BM, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_first,
                                                     int32_t* __restrict__ ntiles) {
  __shared__ int32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_tiles[MOE_MAX_EXPERTS + 1];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = hist[(size_t)c * E + e];
      hist[(size_t)c * E + e] = run;
      run += v;
    }
    s_cnt[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // E <= 1024: a serial scan is a few microseconds at most
    int off = 0, tiles = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = off;
      s_tiles[e] = tiles;
      off += s_cnt[e];
      tiles += (s_cnt[e] + BM - 1) / BM;
    }
    s_off[E] = off;
    s_tiles[E] = tiles;
    *ntiles = tiles;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const int nt = (s_cnt[e] + BM - 1) / BM;
    for (int j = 0; j < nt; ++j) {
      tile_e[s_tiles[e] + j] = e;
      tile_first[s_tiles[e] + j] = s_off[e] + j * BM;
    }
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

// Block: 4 waves. Wave w owns NT 32-row tiles of each of its NM matrices (NM = 2 for gate/up);
// a block covers 4*NT*32 rows of each matrix for one tile of up to 32 token rows. The tile and
// the row slab come from blockIdx.x so that all slabs of a tile run on one XCD (blocks are dealt
// to the 8 XCDs round robin), where they share the tile's activations in L2.
//
// Pipeline, per step of U groups: the block's activations for the next step are loaded (16 bytes
// per thread and group), then each wave's weights for the next step; then this step is computed
// from registers (weights) and an LDS ring (activations); the next step's activations are parked
// in the ring and one barrier closes the step. Loads retire in order, so the activations are
// requested before the weights: waiting for them never waits for the weights in flight.
template <int BITS, int KDIM, int NT, int UMAX, bool GATEUP, bool SHARED>
__global__ __launch_bounds__(kThreads) void k_grouped(GroupArgs g) {
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int NTILE = NM * NT;
  constexpr int NG = KDIM / 64;
  constexpr int U = NG >= UMAX ? UMAX : NG;  // groups per pipeline step
  constexpr int NSTEP = NG / U;
  constexpr int ROWB = KDIM * BITS / 8;
  constexpr int GB = 64 * BITS / 8;  // code bytes per row and group
  constexpr int LB = GB / 2;         // per lane half
  constexpr int ROWS_W = NT * 32;
  constexpr int ROWS_B = 4 * ROWS_W;
  constexpr int AS = U * 8;          // 16-byte activation slots per row and step
  constexpr int ASW = AS >= 16 ? 15 : AS - 1;  // slot swizzle: 16 consecutive rows hit distinct banks
  using Stage = GStage<BITS, NTILE, U>;
  static_assert(!GATEUP || 64 % ROWS_W == 0, "a 64-row group of the SwiGLU output spans whole waves");
  __shared__ float s_lds[NG * kTileM];                  // group sums of the tile's activations, [group][row]
  __shared__ float h_lds[GATEUP ? 4 : 1][kTileM];        // gate/up: per-wave sums of the fp16 SwiGLU outputs
  __shared__ u32x4_t a_lds[2][kTileM * AS];             // activation ring: [step parity][row][slot ^ swizzle]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, hk = lane >> 5;
  const int nslab = (g.nout + ROWS_B - 1) / ROWS_B;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int tau = xcd + 8 * (q / nslab), slab = q % nslab;
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
  auto load_act = [&](int step) {
#pragma unroll
    for (int u = 0; u < U; ++u) a_reg[u] = a_src[(step * U + u) * 8];
  };
  auto park_act = [&](int /*loaded step*/, int slot_step) {
#pragma unroll
    for (int u = 0; u < U; ++u) a_lds[slot_step & 1][a_row * AS + ((u * 8 + a_slot) ^ (a_row & ASW))] = a_reg[u];
  };

  const int r0w = slab * ROWS_B + wave * ROWS_W;  // first row (per matrix) of this wave
  const bool active = r0w < g.nout;               // wave-uniform; idle waves still join the barriers
  const uint8_t* cp[NTILE];
  const uint32_t* sp[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int mi = t / NT, nt = t % NT;
    const int row = min(r0w + nt * 32 + j, g.nout - 1);
    cp[t] = blob + g.off_codes[mi] + (size_t)row * ROWB + hk * LB;
    sp[t] = reinterpret_cast<const uint32_t*>(blob + g.off_sb[mi]) + (size_t)row * NG;
  }
  // unconditional (idle waves read a clamped row): a load skipped on some path would make the
  // compiler's wait counts conservative and drain the prefetch at every barrier
  auto load_w = [&](Stage& st, int step) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = step * U + u;
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        if constexpr (BITS == 4) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(cp[t] + gi * GB);
          st.c[u][t][0] = v[0]; st.c[u][t][1] = v[1]; st.c[u][t][2] = v[2]; st.c[u][t][3] = v[3];
        } else {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(cp[t] + gi * GB);
          st.c[u][t][0] = v[0]; st.c[u][t][1] = v[1];
        }
        st.sb[u][t] = sp[t][gi];
      }
    }
  };

  f32x16_t acc[NTILE];
#pragma unroll
  for (int t = 0; t < NTILE; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

  auto compute = [&](const Stage& st, int step) {
    if (!active) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gi = step * U + u;
      // group sums of this lane's 16 token rows: rows 8a + 4*hk + b for element 4a + b
      float S[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const float4 v = *reinterpret_cast<const float4*>(&s_lds[gi * kTileM + 8 * a4 + 4 * hk]);
        S[4 * a4 + 0] = v.x; S[4 * a4 + 1] = v.y; S[4 * a4 + 2] = v.z; S[4 * a4 + 3] = v.w;
      }
      f16x8_t af[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        af[m] = __builtin_bit_cast(f16x8_t, a_lds[step & 1][j * AS + ((u * 8 + 4 * hk + m) ^ (j & ASW))]);
#pragma unroll
      for (int t = 0; t < NTILE; ++t) {
        f32x16_t d;
#pragma unroll
        for (int v = 0; v < 16; ++v) d[v] = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t w = BITS == 4 ? st.c[u][t][m] : st.c[u][t][m >> 1];
          d = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[m], codes_f16<BITS>(w, m & 1), d, 0, 0, 0);
        }
        const uint32_t p = st.sb[u][t];
        const float sc = bf16_val((uint16_t)(p & 0xFFFFu)), bi = bf16_val((uint16_t)(p >> 16));
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = fmaf(sc, d[v], fmaf(bi, S[v], acc[t][v]));
      }
    }
  };

  // Two weight stages in ping-pong: one is in flight while the other is computed. Every load is
  // issued on every path (past the end it re-reads the last step, from cache), so that the
  // compiler's wait counts stay exact and never drain the loads in flight. (A third stage costs
  // the second wave per SIMD and measured slower.)
  Stage s0, s1;
  load_act(0);
  load_w(s0, 0);
  park_act(0, 0);
  __syncthreads();
#pragma unroll 1
  for (int step = 0; step < NSTEP; step += 2) {
    const int n1 = min(step + 1, NSTEP - 1), n2 = min(step + 2, NSTEP - 1);
    load_act(n1);
    load_w(s1, n1);
    compute(s0, step);
    park_act(n1, step + 1);
    __syncthreads();
    load_act(n2);
    load_w(s0, n2);
    if (step + 1 < NSTEP) compute(s1, step + 1);
    park_act(n2, step + 2);
    __syncthreads();
  }

  // element v of a tile holds token row 8*(v/4) + 4*hk + v%4 and weight row r0w + 32*nt + j
  if constexpr (GATEUP) {
    float part[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * hk + (v & 3);
      float sum = 0.0f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float a = acc[nt][v], c = acc[NT + nt][v];
        const _Float16 h = (_Float16)(a / (1.0f + expf(-a)) * c);
        sum += (float)h;
        const int col = r0w + 32 * nt + j;
        if (active && m < count) g.oh[(size_t)orow(m) * g.nout + (col & ~7) + perm8(col & 7)] = h;
      }
      part[v] = active ? sum : 0.0f;
    }
    // sum over the 32 lanes of each half, then over the waves that share a 64-column group (the
    // group sums of the down projection's input)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
#pragma unroll
      for (int msk = 16; msk >= 1; msk >>= 1) part[v] += __shfl_xor(part[v], msk, 32);
    }
    if (j == 0) {
#pragma unroll
      for (int v = 0; v < 16; ++v) h_lds[wave][8 * (v >> 2) + 4 * hk + (v & 3)] = part[v];
    }
    __syncthreads();
    constexpr int WPG = 64 / ROWS_W;  // waves per group
    for (int i = tid; i < (4 / WPG) * kTileM; i += kThreads) {
      const int m = i % kTileM, gl = i / kTileM;
      const int col0 = slab * ROWS_B + gl * 64;
      if (m >= count || col0 >= g.nout) continue;
      float v = 0.0f;
      for (int w = 0; w < WPG; ++w) v += h_lds[gl * WPG + w][m];
      g.os[(size_t)orow(m) * (g.nout / 64) + col0 / 64] = v;
    }
  } else {
    if (!active) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = r0w + 32 * nt + j;
      if (col >= g.nout) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * hk + (v & 3);
        if (m < count) g.oy[(size_t)orow(m) * g.nout + col] = acc[nt][v];
      }
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

#ifndef BQ_NT_GU
#define BQ_NT_GU 1
#endif
#ifndef BQ_NT_DOWN
#define BQ_NT_DOWN 1
#endif
#ifndef BQ_U_LINE
#define BQ_U_LINE 1
#endif
// 32-row tiles per matrix per wave, and groups per pipeline step: by default a step takes one
// 128-byte line of every row (4 groups at 4-bit, 8 at 2-bit), so that no line is fetched twice.
constexpr int kNTGateUp = BQ_NT_GU;
constexpr int kNTDown = BQ_NT_DOWN;
template <int BITS>
constexpr int kULine = BQ_U_LINE * (BITS == 4 ? 4 : 8);

// Blocks for `tiles` tiles of `nout` rows: slabs of 4*NT*32 rows, tiles padded to a multiple of 8.
unsigned grouped_blocks(int tiles, int nout, int nt) {
  const int nslab = (int)cdiv(nout, 4 * nt * 32);
  return (unsigned)(8 * nslab) * cdiv(tiles, 8);
}

template <int BITS, int KDIM, bool GATEUP>
hipError_t launch_grouped(const GroupArgs& ga, int nout, int T, int N, int E, bool has_shared, hipStream_t s) {
  constexpr int NT = GATEUP ? kNTGateUp : kNTDown;
  constexpr int UM = kULine<BITS>;
  const dim3 block(kThreads);
  const int max_tiles = E + (int)cdiv(N, kTileM);
  hipLaunchKernelGGL((k_grouped<BITS, KDIM, NT, UM, GATEUP, false>), dim3(grouped_blocks(max_tiles, nout, NT)), block,
                     0, s, ga);
  if (has_shared)
    hipLaunchKernelGGL((k_grouped<BITS, KDIM, NT, UM, GATEUP, true>),
                       dim3(grouped_blocks((int)cdiv(T, kTileM), nout, NT)), block, 0, s, ga);
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
  hipLaunchKernelGGL(k_router_gemm, dim3(cdiv(g.E + g.has_shared, kRT), cdiv(T, kRT)), dim3(kThreads), 0, s, T, g.H,
                     g.E, g.has_shared, x, p.router, p.sgate, ws.logits);
  return hipGetLastError();
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
    hipError_t e = launch_router_gemm(g, p, x, T, w.layer, s);
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
