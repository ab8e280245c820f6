// Prefill path of the quantised MoE layer for MI355X (gfx950): many tokens through one layer,
// grouped by expert so that each expert's weights are streamed once per tile of tokens.
//
//   1. prep: every activation is split into bf16 hi + lo (x ~ hi + lo to ~2^-18 relative), and
//      per-64-group sums of hi + lo are taken;
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
// Exactness of the weights. A dequantised weight is s*q + b ("Kernel de dequantización optimizado
// con FMA"), which needs up to 15 significant bits, so rounding weights to bf16 would lose
// accuracy. The MFMA operands are instead the raw codes, which are exact in bf16 as 128 + q (the
// bit pattern 0x4300 | q, made with byte permutes), times the hi and lo activation parts. Per
// 64-wide group the fp32 result D = sum (128 + q) x is scaled in the epilogue:
//   s * D + (b - 128 s) * S,   S = sum x   (hi + lo).
// The 128 offset cancels exactly against the bias term.
//
// MFMA: v_mfma_f32_16x16x32_bf16. A[i][k] sits in lane i + 16*(k/8), element k%8; B[k][j] in lane
// j + 16*(k/8), element k%8; D[i][j] in lane j + 16*(i/4), element i%4 (checked on the device).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "moe_internal.h"

namespace bqmoe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t bf16_rne_bits(float v) {
  uint32_t b = __float_as_uint(v);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Split v into bf16 hi + lo; returns hi + lo as float (what the MFMA sees).
__device__ __forceinline__ float split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = bf16_rne_bits(v);
  const float r = v - bf16_val(hi);
  lo = bf16_rne_bits(r);
  return bf16_val(hi) + bf16_val(lo);
}

// ---- 1. activation prep -------------------------------------------------------------------------
// One block per token: hi/lo bf16 copies and per-64-group sums of hi + lo.
__global__ __launch_bounds__(kThreads) void k_prep(int H, const float* __restrict__ x, uint16_t* __restrict__ xh,
                                                   uint16_t* __restrict__ xl, float* __restrict__ xs) {
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * H;
  // each wave takes whole groups: lane l of a group sums with its neighbours by shuffles
  const int ng = H / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int gi = wave; gi < ng; gi += kThreads / 64) {
    const int j = gi * 64 + lane;
    uint16_t hi, lo;
    float v = split_bf16(xr[j], hi, lo);
    xh[(size_t)t * H + j] = hi;
    xl[(size_t)t * H + j] = lo;
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    if (lane == 0) xs[(size_t)t * ng + gi] = v;
  }
}

// ---- 2. router GEMM (fp64) ------------------------------------------------------------------------
// logits[t][e] = sum_j R[e][j] x[t][j] for e < E, and the shared-gate vector as row E.
// Block tile 64 tokens x 64 rows, k step 32; each thread owns 4 x 4 outputs. Tiles sit in LDS as
// fp64, transposed, so every read is a broadcast or a conflict-free 32-byte run.
constexpr int kRT = 64, kRK = 32;
__global__ __launch_bounds__(kThreads) void k_router_gemm(int T, int H, int E, int has_shared,
                                                          const float* __restrict__ x,
                                                          const uint16_t* __restrict__ router,
                                                          const uint16_t* __restrict__ sgate,
                                                          double* __restrict__ logits) {
  __shared__ double xs[kRK][kRT];
  __shared__ double rs[kRK][kRT];
  const int t0 = blockIdx.y * kRT, e0 = blockIdx.x * kRT;
  const int nrows = E + has_shared;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += kRK) {
    // cooperative loads: 64 x 32 of each (2048 elements, 8 per thread)
    for (int i = threadIdx.x; i < kRT * kRK; i += kThreads) {
      const int r = i / kRK, c = i % kRK;
      const int t = min(t0 + r, T - 1);
      xs[c][r] = (double)x[(size_t)t * H + k0 + c];
      const int e = min(e0 + r, nrows - 1);
      const uint16_t* row = (e < E) ? router + (size_t)e * H : sgate;
      rs[c][r] = (double)bf16_val(row[k0 + c]);
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kRK; ++c) {
      double a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = xs[c][ty * 4 + i]; b[i] = rs[c][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < nrows) logits[(size_t)t * (E + 1) + e] = acc[i][j];
    }
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
  const uint16_t* ah;                // activations, bf16 hi [rows][KDIM]
  const uint16_t* al;                // bf16 lo
  const float* as;                   // group sums of hi + lo [rows][KDIM/64]
  const int32_t* perm;               // routed: position -> entry (t*K + k)
  int K;
  const int32_t* tile_e;
  const int32_t* tile_first;
  const int32_t* ntiles;
  const int32_t* offsets;
  int shared_base;  // output row of the shared expert's token 0 (= T*K)
  int T;
  uint16_t* oh;  // gate/up: SwiGLU output hi/lo [rows][nout], group sums [rows][nout/64]
  uint16_t* ol;
  float* os;
  float* oy;  // down: [rows][nout]
  int nout;
};

// 8 codes -> 8 bf16 values (128 + q) for one MFMA operand.
template <int BITS>
__device__ __forceinline__ bf16x8_t codes_to_bf16(const uint8_t* __restrict__ p) {
  u32x4_t d;
  if constexpr (BITS == 4) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);   // element e at bits 4e..4e+3
    const uint32_t u = w & 0x0F0F0F0Fu;                          // bytes: elements 0, 2, 4, 6
    const uint32_t v = (w >> 4) & 0x0F0F0F0Fu;                   // bytes: elements 1, 3, 5, 7
    // dword j = [u.byte j, 0, v.byte j, 0] | 0x43004300 (v_perm_b32: selectors 0-3 pick u, 4-7 pick v, 12 = 0)
    d[0] = __builtin_amdgcn_perm(v, u, 0x0C040C00u) | 0x43004300u;
    d[1] = __builtin_amdgcn_perm(v, u, 0x0C050C01u) | 0x43004300u;
    d[2] = __builtin_amdgcn_perm(v, u, 0x0C060C02u) | 0x43004300u;
    d[3] = __builtin_amdgcn_perm(v, u, 0x0C070C03u) | 0x43004300u;
  } else {
    const uint32_t w = *reinterpret_cast<const uint16_t*>(p);   // element e at bits 2e..2e+1
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t nib = (w >> (4 * j)) & 0xFu;
      d[j] = 0x43004300u | (nib & 3u) | ((nib >> 2) << 16);
    }
  }
  return __builtin_bit_cast(bf16x8_t, d);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* __restrict__ p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// Block: 4 waves x 16 weight rows (per matrix) = 64 rows, BM = 16*MT token rows.
template <int BITS, int KDIM, int MT, bool GATEUP, bool SHARED>
__global__ __launch_bounds__(kThreads) void k_grouped(GroupArgs g) {
  constexpr int BM = 16 * MT;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int NG = KDIM / 64;
  constexpr int ROWB = KDIM * BITS / 8;
  __shared__ float ssum[4][BM];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lm = lane & 15, lq = lane >> 4;
  int first, count;
  const uint8_t* blob;
  if constexpr (SHARED) {
    first = blockIdx.y * BM;
    count = min(BM, g.T - first);
    blob = g.shared;
  } else {
    const int tau = blockIdx.y;
    if (tau >= *g.ntiles) return;  // uniform per block
    const int e = g.tile_e[tau];
    first = g.tile_first[tau];
    count = min(BM, g.offsets[e + 1] - first);
    blob = g.experts + (size_t)e * g.stride;
  }
  // activation row of token slot m (clamped into the tile)
  auto arow = [&](int m) -> int {
    const int mm = first + min(m, count - 1);
    if constexpr (SHARED) return GATEUP ? mm : g.shared_base + mm;
    else return GATEUP ? g.perm[mm] / g.K : mm;
  };
  auto orow = [&](int m) -> int {
    const int mm = first + m;
    if constexpr (SHARED) return g.shared_base + mm;
    else return mm;
  };
  int ar[MT], sr[MT][4];
#pragma unroll
  for (int st = 0; st < MT; ++st) {
    ar[st] = arow(st * 16 + lm);
#pragma unroll
    for (int e = 0; e < 4; ++e) sr[st][e] = arow(st * 16 + 4 * lq + e);
  }
  const int n = blockIdx.x * 64 + wave * 16 + lm;  // weight row of this lane's B column (and D column)
  f32x4_t acc[MT][NM];
#pragma unroll
  for (int st = 0; st < MT; ++st)
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) acc[st][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int gi = 0; gi < NG; ++gi) {
    bf16x8_t bq[NM][2];
    float sc[NM], bb[NM];
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      const uint8_t* row = blob + g.off_codes[mi] + (size_t)n * ROWB;
#pragma unroll
      for (int h = 0; h < 2; ++h) bq[mi][h] = codes_to_bf16<BITS>(row + ((gi * 64 + 32 * h + 8 * lq) * BITS) / 8);
      const uint32_t p = *reinterpret_cast<const uint32_t*>(blob + g.off_sb[mi] + ((size_t)n * NG + gi) * 4);
      sc[mi] = __uint_as_float(p << 16);
      bb[mi] = __uint_as_float(p & 0xFFFF0000u) - 128.0f * sc[mi];
    }
#pragma unroll
    for (int st = 0; st < MT; ++st) {
      const uint16_t* ph = g.ah + (size_t)ar[st] * KDIM + gi * 64 + 8 * lq;
      const uint16_t* pl = g.al + (size_t)ar[st] * KDIM + gi * 64 + 8 * lq;
      const bf16x8_t xh0 = load_bf16x8(ph), xh1 = load_bf16x8(ph + 32);
      const bf16x8_t xl0 = load_bf16x8(pl), xl1 = load_bf16x8(pl + 32);
      float S[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) S[e] = g.as[(size_t)sr[st][e] * NG + gi];
#pragma unroll
      for (int mi = 0; mi < NM; ++mi) {
        f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh0, bq[mi][0], zero, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl0, bq[mi][0], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh1, bq[mi][1], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl1, bq[mi][1], d, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[st][mi][e] = fmaf(sc[mi], d[e], fmaf(bb[mi], S[e], acc[st][mi][e]));
      }
    }
  }
  if constexpr (GATEUP) {
    // SwiGLU, split to bf16 hi/lo for the down GEMM, and per-row sums over this block's 64 columns
    // (one input group of the down projection).
#pragma unroll
    for (int st = 0; st < MT; ++st) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = st * 16 + 4 * lq + e;
        const float a = acc[st][0][e], c = acc[st][1][e];
        const float hv = a / (1.0f + expf(-a)) * c;
        uint16_t hi, lo;
        float seen = split_bf16(hv, hi, lo);
        if (m < count) {
          const size_t o = (size_t)orow(m) * g.nout + n;
          g.oh[o] = hi;
          g.ol[o] = lo;
        } else {
          seen = 0.0f;
        }
        // sum over the 16 columns of this wave: lanes 16*lq .. 16*lq+15 (one DPP row)
        for (int msk = 8; msk >= 1; msk >>= 1) seen += __shfl_xor(seen, msk, 16);
        if (lm == 0) ssum[wave][m] = seen;
      }
    }
    __syncthreads();
    for (int m = threadIdx.x; m < count; m += kThreads)
      g.os[(size_t)orow(m) * (g.nout / 64) + blockIdx.x] = (ssum[0][m] + ssum[1][m]) + (ssum[2][m] + ssum[3][m]);
  } else {
#pragma unroll
    for (int st = 0; st < MT; ++st)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = st * 16 + 4 * lq + e;
        if (m < count) g.oy[(size_t)orow(m) * g.nout + n] = acc[st][0][e];
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

constexpr int kMTRouted = 2;  // 32 tokens per routed tile (an expert sees about 12 on average)
constexpr int kMTShared = 4;  // 64 tokens per shared-expert tile

unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }

template <int BITS, int KDIM, bool GATEUP>
hipError_t launch_grouped(const GroupArgs& ga, int nout, int T, int N, int E, bool has_shared, hipStream_t s) {
  const dim3 block(kThreads);
  const unsigned nx = (unsigned)(nout / 64);
  const int max_tiles = E + (int)cdiv(N, 16 * kMTRouted);
  hipLaunchKernelGGL((k_grouped<BITS, KDIM, kMTRouted, GATEUP, false>), dim3(nx, max_tiles), block, 0, s, ga);
  if (has_shared)
    hipLaunchKernelGGL((k_grouped<BITS, KDIM, kMTShared, GATEUP, true>), dim3(nx, cdiv(T, 16 * kMTShared)), block, 0,
                       s, ga);
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
  hipLaunchKernelGGL(k_prep, dim3(T), dim3(kThreads), 0, s, H, x, w.xh, w.xl, w.xs);
  const int32_t* idx = idx_in;
  if (idx_in == nullptr) {
    hipError_t e = launch_router_gemm(g, p, x, T, w.layer, s);
    if (e == hipSuccess) e = launch_topk(g, T, w.layer, w.layer.idx, w.layer.w, w.layer.g, nullptr, s);
    if (e != hipSuccess) return e;
    idx = w.layer.idx;
  }
  hipLaunchKernelGGL(k_group_hist, dim3(nchunks), dim3(kChunk), E * sizeof(int32_t), s, N, E, idx, w.hist);
  hipLaunchKernelGGL(k_group_scan, dim3(1), dim3(1024), 0, s, nchunks, E, 16 * kMTRouted, w.hist, w.counts,
                     w.offsets, w.tile_e, w.tile_first, w.ntiles);
  hipLaunchKernelGGL(k_group_place, dim3(nchunks), dim3(kChunk), 0, s, N, E, idx, w.hist, w.offsets, w.pos, w.perm);
  GroupArgs ga{};
  ga.experts = p.experts; ga.stride = p.stride; ga.shared = p.shared;
  ga.perm = w.perm; ga.K = K; ga.tile_e = w.tile_e; ga.tile_first = w.tile_first; ga.ntiles = w.ntiles;
  ga.offsets = w.offsets; ga.shared_base = N; ga.T = T;
  // gate/up + SwiGLU
  ga.off_codes[0] = g.off_codes[0]; ga.off_codes[1] = g.off_codes[1];
  ga.off_sb[0] = g.off_sb[0]; ga.off_sb[1] = g.off_sb[1];
  ga.ah = w.xh; ga.al = w.xl; ga.as = w.xs;
  ga.oh = w.hh; ga.ol = w.hl; ga.os = w.hs; ga.nout = I;
  hipError_t e = dispatch_gateup(g.bits, H, ga, I, T, N, E, g.has_shared != 0, s);
  if (e != hipSuccess) return e;
  // down
  ga.off_codes[0] = g.off_codes[2]; ga.off_sb[0] = g.off_sb[2];
  ga.ah = w.hh; ga.al = w.hl; ga.as = w.hs;
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
