// GPU fill kernels for the seeded synthetic-input generator (definitions in gen.h).
//
// Writes canonical arrays (one byte per code; bf16 scales and biases) straight into device
// memory, so that weight pools too large to generate on the host can be made in place. Every
// value equals the host generator's bit for bit: codes are integer operations only, and the
// uniform draws use one correctly rounded double operation per step (__dsub_rn, __dmul_rn,
// __dadd_rn), which is what gen.c computes with contraction switched off.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGolden); }

__device__ __forceinline__ uint16_t bf16_rne(double v) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t lsb = (b >> 45) & 1u;
  b += ((1ULL << 44) - 1u) + lsb;
  b &= ~((1ULL << 45) - 1u);
  const float f = __double2float_rn(__longlong_as_double((long long)b));  // exact: <= 8 significant bits
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// One thread per 64-bit draw; the draw holds 64/bits consecutive codes.
template <int BITS>
__global__ void fill_codes_kernel(uint64_t key, int64_t nwords, int64_t n, uint8_t* __restrict__ out) {
  constexpr int kPer = 64 / BITS;
  constexpr uint64_t kMask = (1ULL << BITS) - 1u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords; w += stride) {
    const uint64_t x = draw(key, (uint64_t)w);
    const int64_t e0 = w * kPer;
    if (e0 + kPer <= n) {
      // full word: kPer bytes, stored as 16-byte vectors (out is 16-byte aligned, e0 % 16 == 0)
      uint32_t word[kPer / 4];
#pragma unroll
      for (int k = 0; k < kPer / 4; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) v |= (uint32_t)((x >> (BITS * (4 * k + j))) & kMask) << (8 * j);
        word[k] = v;
      }
#pragma unroll
      for (int k = 0; k < kPer / 16; ++k) {
        uint4 q;
        q.x = word[4 * k + 0]; q.y = word[4 * k + 1]; q.z = word[4 * k + 2]; q.w = word[4 * k + 3];
        *reinterpret_cast<uint4*>(out + e0 + 16 * k) = q;
      }
    } else {
      for (int f = 0; f < kPer && e0 + f < n; ++f) out[e0 + f] = (uint8_t)((x >> (BITS * f)) & kMask);
    }
  }
}

__global__ void fill_uniform_bf16_kernel(uint64_t key, double lo, double hi, int64_t n, uint16_t* __restrict__ out) {
  const double d = __dsub_rn(hi, lo);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < n; m += stride) {
    const double t = (double)(draw(key, (uint64_t)m) >> 11) * 0x1p-53;  // exact
    const double v = __dadd_rn(lo, __dmul_rn(d, t));
    out[m] = bf16_rne(v);
  }
}

__global__ void fill_ints_u16_kernel(uint64_t key, int lo, uint64_t span, int64_t n, uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; m < n; m += stride)
    out[m] = (uint16_t)(lo + (int)(draw(key, (uint64_t)m) % span));
}

int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" {

// Codes [0, n) of the stream `key`, one byte per code, into device memory `out` (16-byte aligned).
// Returns 0, -1 for bad arguments, or a positive hipError_t from the launch.
int bqgen_fill_codes(uint64_t key, int bits, int64_t n, void* out, void* stream) {
  if (out == nullptr || n < 0 || (bits != 2 && bits != 4) || (reinterpret_cast<uintptr_t>(out) & 15u)) return -1;
  if (n == 0) return 0;
  const int per = 64 / bits;
  const int64_t nwords = (n + per - 1) / per;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (bits == 4)
    fill_codes_kernel<4><<<grid_for(nwords), 256, 0, s>>>(key, nwords, n, static_cast<uint8_t*>(out));
  else
    fill_codes_kernel<2><<<grid_for(nwords), 256, 0, s>>>(key, nwords, n, static_cast<uint8_t*>(out));
  return (int)hipGetLastError();
}

// Uniform draws [0, n) in [lo, hi], rounded to bf16, into device memory `out`.
int bqgen_fill_uniform_bf16(uint64_t key, double lo, double hi, int64_t n, void* out, void* stream) {
  if (out == nullptr || n < 0 || (reinterpret_cast<uintptr_t>(out) & 1u)) return -1;
  if (n == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fill_uniform_bf16_kernel<<<grid_for(n), 256, 0, s>>>(key, lo, hi, n, static_cast<uint16_t*>(out));
  return (int)hipGetLastError();
}

// Integers [0, n) in [lo, hi] (0 <= lo <= hi <= 65535), one uint16 each, into device memory `out`.
int bqgen_fill_ints_u16(uint64_t key, int lo, int hi, int64_t n, void* out, void* stream) {
  if (out == nullptr || n < 0 || lo < 0 || hi < lo || hi > 65535 || (reinterpret_cast<uintptr_t>(out) & 1u)) return -1;
  if (n == 0) return 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fill_ints_u16_kernel<<<grid_for(n), 256, 0, s>>>(key, lo, (uint64_t)(hi - lo) + 1u, n, static_cast<uint16_t*>(out));
  return (int)hipGetLastError();
}

}  // extern "C"
