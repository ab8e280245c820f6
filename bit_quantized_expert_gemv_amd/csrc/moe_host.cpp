// Host side of the C ABI declared in include/moe.h: argument validation (before any HIP call),
// workspace layout, the host packer, and the per-call kernel sequences.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "moe.h"
#include "moe_internal.h"

namespace bqmoe {
namespace {

thread_local std::string g_last_error;

int fail(int code, const char* why) {
  g_last_error = why ? why : "";
  return code;
}

int ok() {
  g_last_error.clear();
  return MOE_OK;
}

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  static thread_local char buf[160];
  snprintf(buf, sizeof(buf), "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return fail(MOE_EHIP, buf);
}

// Validates the descriptor for the kernels; returns MOE_OK or an error code with g_last_error set.
int check_layer(const moe_layer_t* L, Geometry* g) {
  if (L == nullptr) return fail(MOE_EINVAL, "layer is NULL");
  const char* why = nullptr;
  if (!geometry_from(L, g, &why)) return fail(MOE_EUNSUPPORTED, why);
  if (L->experts_dev == nullptr) return fail(MOE_EINVAL, "experts_dev is NULL");
  if (!aligned(L->experts_dev, 256)) return fail(MOE_EINVAL, "experts_dev must be 256-byte aligned");
  if (L->expert_stride < g->blob_bytes || (L->expert_stride & 255u) != 0)
    return fail(MOE_EINVAL, "expert_stride must be >= moe_blob_bytes() and a multiple of 256");
  if (L->router_dev == nullptr || !aligned(L->router_dev, 16))
    return fail(MOE_EINVAL, "router_dev must be non-NULL and 16-byte aligned");
  if (L->has_shared) {
    if (L->shared_blob_dev == nullptr || !aligned(L->shared_blob_dev, 256))
      return fail(MOE_EINVAL, "shared_blob_dev must be non-NULL and 256-byte aligned when has_shared");
    if (L->shared_gate_dev == nullptr || !aligned(L->shared_gate_dev, 16))
      return fail(MOE_EINVAL, "shared_gate_dev must be non-NULL and 16-byte aligned when has_shared");
  }
  return MOE_OK;
}

LayerPtrs ptrs_of(const moe_layer_t* L) {
  LayerPtrs p;
  p.experts = static_cast<const uint8_t*>(L->experts_dev);
  p.stride = L->expert_stride;
  p.shared = static_cast<const uint8_t*>(L->shared_blob_dev);
  p.router = L->router_dev;
  p.sgate = L->shared_gate_dev;
  return p;
}

int check_act(const void* p, const char* name) {
  static thread_local char buf[96];
  if (p == nullptr || !aligned(p, 16)) {
    snprintf(buf, sizeof(buf), "%s must be non-NULL and 16-byte aligned", name);
    return fail(MOE_EINVAL, buf);
  }
  return MOE_OK;
}

}  // namespace

bool geometry_from(const moe_layer_t* L, Geometry* g, const char** why) {
  if (L->bits != 2 && L->bits != 4) { *why = "bits must be 2 or 4"; return false; }
  if (L->group != 64 && !(L->group == 32 && L->bits == 4)) {
    *why = "group must be 64 (affine), or 32 with bits 4 (MXFP4)";
    return false;
  }
  const bool mx = L->group == 32;
  if (!pow2_in(L->hidden, 256, 8192)) { *why = "hidden must be a power of two in [256, 8192]"; return false; }
  if (!pow2_in(L->inter, 64, 2048)) { *why = "inter must be a power of two in [64, 2048]"; return false; }
  if (L->n_experts < 1 || L->n_experts > MOE_MAX_EXPERTS) { *why = "n_experts must be in [1, 1024]"; return false; }
  if (L->top_k < 1 || L->top_k > MOE_MAX_TOP_K || L->top_k > L->n_experts) {
    *why = "top_k must be in [1, min(n_experts, 8)]";
    return false;
  }
  if (L->has_shared != 0 && L->has_shared != 1) { *why = "has_shared must be 0 or 1"; return false; }
  const int form = L->flags & ~MOE_FLAG_DECODE_CHAIN;
  if (form != 0 && form != MOE_FLAG_DEQUANT_LITERAL && form != MOE_FLAG_DEQUANT_NAIVE) {
    *why = "flags must be 0, MOE_FLAG_DEQUANT_LITERAL or MOE_FLAG_DEQUANT_NAIVE, optionally with MOE_FLAG_DECODE_CHAIN";
    return false;
  }
  g->chain = (L->flags & MOE_FLAG_DECODE_CHAIN) != 0;
  if (mx && form != 0) { *why = "the dequant-form flags apply to the affine format only"; return false; }
  g->form = mx ? 3 : form == MOE_FLAG_DEQUANT_LITERAL ? 1 : form == MOE_FLAG_DEQUANT_NAIVE ? 2 : 0;
  g->H = L->hidden; g->I = L->inter; g->E = L->n_experts; g->K = L->top_k;
  g->has_shared = L->has_shared; g->NE = g->K + g->has_shared;
  g->bits = L->bits; g->G = L->group;
  const uint64_t cb = (uint64_t)g->I * g->H * g->bits / 8;
  const uint64_t sbb = (uint64_t)g->I * (g->H / g->G) * (mx ? 1 : 4);  // (scale, bias) words or E8M0 bytes
  for (int m = 0; m < 3; ++m) {
    g->off_codes[m] = m * cb;
    g->off_sb[m] = 3 * cb + m * sbb;
  }
  g->blob_bytes = 3 * cb + 3 * sbb;
  return true;
}

size_t workspace_layer_bytes(const Geometry& g, int T) {
  const size_t t = (size_t)T;
  return MOE_WS_SYNC_BYTES + align256(t * (g.E + 1) * 8) + align256(t * g.K * 4) + align256(t * g.K * 4) + align256(t * 4) +
         align256(t * g.NE * g.I * 4) + align256(t * g.H * 4) + align256((size_t)g.E * 8);
}

namespace {
struct Carver {
  uint8_t* p;
  size_t used = 0;
  template <class T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(p == nullptr ? nullptr : p + used);
    used += align256(count * sizeof(T));
    return r;
  }
};

PrefillWorkspace carve_prefill_impl(const Geometry& g, int T, void* base, size_t* total) {
  Carver c{static_cast<uint8_t*>(base)};
  c.take<uint8_t>(MOE_WS_SYNC_BYTES);  // the sync region, which only the single-launch decode uses
  const size_t t = (size_t)T, N = t * g.K, R = N + t * g.has_shared;
  PrefillWorkspace w;
  w.layer.logits = c.take<double>(t * (g.E + 1));
  w.layer.idx = c.take<int32_t>(N);
  w.layer.w = c.take<float>(N);
  w.layer.g = c.take<float>(t);
  w.layer.h = nullptr;
  w.layer.u = nullptr;
  w.layer.rnorm = c.take<double>(g.E);
  const bool mx = g.form == 3;
  w.xq = mx ? nullptr : c.take<uint16_t>(t * g.H);
  w.xs = mx ? nullptr : c.take<float>(t * (g.H / 64));
  w.xu = mx ? nullptr : c.take<float>(t);
  w.x8 = mx ? c.take<uint8_t>(3 * t * g.H) : nullptr;
  w.xsc = mx ? c.take<uint8_t>(3 * t * (g.H / 32)) : nullptr;
  w.hist = c.take<int32_t>(((N + 255) / 256) * g.E);
  w.counts = c.take<int32_t>(g.E);
  w.offsets = c.take<int32_t>(g.E + 1);
  w.tile_e = c.take<int32_t>(g.E + (N + 31) / 32);
  w.tile_first = c.take<int32_t>(g.E + (N + 31) / 32);
  w.ntiles = c.take<int32_t>(1);
  w.pos = c.take<int32_t>(N);
  w.perm = c.take<int32_t>(N);
  w.hq = mx ? nullptr : c.take<uint16_t>(R * g.I);
  w.hs = mx ? nullptr : c.take<float>(R * (g.I / 64));
  w.hu = mx ? nullptr : c.take<float>(R * (g.I / 64));
  w.h32 = mx ? c.take<float>(R * g.I) : nullptr;
  w.h8 = mx ? c.take<uint8_t>(3 * R * g.I) : nullptr;
  w.hsc = mx ? c.take<uint8_t>(3 * R * (g.I / 32)) : nullptr;
  w.y = c.take<float>(R * g.H);
  *total = c.used;
  return w;
}
}  // namespace

size_t workspace_prefill_bytes(const Geometry& g, int T) {
  size_t total = 0;
  carve_prefill_impl(g, T, nullptr, &total);
  return total;
}

PrefillWorkspace carve_prefill(const Geometry& g, int T, void* base) {
  size_t total = 0;
  return carve_prefill_impl(g, T, base, &total);
}

Workspace carve_workspace(const Geometry& g, int T, void* base) {
  const size_t t = (size_t)T;
  uint8_t* p = static_cast<uint8_t*>(base) + MOE_WS_SYNC_BYTES;  // after the sync region
  Workspace ws;
  ws.logits = reinterpret_cast<double*>(p); p += align256(t * (g.E + 1) * 8);
  ws.idx = reinterpret_cast<int32_t*>(p); p += align256(t * g.K * 4);
  ws.w = reinterpret_cast<float*>(p); p += align256(t * g.K * 4);
  ws.g = reinterpret_cast<float*>(p); p += align256(t * 4);
  ws.h = reinterpret_cast<float*>(p); p += align256(t * g.NE * g.I * 4);
  ws.u = reinterpret_cast<float*>(p); p += align256(t * g.H * 4);
  ws.rnorm = reinterpret_cast<double*>(p);
  return ws;
}

}  // namespace bqmoe

using namespace bqmoe;

extern "C" {

size_t moe_blob_bytes(int hidden, int inter, int bits, int group) {
  if ((bits != 2 && bits != 4) || (group != 64 && !(group == 32 && bits == 4))) return 0;
  if (hidden <= 0 || inter <= 0 || hidden % 64 != 0 || inter % 64 != 0) return 0;
  const uint64_t w = (uint64_t)hidden * inter;
  return (size_t)(3 * w * bits / 8 + 3 * (w / group) * (group == 32 ? 1 : 4));
}

size_t moe_workspace_bytes(const moe_layer_t* layer, int T) {
  Geometry g;
  const char* why = nullptr;
  if (layer == nullptr || T < 0 || !geometry_from(layer, &g, &why)) return 0;
  const int t = T < 1 ? 1 : T;
  size_t n = workspace_layer_bytes(g, t);
  if (t >= BQ_PREFILL_MIN) {
    const size_t pf = workspace_prefill_bytes(g, t);
    if (pf > n) n = pf;
  }
  return n;
}

int moe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < (size_t)MOE_WS_SYNC_BYTES) return fail(MOE_ENOSPC, "workspace smaller than MOE_WS_SYNC_BYTES");
  return hip_status(launch_zero(ws, MOE_WS_SYNC_BYTES, static_cast<hipStream_t>(stream)));
}

size_t moe_stack_workspace_bytes(const moe_layer_t* layer, int T) {
  const size_t base = moe_workspace_bytes(layer, T);
  if (base == 0) return 0;
  return base + 2 * align256((size_t)(T < 1 ? 1 : T) * layer->hidden * 4);
}

int moe_pack_expert(int hidden, int inter, int bits, int group, const moe_expert_arrays_t* a, void* blob_host) {
  const size_t bytes = moe_blob_bytes(hidden, inter, bits, group);
  if (bytes == 0)
    return fail(MOE_EUNSUPPORTED, "unsupported blob shape (bits 2/4 with group 64, or bits 4 with group 32; dims multiple of 64)");
  if (a == nullptr || blob_host == nullptr) return fail(MOE_EINVAL, "arrays and blob must be non-NULL");
  const bool mx = group == 32;
  for (int m = 0; m < 3; ++m)
    if (a->q[m] == nullptr || a->scale[m] == nullptr || (!mx && a->bias[m] == nullptr))
      return fail(MOE_EINVAL, "every q/scale array (and bias, for the affine format) must be non-NULL");
  const int64_t n = (int64_t)hidden * inter;
  if (mx)
    for (int m = 0; m < 3; ++m)
      for (int64_t i = 0; i < n / group; ++i)
        if (a->scale[m][i] > 255) return fail(MOE_EINVAL, "an E8M0 scale does not fit in 8 bits");
  const int per = 8 / bits;
  const uint8_t lim = (uint8_t)(1u << bits);
  for (int m = 0; m < 3; ++m)
    for (int64_t i = 0; i < n; ++i)
      if (a->q[m][i] >= lim) return fail(MOE_EINVAL, "a code does not fit in `bits` bits");
  uint8_t* out = static_cast<uint8_t*>(blob_host);
  const int64_t cb = n * bits / 8, ng = n / group;
  for (int m = 0; m < 3; ++m) {
    // row-major in both layouts: element i of the matrix is element i of the flattened code stream
    uint8_t* codes = out + m * cb;
    for (int64_t k = 0; k < cb; ++k) {
      uint32_t v = 0;
      for (int j = 0; j < per; ++j) v |= (uint32_t)a->q[m][k * per + j] << (bits * j);
      codes[k] = (uint8_t)v;
    }
    if (mx) {
      uint8_t* sc = out + 3 * cb + m * ng;
      for (int64_t k = 0; k < ng; ++k) sc[k] = (uint8_t)a->scale[m][k];
      continue;
    }
    uint8_t* sb = out + 3 * cb + m * ng * 4;
    for (int64_t k = 0; k < ng; ++k) {
      const uint32_t word = (uint32_t)a->scale[m][k] | ((uint32_t)a->bias[m][k] << 16);
      memcpy(sb + 4 * k, &word, 4);
    }
  }
  return ok();
}

int moe_pack_expert_device(int hidden, int inter, int bits, int group, const moe_expert_arrays_t* a, void* blob_dev,
                           void* stream) {
  if (moe_blob_bytes(hidden, inter, bits, group) == 0)
    return fail(MOE_EUNSUPPORTED, "unsupported blob shape (bits 2/4 with group 64, or bits 4 with group 32; dims multiple of 64)");
  if (a == nullptr || blob_dev == nullptr) return fail(MOE_EINVAL, "arrays and blob must be non-NULL");
  for (int m = 0; m < 3; ++m)
    if (a->q[m] == nullptr || a->scale[m] == nullptr || (group != 32 && a->bias[m] == nullptr))
      return fail(MOE_EINVAL, "every q/scale array (and bias, for the affine format) must be non-NULL");
  if (!aligned(blob_dev, 4)) return fail(MOE_EINVAL, "blob_dev must be 4-byte aligned");
  return hip_status(launch_pack(hidden, inter, bits, group, a, static_cast<uint8_t*>(blob_dev),
                                static_cast<hipStream_t>(stream)));
}

int moe_dequant(const moe_layer_t* layer, int expert, int matrix, int out_dtype, void* w_out, void* stream) {
  Geometry g;
  int rc = check_layer(layer, &g);
  if (rc) return rc;
  if (expert < -1 || expert >= g.E) return fail(MOE_EINVAL, "expert must be in [-1, n_experts)");
  if (expert == -1 && !g.has_shared) return fail(MOE_EINVAL, "expert -1 needs a shared expert");
  if (matrix < 0 || matrix > 2) return fail(MOE_EINVAL, "matrix must be 0 (gate), 1 (up) or 2 (down)");
  if (out_dtype != 0 && out_dtype != 1) return fail(MOE_EINVAL, "out_dtype must be 0 (fp32) or 1 (bf16)");
  if (w_out == nullptr) return fail(MOE_EINVAL, "w_out is NULL");
  const uint8_t* blob = expert < 0 ? static_cast<const uint8_t*>(layer->shared_blob_dev)
                                   : static_cast<const uint8_t*>(layer->experts_dev) + (size_t)expert * layer->expert_stride;
  return hip_status(launch_dequant(g, blob, matrix, out_dtype, w_out, static_cast<hipStream_t>(stream)));
}

namespace {
// The grouped (prefill) path, from MOE_PREFILL_MIN_TOKENS tokens (MXFP4 layers need inter >= 128:
// their grouped GEMM steps K by 128).
bool use_prefill(const Geometry& g, int T) { return T >= BQ_PREFILL_MIN && (g.form != 3 || g.I >= 128); }

// The MXFP4 grouped GEMMs address their activation planes (3 E4M3 terms of [rows][K]) with 32-bit
// buffer offsets: both the input's planes (T rows of H) and the SwiGLU outputs' (T*(K+shared)
// rows of I) must stay under 2^31 bytes.
int check_prefill_size(const Geometry& g, int T) {
  if (!use_prefill(g, T) || g.form != 3) return MOE_OK;
  const uint64_t rows = (uint64_t)T * (g.K + g.has_shared);
  if (3ull * T * g.H >= (1ull << 31) || 3ull * rows * g.I >= (1ull << 31))
    return fail(MOE_EUNSUPPORTED, "too many tokens for one MXFP4 prefill call (3*T*hidden and "
                                  "3*T*(top_k+shared)*inter must stay below 2^31)");
  return MOE_OK;
}

size_t needed_ws(const Geometry& g, int T) {
  size_t n = workspace_layer_bytes(g, T);
  if (T >= BQ_PREFILL_MIN) {
    const size_t pf = workspace_prefill_bytes(g, T);
    if (pf > n) n = pf;
  }
  return n;
}

// Argument checks shared by moe_layer_forward and moe_layer_forward_noalloc (no HIP call). Returns
// MOE_OK with T == 0 for the empty call.
int check_layer_call(const moe_layer_t* layer, const float* x, const float* residual, int T, float* out, Geometry* g) {
  int rc = check_layer(layer, g);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if ((rc = check_act(x, "x"))) return rc;
  if ((rc = check_act(out, "out"))) return rc;
  if (residual == nullptr) return fail(MOE_EINVAL, "residual is NULL");
  if (x == out) return fail(MOE_EINVAL, "x and out may not alias");
  return check_prefill_size(*g, T);
}
}  // namespace

int moe_router(const moe_layer_t* layer, const float* x, int T, int32_t* idx, float* w, float* shared_g,
               double* logits, void* ws, size_t ws_bytes, void* stream) {
  Geometry g;
  int rc = check_layer(layer, &g);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if ((rc = check_act(x, "x"))) return rc;
  if (idx == nullptr || w == nullptr) return fail(MOE_EINVAL, "idx and w must be non-NULL");
  if (ws == nullptr || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < needed_ws(g, T)) return fail(MOE_ENOSPC, "workspace smaller than moe_workspace_bytes()");
  const Workspace W = carve_workspace(g, T, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_router_select(g, ptrs_of(layer), x, T, W, idx, w, shared_g, logits, nullptr, s);
  return hip_status(e);
}

int moe_router_approx_logits(const moe_layer_t* layer, const float* x, int T, double* logits, double* kc,
                             void* stream) {
  Geometry g;
  int rc = check_layer(layer, &g);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if ((rc = check_act(x, "x"))) return rc;
  if (logits == nullptr || !aligned(logits, 8)) return fail(MOE_EINVAL, "logits must be non-NULL and 8-byte aligned");
  double k = 0.0;
  const hipError_t e = launch_router_approx(g, ptrs_of(layer), x, T, logits, &k, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && kc != nullptr) *kc = k;
  return hip_status(e);
}

int moe_expert_ffn(const moe_layer_t* layer, const float* x, int T, const int32_t* idx, float* y, void* ws,
                   size_t ws_bytes, void* stream) {
  return moe_expert_ffn_checked(layer, x, T, idx, y, ws, ws_bytes, nullptr, stream);
}

int moe_expert_ffn_checked(const moe_layer_t* layer, const float* x, int T, const int32_t* idx, float* y, void* ws,
                           size_t ws_bytes, int32_t* err, void* stream) {
  Geometry g;
  int rc = check_layer(layer, &g);
  if (rc) return rc;
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if ((rc = check_act(x, "x"))) return rc;
  if ((rc = check_act(y, "y"))) return rc;
  if (idx == nullptr) return fail(MOE_EINVAL, "idx is NULL");
  if (ws == nullptr || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < needed_ws(g, T)) return fail(MOE_ENOSPC, "workspace smaller than moe_workspace_bytes()");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LayerPtrs p = ptrs_of(layer);
  if ((rc = check_prefill_size(g, T))) return rc;
  if (err != nullptr && !aligned(err, 4)) return fail(MOE_EINVAL, "err must be 4-byte aligned");
  if (use_prefill(g, T))
    return hip_status(launch_prefill(g, p, x, nullptr, T, carve_prefill(g, T, ws), idx, nullptr, nullptr, y, err, s));
  const Workspace W = carve_workspace(g, T, ws);
  hipError_t e = launch_gateup(g, p, x, T, W, idx, nullptr, true, err, s);
  if (e == hipSuccess) e = launch_down(g, p, T, W, idx, nullptr, nullptr, y, s);
  return hip_status(e);
}

int moe_combine(const moe_layer_t* layer, const float* residual, const float* y, const float* w, const float* shared_g,
                int T, float* out, void* stream) {
  Geometry g;
  const char* why = nullptr;
  if (layer == nullptr) return fail(MOE_EINVAL, "layer is NULL");
  if (!geometry_from(layer, &g, &why)) return fail(MOE_EUNSUPPORTED, why);
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if (residual == nullptr || y == nullptr || w == nullptr || out == nullptr)
    return fail(MOE_EINVAL, "residual, y, w and out must be non-NULL");
  if (g.has_shared && shared_g == nullptr) return fail(MOE_EINVAL, "shared_g is NULL but the layer has a shared expert");
  return hip_status(launch_combine(g, T, residual, y, w, shared_g, out, static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_layer_t* layer, const float* x, const float* residual, int T, float* out,
                      int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return moe_layer_forward_timed(layer, x, residual, T, out, idx_out, ws, ws_bytes, stream, nullptr);
}

int moe_layer_forward_timed(const moe_layer_t* layer, const float* x, const float* residual, int T, float* out,
                            int32_t* idx_out, void* ws, size_t ws_bytes, void* stream, void* const* events) {
  Geometry g;
  int rc = check_layer_call(layer, x, residual, T, out, &g);
  if (rc || T == 0) return rc;
  if (ws == nullptr || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  if (ws_bytes < needed_ws(g, T)) return fail(MOE_ENOSPC, "workspace smaller than moe_workspace_bytes()");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LayerPtrs p = ptrs_of(layer);
  auto ev = [&](int k) {
    KernelEvents e;
    if (events != nullptr) {
      e.start = static_cast<hipEvent_t>(events[2 * k]);
      e.stop = static_cast<hipEvent_t>(events[2 * k + 1]);
    }
    return e;
  };
  if (use_prefill(g, T)) {
    // many kernels: events[0] and events[5] are recorded around all of them
    hipError_t e = hipSuccess;
    if (events != nullptr && events[0] != nullptr) e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s);
    if (e == hipSuccess)
      e = launch_prefill(g, p, x, residual, T, carve_prefill(g, T, ws), nullptr, idx_out, out, nullptr, nullptr, s);
    if (e == hipSuccess && events != nullptr && events[5] != nullptr)
      e = hipEventRecord(static_cast<hipEvent_t>(events[5]), s);
    return hip_status(e);
  }
  const Workspace W = carve_workspace(g, T, ws);
  if (T == 1 && pair_supported(g))
    return hip_status(launch_pair(g, p, x, nullptr, 0.0f, residual, out, idx_out, W, static_cast<uint8_t*>(ws),
                                  nullptr, s, ev(0), ev(2)));
  hipError_t e = launch_router_phase(g, p, x, nullptr, 0.0f, T, W, s, ev(0));
  if (e == hipSuccess) e = launch_gateup(g, p, x, T, W, nullptr, idx_out, true, nullptr, s, ev(1));
  if (e == hipSuccess) e = launch_down(g, p, T, W, W.idx, residual, out, nullptr, s, ev(2));
  return hip_status(e);
}

int moe_layer_plan(const moe_layer_t* layer, int T) {
  if (layer == nullptr) return fail(MOE_EINVAL, "layer is NULL");
  Geometry g;
  const char* why = nullptr;
  if (!geometry_from(layer, &g, &why)) return fail(MOE_EUNSUPPORTED, why);
  if (T < 1) return fail(MOE_EINVAL, "T must be >= 1");
  ok();
  if (use_prefill(g, T)) return MOE_PLAN_PREFILL;
  return T == 1 && pair_supported(g) ? MOE_PLAN_PAIR : MOE_PLAN_CHAIN;
}

int moe_layer_forward_noalloc(const moe_layer_t* layer, const float* x, const float* residual, int T, float* out,
                              int32_t* idx_out, void* stream) {
  Geometry g;
  int rc = check_layer_call(layer, x, residual, T, out, &g);
  if (rc || T == 0) return rc;
  if (needed_ws(g, T) > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ENOSPC, "this layer and T need more workspace than MOE_NOALLOC_SCRATCH_BYTES; call "
                            "moe_layer_forward with a workspace of moe_workspace_bytes()");
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  return moe_layer_forward_timed(layer, x, residual, T, out, idx_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_stack_forward(const moe_layer_t* layers, int L, float eps, const float* x, int T, float* out,
                      int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (layers == nullptr || L < 1) return fail(MOE_EINVAL, "layers must be non-NULL and L >= 1");
  Geometry g;
  int rc = check_layer(&layers[0], &g);
  if (rc) return rc;
  for (int l = 1; l < L; ++l) {
    Geometry gl;
    if ((rc = check_layer(&layers[l], &gl))) return rc;
    if (gl.H != g.H || gl.I != g.I || gl.E != g.E || gl.K != g.K || gl.bits != g.bits || gl.G != g.G ||
        gl.form != g.form || gl.has_shared != g.has_shared)
      return fail(MOE_EINVAL, "all layers must share hidden, inter, n_experts, top_k, bits, group, flags and has_shared");
  }
  if (!(eps >= 0.0f)) return fail(MOE_EINVAL, "eps must be >= 0");
  if (T < 0) return fail(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return ok();
  if ((rc = check_act(x, "x"))) return rc;
  if ((rc = check_act(out, "out"))) return rc;
  if (ws == nullptr || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be non-NULL and 256-byte aligned");
  const size_t base = workspace_layer_bytes(g, T);
  const size_t hb = align256((size_t)T * g.H * 4);
  if (ws_bytes < base + 2 * hb) return fail(MOE_ENOSPC, "workspace smaller than moe_stack_workspace_bytes()");
  const Workspace W = carve_workspace(g, T, ws);
  float* hbuf[2] = {reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + base),
                    reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + base + hb)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* h = x;  // h_l
  hipError_t e = hipSuccess;
  for (int l = 0; l < L && e == hipSuccess; ++l) {
    const LayerPtrs p = ptrs_of(&layers[l]);
    float* h_next = (l == L - 1) ? out : hbuf[l & 1];
    const float* norm_src = (l == 0) ? nullptr : h;
    const float* xin = (l == 0) ? x : W.u;
    int32_t* io = idx_out ? idx_out + (size_t)l * T * g.K : nullptr;
    if (T == 1 && pair_supported(g)) {
      e = launch_pair(g, p, x, norm_src, eps, h, h_next, io, W, static_cast<uint8_t*>(ws), nullptr, s);
    } else {
      e = launch_router_phase(g, p, x, norm_src, eps, T, W, s);
      if (e == hipSuccess) e = launch_gateup(g, p, xin, T, W, nullptr, io, true, nullptr, s);
      if (e == hipSuccess) e = launch_down(g, p, T, W, W.idx, h, h_next, nullptr, s);
    }
    h = h_next;
  }
  return hip_status(e);
}

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or format";
    case MOE_ENOSPC: return "workspace too small";
    case MOE_EHIP: return "HIP error";
    case MOE_ETIMEOUT: return "the decode's first kernel gave up waiting for its blocks";
    default: return "unknown error";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
