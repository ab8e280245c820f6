"""ctypes binding of libbqmoe.so (include/moe.h), with the same names as the C entry points.

Argument marshalling only: every step of the layer runs in the HIP library. Torch tensors are
accepted for device buffers (their data_ptr is passed) and torch streams for streams.
PyTorch supplies device memory and streams and nothing else. A missing library is an error;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbqmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOSPC, MOE_EHIP, MOE_ETIMEOUT = 0, -1, -2, -3, -4, -5
MOE_MAX_TOP_K, MOE_MAX_EXPERTS, MOE_PREFILL_MIN_TOKENS = 8, 1024, 48
MOE_ROUTER_BATCH_MIN_TOKENS, MOE_ROUTER_CERTIFIED_MIN_TOKENS = 96, 512
MOE_FLAG_DEQUANT_LITERAL, MOE_FLAG_DEQUANT_NAIVE = 1, 2
MOE_FLAG_DECODE_CHAIN = 4
MOE_WS_SYNC_BYTES = 32768
MOE_PLAN_PAIR, MOE_PLAN_CHAIN, MOE_PLAN_PREFILL = 1, 2, 3
MOE_NOALLOC_SCRATCH_BYTES = 33554432

c_i32, c_u64, c_size, c_vp, c_f32 = ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


class moe_layer_t(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("inter", c_i32), ("n_experts", c_i32), ("top_k", c_i32),
                ("has_shared", c_i32), ("bits", c_i32), ("group", c_i32), ("flags", c_i32),
                ("experts_dev", c_vp), ("expert_stride", c_u64), ("shared_blob_dev", c_vp),
                ("router_dev", c_vp), ("shared_gate_dev", c_vp)]


class moe_expert_arrays_t(ctypes.Structure):
    _fields_ = [("q", c_vp * 3), ("scale", c_vp * 3), ("bias", c_vp * 3)]


# name -> (restype, argtypes); the set of symbols include/moe.h declares
SIGNATURES = {
    "moe_blob_bytes": (c_size, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "moe_workspace_bytes": (c_size, [ctypes.POINTER(moe_layer_t), ctypes.c_int]),
    "moe_stack_workspace_bytes": (c_size, [ctypes.POINTER(moe_layer_t), ctypes.c_int]),
    "moe_workspace_init": (ctypes.c_int, [c_vp, c_size, c_vp]),
    "moe_pack_expert": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.POINTER(moe_expert_arrays_t), c_vp]),
    "moe_pack_expert_device": (ctypes.c_int, [ctypes.c_int] * 4 + [ctypes.POINTER(moe_expert_arrays_t), c_vp, c_vp]),
    "moe_dequant": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), ctypes.c_int, ctypes.c_int, ctypes.c_int, c_vp, c_vp]),
    "moe_router": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_vp,
                                  c_size, c_vp]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, ctypes.c_int, c_vp, c_vp, c_vp, c_size, c_vp]),
    "moe_expert_ffn_checked": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, ctypes.c_int, c_vp, c_vp, c_vp, c_size,
                                              c_vp, c_vp]),
    "moe_router_approx_logits": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, ctypes.c_int, c_vp,
                                                ctypes.POINTER(ctypes.c_double), c_vp]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, c_vp, c_vp, c_vp, ctypes.c_int, c_vp, c_vp]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, c_vp, ctypes.c_int, c_vp, c_vp, c_vp,
                                         c_size, c_vp]),
    "moe_layer_plan": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), ctypes.c_int]),
    "moe_layer_forward_timed": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, c_vp, ctypes.c_int, c_vp, c_vp, c_vp,
                                               c_size, c_vp, ctypes.POINTER(c_vp)]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), c_vp, c_vp, ctypes.c_int, c_vp, c_vp,
                                                 c_vp]),
    "moe_stack_forward": (ctypes.c_int, [ctypes.POINTER(moe_layer_t), ctypes.c_int, c_f32, c_vp, ctypes.c_int, c_vp,
                                         c_vp, c_vp, c_size, c_vp]),
    "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


class MoeError(RuntimeError):
    def __init__(self, code: int, fn: str):
        self.code = code
        detail = lib().moe_last_error().decode()
        super().__init__(f"{fn} failed: {lib().moe_strerror(code).decode()} ({code}): {detail}")


def _check(code: int, fn: str) -> None:
    if code != MOE_OK:
        raise MoeError(code, fn)


def ptr(t) -> int | None:
    """Device/host address of a torch tensor, numpy array, raw int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    raise TypeError(f"cannot take the address of {type(t)}")


def stream_handle(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_layer(hidden, inter, n_experts, top_k, bits, experts, expert_stride, router, shared_blob=None,
               shared_gate=None, group=64, flags=0) -> moe_layer_t:
    return moe_layer_t(hidden, inter, n_experts, top_k, 1 if shared_blob is not None else 0, bits, group, flags,
                       ptr(experts), expert_stride, ptr(shared_blob), ptr(router), ptr(shared_gate))


def _ref(layer):
    return ctypes.byref(layer) if isinstance(layer, moe_layer_t) else layer


# ---- entry points (same names as the C ABI) ---------------------------------------------------------

def moe_blob_bytes(hidden: int, inter: int, bits: int, group: int = 64) -> int:
    return lib().moe_blob_bytes(hidden, inter, bits, group)


def moe_workspace_bytes(layer, T: int) -> int:
    return lib().moe_workspace_bytes(_ref(layer), T)


def moe_stack_workspace_bytes(layer, T: int) -> int:
    return lib().moe_stack_workspace_bytes(_ref(layer), T)


def moe_workspace_init(ws, ws_bytes: int, stream=None) -> None:
    _check(lib().moe_workspace_init(ptr(ws), ws_bytes, stream_handle(stream)), "moe_workspace_init")


def _arrays(q, scale, bias) -> moe_expert_arrays_t:
    a = moe_expert_arrays_t()
    for m in range(3):
        a.q[m], a.scale[m], a.bias[m] = ptr(q[m]), ptr(scale[m]), ptr(bias[m])
    return a


def moe_pack_expert(hidden, inter, bits, group, q, scale, bias, blob_host) -> None:
    a = _arrays(q, scale, bias)
    _check(lib().moe_pack_expert(hidden, inter, bits, group, ctypes.byref(a), ptr(blob_host)), "moe_pack_expert")


def moe_pack_expert_device(hidden, inter, bits, group, q, scale, bias, blob_dev, stream=None) -> None:
    a = _arrays(q, scale, bias)
    _check(lib().moe_pack_expert_device(hidden, inter, bits, group, ctypes.byref(a), ptr(blob_dev),
                                        stream_handle(stream)), "moe_pack_expert_device")


def moe_dequant(layer, expert: int, matrix: int, out_dtype: int, w_out, stream=None) -> None:
    _check(lib().moe_dequant(_ref(layer), expert, matrix, out_dtype, ptr(w_out), stream_handle(stream)), "moe_dequant")


def moe_router(layer, x, T, idx, w, shared_g, logits, ws, ws_bytes, stream=None) -> None:
    _check(lib().moe_router(_ref(layer), ptr(x), T, ptr(idx), ptr(w), ptr(shared_g), ptr(logits), ptr(ws), ws_bytes,
                            stream_handle(stream)), "moe_router")


def moe_expert_ffn(layer, x, T, idx, y, ws, ws_bytes, stream=None) -> None:
    _check(lib().moe_expert_ffn(_ref(layer), ptr(x), T, ptr(idx), ptr(y), ptr(ws), ws_bytes, stream_handle(stream)),
           "moe_expert_ffn")


def moe_expert_ffn_checked(layer, x, T, idx, y, ws, ws_bytes, err, stream=None) -> None:
    _check(lib().moe_expert_ffn_checked(_ref(layer), ptr(x), T, ptr(idx), ptr(y), ptr(ws), ws_bytes, ptr(err),
                                        stream_handle(stream)), "moe_expert_ffn_checked")


def moe_router_approx_logits(layer, x, T, logits, stream=None) -> float:
    kc = ctypes.c_double(0.0)
    _check(lib().moe_router_approx_logits(_ref(layer), ptr(x), T, ptr(logits), ctypes.byref(kc), stream_handle(stream)),
           "moe_router_approx_logits")
    return kc.value


def moe_combine(layer, residual, y, w, shared_g, T, out, stream=None) -> None:
    _check(lib().moe_combine(_ref(layer), ptr(residual), ptr(y), ptr(w), ptr(shared_g), T, ptr(out),
                             stream_handle(stream)), "moe_combine")


def moe_layer_forward(layer, x, residual, T, out, idx_out, ws, ws_bytes, stream=None) -> None:
    _check(lib().moe_layer_forward(_ref(layer), ptr(x), ptr(residual), T, ptr(out), ptr(idx_out), ptr(ws), ws_bytes,
                                   stream_handle(stream)), "moe_layer_forward")


def moe_layer_plan(layer, T: int) -> int:
    """MOE_PLAN_PAIR, MOE_PLAN_CHAIN or MOE_PLAN_PREFILL for T tokens of this layer on the current device."""
    code = lib().moe_layer_plan(_ref(layer), T)
    if code < 0:
        raise MoeError(code, "moe_layer_plan")
    return code


def moe_layer_forward_noalloc(layer, x, residual, T, out, idx_out, stream=None) -> None:
    _check(lib().moe_layer_forward_noalloc(_ref(layer), ptr(x), ptr(residual), T, ptr(out), ptr(idx_out),
                                           stream_handle(stream)), "moe_layer_forward_noalloc")


def moe_layer_forward_timed(layer, x, residual, T, out, idx_out, ws, ws_bytes, events, stream=None) -> None:
    """events: 6 raw hipEvent_t handles (ints) or None entries."""
    ev = (c_vp * 6)(*[(e if e else None) for e in events])
    _check(lib().moe_layer_forward_timed(_ref(layer), ptr(x), ptr(residual), T, ptr(out), ptr(idx_out), ptr(ws),
                                         ws_bytes, stream_handle(stream), ev), "moe_layer_forward_timed")


def moe_stack_forward(layers, eps, x, T, out, idx_out, ws, ws_bytes, stream=None) -> None:
    arr = (moe_layer_t * len(layers))(*layers)
    _check(lib().moe_stack_forward(arr, len(layers), eps, ptr(x), T, ptr(out), ptr(idx_out), ptr(ws), ws_bytes,
                                   stream_handle(stream)), "moe_stack_forward")


def moe_strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()
