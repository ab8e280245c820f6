"""ORACLE — test infrastructure only.

Plain fp64 CPU reference of the quantised MoE layer. It wraps ``liboracle.so``, built from
``oracle.c``; the sources, readings and pins are listed in ``oracle.h``. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import this package.
The GPU library never does.

The layer is composed here in the pages' order. The router result picks the experts
(HN thread "Flash-MoE: Running a 397B Parameter Model on a Laptop"). The experts run dequant
mat-vec, SwiGLU and dequant mat-vec; the outputs are combined with the gated shared expert and
the residual (GN+ summary, "Tecnologías clave > Metal Compute Shaders"). In the stack, combine,
norm and residual feed the next layer ("Deferred GPU Expert Compute").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        i64, vp, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        L.oracle_dequant.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.oracle_matvec.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_router_logits.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_topk.argtypes = [i64, i64, vp, vp]
        L.oracle_route_weights.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_shared_gate.argtypes = [i64, vp, vp]
        L.oracle_shared_gate.restype = dbl
        L.oracle_expert.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [i64, i64, vp, vp, vp, dbl, vp, vp]
        L.oracle_rmsnorm.argtypes = [i64, dbl, vp, vp]
        L.oracle_dequant_mx.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_expert_mx.argtypes = [i64, i64, vp, vp, vp, vp, vp]
        for f in (L.oracle_dequant, L.oracle_matvec, L.oracle_router_logits, L.oracle_topk,
                  L.oracle_route_weights, L.oracle_expert, L.oracle_combine, L.oracle_rmsnorm,
                  L.oracle_dequant_mx, L.oracle_expert_mx):
            f.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def dequant(q, scale, bias, group: int) -> np.ndarray:
    q = _c(q, np.uint8)
    rows, cols = q.shape
    s, b = _c(scale, np.uint16), _c(bias, np.uint16)
    assert s.shape == (rows, cols // group) and b.shape == s.shape
    W = np.empty((rows, cols), dtype=np.float64)
    lib().oracle_dequant(rows, cols, group, _p(q), _p(s), _p(b), _p(W))
    return W


def dequant_mx(q, scale) -> np.ndarray:
    """MXFP4: W = e2m1(q) * 2^(scale - 127), one E8M0 scale per block of 32 along a row (see oracle.h)."""
    q = _c(q, np.uint8)
    rows, cols = q.shape
    s = _c(scale, np.uint16)
    assert s.shape == (rows, cols // 32)
    W = np.empty((rows, cols), dtype=np.float64)
    lib().oracle_dequant_mx(rows, cols, _p(q), _p(s), _p(W))
    return W


def matvec(W, v) -> np.ndarray:
    W, v = _c(W, np.float64), _c(v, np.float64)
    out = np.empty(W.shape[0], dtype=np.float64)
    lib().oracle_matvec(W.shape[0], W.shape[1], _p(W), _p(v), _p(out))
    return out


def router_logits(R, x) -> np.ndarray:
    R, x = _c(R, np.uint16), _c(x, np.float64)
    out = np.empty(R.shape[0], dtype=np.float64)
    lib().oracle_router_logits(R.shape[0], R.shape[1], _p(R), _p(x), _p(out))
    return out


def topk(logits, K: int) -> np.ndarray:
    logits = _c(logits, np.float64)
    idx = np.empty(K, dtype=np.int32)
    lib().oracle_topk(logits.shape[0], K, _p(logits), _p(idx))
    return idx


def route_weights(logits, idx) -> np.ndarray:
    logits, idx = _c(logits, np.float64), _c(idx, np.int32)
    w = np.empty(idx.shape[0], dtype=np.float64)
    lib().oracle_route_weights(logits.shape[0], idx.shape[0], _p(logits), _p(idx), _p(w))
    return w


def shared_gate(gs, x) -> float:
    gs, x = _c(gs, np.uint16), _c(x, np.float64)
    return float(lib().oracle_shared_gate(gs.shape[0], _p(gs), _p(x)))


def expert(x, ex, group: int, want_h: bool = False):
    """ex: an object with .mats = [gate, up, down], each with .q, .scale, .bias canonical arrays, and
    .fmt ("affine", or "mxfp4": E2M1 codes with E8M0 scales per 32 and no bias; group is then unused)."""
    if getattr(ex, "fmt", "affine") == "mxfp4":
        return _expert_mx(x, ex, want_h)
    x = _c(x, np.float64)
    mats = [(_c(m.q, np.uint8), _c(m.scale, np.uint16), _c(m.bias, np.uint16)) for m in ex.mats]
    I, H = mats[0][0].shape
    assert mats[1][0].shape == (I, H) and mats[2][0].shape == (H, I) and x.shape == (H,)
    qs = (ctypes.c_void_p * 3)(*[m[0].ctypes.data for m in mats])
    ss = (ctypes.c_void_p * 3)(*[m[1].ctypes.data for m in mats])
    bs = (ctypes.c_void_p * 3)(*[m[2].ctypes.data for m in mats])
    y = np.empty(H, dtype=np.float64)
    h = np.empty(I, dtype=np.float64) if want_h else None
    lib().oracle_expert(H, I, group, _p(x), qs, ss, bs, _p(y), _p(h))
    return (y, h) if want_h else y


def _expert_mx(x, ex, want_h: bool):
    x = _c(x, np.float64)
    mats = [(_c(m.q, np.uint8), _c(m.scale, np.uint16)) for m in ex.mats]
    I, H = mats[0][0].shape
    assert mats[1][0].shape == (I, H) and mats[2][0].shape == (H, I) and x.shape == (H,)
    qs = (ctypes.c_void_p * 3)(*[m[0].ctypes.data for m in mats])
    ss = (ctypes.c_void_p * 3)(*[m[1].ctypes.data for m in mats])
    y = np.empty(H, dtype=np.float64)
    h = np.empty(I, dtype=np.float64) if want_h else None
    lib().oracle_expert_mx(H, I, _p(x), qs, ss, _p(y), _p(h))
    return (y, h) if want_h else y


def combine(res, y, w, g, ys) -> np.ndarray:
    res, y, w = _c(res, np.float64), _c(y, np.float64), _c(w, np.float64)
    ys = None if ys is None else _c(ys, np.float64)
    K, H = y.shape
    out = np.empty(H, dtype=np.float64)
    lib().oracle_combine(H, K, _p(res), _p(y), _p(w), float(g), _p(ys), _p(out))
    return out


def rmsnorm(h, eps: float) -> np.ndarray:
    h = _c(h, np.float64)
    u = np.empty_like(h)
    lib().oracle_rmsnorm(h.shape[0], float(eps), _p(h), _p(u))
    return u


@dataclass
class LayerResult:
    out: np.ndarray  # [H]
    idx: np.ndarray  # [K] int32, descending logit
    w: np.ndarray  # [K]
    g: float  # shared-expert gate (nan when there is no shared expert)
    logits: np.ndarray  # [E]
    y: np.ndarray  # [K(+1)][H] expert outputs, shared last
    margin: float  # fp64 gap between the K-th and (K+1)-th largest logit (inf when K == E)


def layer(x, res, router, gate_vec, get_expert, K: int, group: int, shared_expert=None) -> LayerResult:
    """One MoE layer for one token. get_expert(e) returns expert e's canonical arrays."""
    logits = router_logits(router, x)
    idx = topk(logits, K)
    order = np.sort(logits)[::-1]
    margin = float(order[K - 1] - order[K]) if K < len(order) else float("inf")
    w = route_weights(logits, idx)
    ys = [expert(x, get_expert(int(e)), group) for e in idx]
    if shared_expert is not None:
        g = shared_gate(gate_vec, x)
        y_sh = expert(x, shared_expert, group)
        out = combine(res, np.stack(ys), w, g, y_sh)
        ys.append(y_sh)
    else:
        g = float("nan")
        out = combine(res, np.stack(ys), w, 0.0, None)
    return LayerResult(out, idx, w, g, logits, np.stack(ys), margin)


@dataclass
class StackResult:
    out: np.ndarray  # h_L [H]
    idx: np.ndarray  # [L][K] top-K per layer
    margin: np.ndarray  # [L] fp64 gap between the K-th and (K+1)-th logit per layer


def stack(x, layers, K: int, group: int, eps: float) -> StackResult:
    """A stack of MoE layers for one token (GN+ summary, "Deferred GPU Expert Compute": combine, norm
    and residual feed the next layer). h_0 = x; layer l reads u_l = h_l for l = 0 and
    u_l = rmsnorm(h_l) for l >= 1, and h_{l+1} = h_l + MoE_l(u_l).

    layers[l] = (router, gate_vec, get_expert, shared_expert).
    """
    h = np.asarray(x, dtype=np.float64)
    idx_all, margins = [], []
    for l, (router, gate_vec, get_expert, shared) in enumerate(layers):
        u = h if l == 0 else rmsnorm(h, eps)
        r = layer(u, h, router, gate_vec, get_expert, K, group, shared_expert=shared)
        idx_all.append(r.idx)
        margins.append(r.margin)
        h = r.out
    return StackResult(h, np.stack(idx_all), np.asarray(margins))
