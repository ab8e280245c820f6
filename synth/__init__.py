"""Seeded synthetic inputs for the quantised MoE expert layer workloads.

This package only makes inputs. It holds none of the layer's arithmetic, and both the oracle
and the GPU library are fed from it. The generator is defined in ``gen.h``. ``gen.c`` is its
host implementation and ``gen_fill.hip`` its GPU twin. The two agree bit for bit on codes,
scales and biases. Normal draws (router, shared gate, activations) are made on the host only.

Workloads model one MoE layer of the 397B, 512-expert, hidden-4096 model that the Flash-MoE
pages describe (GN+ summary, "Arquitectura del modelo" / "Arsitektur model": 60 layers,
512 experts per layer, 4 active per token counting one shared expert, hidden 4096). The
4-bit and 2-bit expert formats are the two configurations on those pages ("Resultados de
rendimiento"). The value distributions are the synthetic stand-ins for the missing trained
weights. The MXFP4 workloads take the expert format and the top-6 routing of the page "300b on
32gb MoE-streaming findings + optimisations" (its summary) at the same layer shape: E2M1 codes in
blocks of 32 with an E8M0 scale per block, no bias.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))

# tensor ids (gen.h)
T_X, T_ROUTER, T_SHARED_GATE, T_CODES, T_SCALE, T_BIAS = 1, 2, 3, 4, 5, 6
SHARED = -1  # expert id of the shared expert
GATE, UP, DOWN = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one workload."""

    name: str
    hidden: int
    n_experts: int
    inter: int
    top_k: int
    bits: int
    group: int = 64
    has_shared: bool = True
    tokens: int = 1
    layers: int = 1
    scale_range: tuple = (0.001, 0.01)
    bias_range: tuple = (-0.08, -0.005)
    router_sigma: float = 0.02
    gate_sigma: float = 0.02
    x_sigma: float = 1.0
    seed: int = 0
    weight_family: int = 0  # key family of the weights (layer l uses layer index l)
    x_family: int = 0  # key family of the activations
    prefill: bool = False
    fmt: str = "affine"  # "affine" (bf16 scale + bias per group) or "mxfp4" (E8M0 scale per 32, group 32)
    mx_scale_range: tuple = (118, 122)  # E8M0 scale bytes: 2^-9 .. 2^-5

    def matrix_shape(self, m: int) -> tuple:
        return (self.inter, self.hidden) if m in (GATE, UP) else (self.hidden, self.inter)


_FOUR_BIT = dict(bits=4, scale_range=(0.001, 0.01), bias_range=(-0.08, -0.005))
_TWO_BIT = dict(bits=2, scale_range=(0.004, 0.04), bias_range=(-0.06, -0.004))

WORKLOADS = {
    # tiny layer, 1 token: H256, E8, I128, top-2 routed + shared, 4-bit, seed 0
    "tiny": Workload("tiny", 256, 8, 128, 2, tokens=1, weight_family=0, x_family=0, **_FOUR_BIT),
    # single-token decode at the model's shape, 4-bit, 1000 seeded tokens
    "decode4": Workload("decode4", 4096, 512, 1024, 3, tokens=1000, weight_family=1, x_family=1, **_FOUR_BIT),
    # as decode4 with 2-bit experts
    "decode2": Workload("decode2", 4096, 512, 1024, 3, tokens=1000, weight_family=2, x_family=2, **_TWO_BIT),
    # 2048-token prefill through the decode4 layer (same weights)
    "prefill4": Workload("prefill4", 4096, 512, 1024, 3, tokens=2048, weight_family=1, x_family=3,
                         prefill=True, **_FOUR_BIT),
    # 60-layer decode stack of decode4-shaped layers (layer 0 has decode4's weights), 128 tokens
    "stack60": Workload("stack60", 4096, 512, 1024, 3, tokens=128, layers=60, weight_family=1, x_family=4,
                        **_FOUR_BIT),
}

_MX = dict(bits=4, group=32, fmt="mxfp4")
WORKLOADS.update({
    # tiny MXFP4 layer, top-6 of 8 experts + shared
    "tinymx": Workload("tinymx", 256, 8, 128, 6, tokens=1, weight_family=6, x_family=6, **_MX),
    # single-token decode at the model's shape with MXFP4 experts and top-6 routing
    "decodemx": Workload("decodemx", 4096, 512, 1024, 6, tokens=1000, weight_family=7, x_family=7, **_MX),
    # 2048-token prefill through the decodemx layer
    "prefillmx": Workload("prefillmx", 4096, 512, 1024, 6, tokens=2048, weight_family=7, x_family=8,
                          prefill=True, **_MX),
})

_host = None
_gpu = None


def _load(name):
    path = os.path.join(_HERE, name)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    return ctypes.CDLL(path)


def host_lib():
    global _host
    if _host is None:
        lib = _load("libbqsynth.so")
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.bq_mix64.argtypes, lib.bq_mix64.restype = [u64], u64
        lib.bq_draw.argtypes, lib.bq_draw.restype = [u64, u64], u64
        lib.bq_tensor_key.argtypes, lib.bq_tensor_key.restype = [u64, i64, i64, i64, i64, i64], u64
        lib.bq_bf16_rne.argtypes, lib.bq_bf16_rne.restype = [dbl], ctypes.c_uint16
        lib.bq_gen_codes.argtypes, lib.bq_gen_codes.restype = [u64, i32, i64, i64, vp], None
        lib.bq_gen_uniform_bf16.argtypes, lib.bq_gen_uniform_bf16.restype = [u64, dbl, dbl, i64, i64, vp], None
        lib.bq_gen_normal_bf16.argtypes, lib.bq_gen_normal_bf16.restype = [u64, dbl, i64, i64, vp], None
        lib.bq_gen_normal_f32.argtypes, lib.bq_gen_normal_f32.restype = [u64, dbl, i64, i64, vp], None
        lib.bq_gen_ints_u16.argtypes, lib.bq_gen_ints_u16.restype = [u64, i32, i32, i64, i64, vp], None
        _host = lib
    return _host


def gpu_lib():
    global _gpu
    if _gpu is None:
        lib = _load("libbqsynth_gpu.so")
        u64, i64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.bqgen_fill_codes.argtypes, lib.bqgen_fill_codes.restype = [u64, i32, i64, vp, vp], i32
        lib.bqgen_fill_uniform_bf16.argtypes, lib.bqgen_fill_uniform_bf16.restype = [u64, dbl, dbl, i64, vp, vp], i32
        lib.bqgen_fill_ints_u16.argtypes, lib.bqgen_fill_ints_u16.restype = [u64, i32, i32, i64, vp, vp], i32
        _gpu = lib
    return _gpu


def key(w: Workload, family: int, layer: int, tensor: int, expert: int = SHARED, matrix: int = 0) -> int:
    return host_lib().bq_tensor_key(w.seed, family, layer, tensor, expert, matrix)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---- host generation --------------------------------------------------------------------------

def codes(k: int, bits: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    host_lib().bq_gen_codes(k, bits, start, n, _ptr(out))
    return out


def uniform_bf16(k: int, lo: float, hi: float, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().bq_gen_uniform_bf16(k, lo, hi, start, n, _ptr(out))
    return out


def ints_u16(k: int, lo: int, hi: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().bq_gen_ints_u16(k, lo, hi, start, n, _ptr(out))
    return out


def normal_bf16(k: int, sigma: float, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().bq_gen_normal_bf16(k, sigma, start, n, _ptr(out))
    return out


def normal_f32(k: int, sigma: float, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().bq_gen_normal_f32(k, sigma, start, n, _ptr(out))
    return out


@dataclass
class MatrixArrays:
    """Canonical arrays of one quantised matrix: q[rows][cols] codes, scale/bias[rows][cols/group] bf16
    (affine). For MXFP4, q holds E2M1 codes, scale the E8M0 bytes (uint16 each) and bias is None."""

    q: np.ndarray
    scale: np.ndarray
    bias: np.ndarray | None
    fmt: str = "affine"


@dataclass
class ExpertArrays:
    gate: MatrixArrays
    up: MatrixArrays
    down: MatrixArrays
    mats: list = field(init=False)

    def __post_init__(self):
        self.mats = [self.gate, self.up, self.down]

    @property
    def fmt(self) -> str:
        return self.gate.fmt


def matrix_arrays(w: Workload, layer: int, expert: int, m: int) -> MatrixArrays:
    rows, cols = w.matrix_shape(m)
    fam = w.weight_family
    q = codes(key(w, fam, layer, T_CODES, expert, m), w.bits, rows * cols).reshape(rows, cols)
    ng = rows * (cols // w.group)
    if w.fmt == "mxfp4":
        s = ints_u16(key(w, fam, layer, T_SCALE, expert, m), *w.mx_scale_range, ng).reshape(rows, cols // w.group)
        return MatrixArrays(q, s, None, "mxfp4")
    s = uniform_bf16(key(w, fam, layer, T_SCALE, expert, m), *w.scale_range, ng).reshape(rows, cols // w.group)
    b = uniform_bf16(key(w, fam, layer, T_BIAS, expert, m), *w.bias_range, ng).reshape(rows, cols // w.group)
    return MatrixArrays(q, s, b)


def expert_arrays(w: Workload, layer: int, expert: int) -> ExpertArrays:
    return ExpertArrays(*(matrix_arrays(w, layer, expert, m) for m in (GATE, UP, DOWN)))


def router_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """bf16 bit patterns [E][H]."""
    k = key(w, w.weight_family, layer, T_ROUTER)
    return normal_bf16(k, w.router_sigma, w.n_experts * w.hidden).reshape(w.n_experts, w.hidden)


def shared_gate_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """bf16 bit patterns [H]."""
    k = key(w, w.weight_family, layer, T_SHARED_GATE)
    return normal_bf16(k, w.gate_sigma, w.hidden)


def tokens_x(w: Workload, t0: int, n: int, family: int | None = None) -> np.ndarray:
    """fp32 activations of tokens [t0, t0+n), shape [n][H]; token t is elements [t*H, (t+1)*H)."""
    fam = w.x_family if family is None else family
    k = key(w, fam, 0, T_X)
    return normal_f32(k, w.x_sigma, n * w.hidden, start=t0 * w.hidden).reshape(n, w.hidden)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---- device generation (canonical arrays written in place) -------------------------------------

def fill_matrix_device(w: Workload, layer: int, expert: int, m: int, q_ptr: int, s_ptr: int, b_ptr: int,
                       stream: int) -> None:
    """Write the canonical arrays of one matrix into device buffers (q: rows*cols bytes, 16-B aligned)."""
    g = gpu_lib()
    rows, cols = w.matrix_shape(m)
    fam = w.weight_family
    ng = rows * (cols // w.group)
    rc = g.bqgen_fill_codes(key(w, fam, layer, T_CODES, expert, m), w.bits, rows * cols, q_ptr, stream)
    if w.fmt == "mxfp4":
        rc = rc or g.bqgen_fill_ints_u16(key(w, fam, layer, T_SCALE, expert, m), *w.mx_scale_range, ng, s_ptr, stream)
        if rc != 0:
            raise RuntimeError(f"synthetic fill failed with code {rc}")
        return
    rc = rc or g.bqgen_fill_uniform_bf16(key(w, fam, layer, T_SCALE, expert, m), *w.scale_range, ng, s_ptr, stream)
    rc = rc or g.bqgen_fill_uniform_bf16(key(w, fam, layer, T_BIAS, expert, m), *w.bias_range, ng, b_ptr, stream)
    if rc != 0:
        raise RuntimeError(f"synthetic fill failed with code {rc}")
