"""The C-ABI library without a GPU: it loads, exports every declared symbol, sizes and packs blobs,
and rejects bad arguments on the host before any HIP call (CPU only)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_expert_gemv_amd as bq
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    syms = declared_symbols()
    assert len(syms) >= 12
    L = bq.lib()
    for s in syms:
        assert hasattr(L, s), f"{s} declared in moe.h but not exported"
    assert set(syms) == set(bq.SIGNATURES), "binding and header disagree"


def test_no_oracle_in_product():
    """The product package and library never reference the oracle."""
    pkg = os.path.join(ROOT, "bit_quantized_expert_gemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "oracle/" not in txt and "liboracle" not in txt, f


def test_blob_bytes_closed_form():
    for H, I in ((256, 128), (4096, 1024), (1024, 4096), (512, 64)):
        for bits in (2, 4):
            n = 3 * H * I
            assert bq.moe_blob_bytes(H, I, bits) == n * bits // 8 + (n // 64) * 4
    assert bq.moe_blob_bytes(4096, 1024, 4) == 7_077_888
    assert bq.moe_blob_bytes(4096, 1024, 2) == 3_932_160
    assert bq.moe_blob_bytes(256, 128, 4) == 55_296
    assert bq.moe_blob_bytes(4096, 1024, 3) == 0
    # MXFP4: 4-bit codes plus one E8M0 byte per block of 32
    for H, I in ((256, 128), (4096, 1024)):
        n = 3 * H * I
        assert bq.moe_blob_bytes(H, I, 4, 32) == n // 2 + n // 32
    assert bq.moe_blob_bytes(4096, 1024, 4, 32) == 6_684_672
    assert bq.moe_blob_bytes(4096, 1024, 2, 32) == 0
    assert bq.moe_blob_bytes(4096, 1024, 4, 16) == 0
    assert bq.moe_blob_bytes(100, 1024, 4) == 0


def _unpack_codes(raw: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Independent unpacking of the blob's code bytes: element c sits at byte c*bits/8, lowest bits first."""
    per = 8 // bits
    fields = [(raw >> (bits * j)) & ((1 << bits) - 1) for j in range(per)]
    return np.stack(fields, axis=1).reshape(-1)[:n]


@pytest.mark.parametrize("name", ["tiny", "decode2"])
def test_host_pack_roundtrip(name):
    w = synth.WORKLOADS[name]
    if name == "decode2":  # keep the CPU test small: a reduced-width layer with the 2-bit recipe
        w = synth.Workload("small2", 512, 4, 128, 2, bits=2, scale_range=w.scale_range, bias_range=w.bias_range)
    ex = synth.expert_arrays(w, 0, 1)
    H, I = w.hidden, w.inter
    blob = np.zeros(bq.moe_blob_bytes(H, I, w.bits), dtype=np.uint8)
    bq.moe_pack_expert(H, I, w.bits, 64, [m.q for m in ex.mats], [m.scale for m in ex.mats],
                       [m.bias for m in ex.mats], blob)
    cb = I * H * w.bits // 8
    ng = I * H // 64
    for m, mat in enumerate(ex.mats):
        codes = _unpack_codes(blob[m * cb:(m + 1) * cb], w.bits, I * H)
        assert np.array_equal(codes, mat.q.reshape(-1))
        sb = blob[3 * cb + m * ng * 4: 3 * cb + (m + 1) * ng * 4].view(np.uint32)
        assert np.array_equal((sb & 0xFFFF).astype(np.uint16), mat.scale.reshape(-1))
        assert np.array_equal((sb >> 16).astype(np.uint16), mat.bias.reshape(-1))


def test_host_pack_roundtrip_mx():
    w = synth.WORKLOADS["tinymx"]
    ex = synth.expert_arrays(w, 0, 1)
    H, I = w.hidden, w.inter
    blob = np.zeros(bq.moe_blob_bytes(H, I, 4, 32), dtype=np.uint8)
    bq.moe_pack_expert(H, I, 4, 32, [m.q for m in ex.mats], [m.scale for m in ex.mats], [None] * 3, blob)
    cb, nb = I * H // 2, I * H // 32
    for m, mat in enumerate(ex.mats):
        assert np.array_equal(_unpack_codes(blob[m * cb:(m + 1) * cb], 4, I * H), mat.q.reshape(-1))
        assert np.array_equal(blob[3 * cb + m * nb: 3 * cb + (m + 1) * nb], mat.scale.reshape(-1).astype(np.uint8))
    big = [m.scale.copy() for m in ex.mats]
    big[1][0, 0] = 256
    with pytest.raises(bq.MoeError) as e:
        bq.moe_pack_expert(H, I, 4, 32, [m.q for m in ex.mats], big, [None] * 3, blob)
    assert e.value.code == bq.MOE_EINVAL


def test_host_pack_rejects_wide_codes():
    H, I = 256, 64
    q = [np.zeros(H * I, np.uint8) for _ in range(3)]
    s = [np.zeros(H * I // 64, np.uint16) for _ in range(3)]
    q[2][17] = 4
    blob = np.zeros(bq.moe_blob_bytes(H, I, 2), np.uint8)
    with pytest.raises(bq.MoeError) as e:
        bq.moe_pack_expert(H, I, 2, 64, q, s, s, blob)
    assert e.value.code == bq.MOE_EINVAL


FAKE = 1 << 40  # a 256-aligned address that validation never dereferences


def _layer(**kw):
    base = dict(hidden=4096, inter=1024, n_experts=512, top_k=3, bits=4, experts=FAKE,
                expert_stride=7_077_888, router=FAKE, shared_blob=FAKE, shared_gate=FAKE)
    base.update(kw)
    return bq.make_layer(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(bits=3), bq.MOE_EUNSUPPORTED),
    (dict(group=16), bq.MOE_EUNSUPPORTED),
    (dict(hidden=3000), bq.MOE_EUNSUPPORTED),
    (dict(hidden=128), bq.MOE_EUNSUPPORTED),
    (dict(inter=96), bq.MOE_EUNSUPPORTED),
    (dict(n_experts=2048), bq.MOE_EUNSUPPORTED),
    (dict(top_k=9), bq.MOE_EUNSUPPORTED),
    (dict(top_k=0), bq.MOE_EUNSUPPORTED),
    (dict(n_experts=2, top_k=3), bq.MOE_EUNSUPPORTED),
    (dict(experts=0), bq.MOE_EINVAL),
    (dict(experts=FAKE + 16), bq.MOE_EINVAL),
    (dict(expert_stride=7_077_888 - 256), bq.MOE_EINVAL),
    (dict(expert_stride=7_077_888 + 8), bq.MOE_EINVAL),
    (dict(router=0), bq.MOE_EINVAL),
    (dict(shared_gate=FAKE + 2), bq.MOE_EINVAL),
    (dict(flags=3), bq.MOE_EUNSUPPORTED),
    (dict(flags=-1), bq.MOE_EUNSUPPORTED),
    (dict(flags=12), bq.MOE_EUNSUPPORTED),
    (dict(flags=7), bq.MOE_EUNSUPPORTED),
    (dict(flags=8), bq.MOE_EUNSUPPORTED),
    (dict(bits=2, group=32), bq.MOE_EUNSUPPORTED),
    (dict(group=32, expert_stride=6_684_672 + 256, flags=1), bq.MOE_EUNSUPPORTED),
])
def test_layer_validation(kw, code):
    layer = _layer(**kw)
    if "shared_gate" in kw and kw["shared_gate"] == FAKE + 2:
        pass
    rc = bq.lib().moe_layer_forward(ctypes.byref(layer), FAKE, FAKE, 1, FAKE + 4096, None, FAKE, 1 << 30, None)
    assert rc == code, bq.moe_last_error()
    assert bq.moe_last_error() != ""


def test_call_validation():
    L = bq.lib()
    layer = _layer()
    ref = ctypes.byref(layer)
    need = bq.moe_workspace_bytes(layer, 1)
    assert need > 0
    # workspace too small
    assert L.moe_layer_forward(ref, FAKE, FAKE, 1, FAKE + 4096, None, FAKE, need - 1, None) == bq.MOE_ENOSPC
    # misaligned activations / workspace, aliasing, negative T
    assert L.moe_layer_forward(ref, FAKE + 4, FAKE, 1, FAKE + 4096, None, FAKE, need, None) == bq.MOE_EINVAL
    assert L.moe_layer_forward(ref, FAKE, FAKE, 1, FAKE + 4096, None, FAKE + 64, need, None) == bq.MOE_EINVAL
    assert L.moe_layer_forward(ref, FAKE, FAKE, 1, FAKE, None, FAKE, need, None) == bq.MOE_EINVAL
    assert L.moe_layer_forward(ref, FAKE, FAKE, -1, FAKE + 4096, None, FAKE, need, None) == bq.MOE_EINVAL
    # T == 0 is a no-op that touches nothing
    assert L.moe_layer_forward(ref, None, None, 0, None, None, None, 0, None) == bq.MOE_OK
    assert L.moe_router(ref, FAKE, 1, None, FAKE, None, None, FAKE, need, None) == bq.MOE_EINVAL
    assert L.moe_expert_ffn(ref, FAKE, 1, None, FAKE, FAKE, need, None) == bq.MOE_EINVAL
    assert L.moe_combine(ref, FAKE, FAKE, FAKE, None, 1, FAKE, None) == bq.MOE_EINVAL
    assert L.moe_dequant(ref, 512, 0, 0, FAKE, None) == bq.MOE_EINVAL
    assert L.moe_dequant(ref, 0, 3, 0, FAKE, None) == bq.MOE_EINVAL
    assert L.moe_dequant(ref, 0, 0, 2, FAKE, None) == bq.MOE_EINVAL
    no_shared = _layer(shared_blob=None, shared_gate=None)
    assert L.moe_dequant(ctypes.byref(no_shared), -1, 0, 0, FAKE, None) == bq.MOE_EINVAL
    # an MXFP4 prefill whose activation planes would pass 2^31 bytes is refused before any HIP call
    mx = _layer(group=32, expert_stride=6_684_672 + 256, top_k=6)
    big = 180_000  # 3 * T * 4096 >= 2^31
    assert L.moe_layer_forward(ctypes.byref(mx), FAKE, FAKE, big, FAKE + (1 << 36), None, FAKE, 1 << 62,
                               None) == bq.MOE_EUNSUPPORTED
    assert "2^31" in bq.moe_last_error()
    # the stack: mismatched layers, bad eps, small workspace
    other = _layer(top_k=2)
    arr = (bq.moe_layer_t * 2)(layer, other)
    assert L.moe_stack_forward(arr, 2, 1e-6, FAKE, 1, FAKE + 4096, None, FAKE, 1 << 30, None) == bq.MOE_EINVAL
    arr = (bq.moe_layer_t * 2)(layer, layer)
    assert L.moe_stack_forward(arr, 2, -1.0, FAKE, 1, FAKE + 4096, None, FAKE, 1 << 30, None) == bq.MOE_EINVAL
    sneed = bq.moe_stack_workspace_bytes(layer, 1)
    assert sneed > need
    assert L.moe_stack_forward(arr, 2, 1e-6, FAKE, 1, FAKE + 4096, None, FAKE, sneed - 1, None) == bq.MOE_ENOSPC
    assert L.moe_stack_forward(arr, 0, 1e-6, FAKE, 1, FAKE + 4096, None, FAKE, sneed, None) == bq.MOE_EINVAL
    # layers that differ in format or dequant form are refused before any launch: an affine layer 0
    # with an MXFP4 layer 1 would otherwise read layer 1's pool with affine offsets
    mx = _layer(group=32, bits=4, expert_stride=6_684_672 + 256)
    for second in (mx, _layer(flags=1), _layer(flags=2)):
        arr = (bq.moe_layer_t * 2)(layer, second)
        assert L.moe_stack_forward(arr, 2, 1e-6, FAKE, 1, FAKE + 4096, None, FAKE, 1 << 30, None) == bq.MOE_EINVAL
        assert "group" in bq.moe_last_error()


def test_noalloc_validation():
    """The no-allocation entry point checks its arguments and its fixed scratch size before any HIP
    call, so these run without a GPU."""
    L = bq.lib()
    layer = _layer()
    ref = ctypes.byref(layer)
    assert L.moe_layer_forward_noalloc(ref, None, None, 0, None, None, None) == bq.MOE_OK
    assert L.moe_layer_forward_noalloc(ref, FAKE + 4, FAKE, 1, FAKE + 4096, None, None) == bq.MOE_EINVAL
    assert L.moe_layer_forward_noalloc(ref, FAKE, FAKE, 1, FAKE, None, None) == bq.MOE_EINVAL
    assert L.moe_layer_forward_noalloc(ref, FAKE, FAKE, -1, FAKE + 4096, None, None) == bq.MOE_EINVAL
    big = next(T for T in range(64, 4096, 16) if bq.moe_workspace_bytes(layer, T) > bq.MOE_NOALLOC_SCRATCH_BYTES)
    assert bq.moe_workspace_bytes(layer, big - 16) <= bq.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_layer_forward_noalloc(ref, FAKE, FAKE, big, FAKE + (1 << 32), None, None) == bq.MOE_ENOSPC
    assert "MOE_NOALLOC_SCRATCH_BYTES" in bq.moe_last_error()


def test_workspace_monotone():
    layer = _layer()
    sizes = [bq.moe_workspace_bytes(layer, t) for t in (1, 2, 64, 2048)]
    assert sizes == sorted(sizes) and sizes[0] % 256 == 0
    bad = _layer(bits=3)
    assert bq.moe_workspace_bytes(bad, 1) == 0


def test_strerror():
    for c in (0, -1, -2, -3, -4, -5):
        assert bq.moe_strerror(c) != "unknown error"
    assert bq.moe_strerror(-99) == "unknown error"


def test_binding_constants_match_header():
    """The binding's copies of the header's numeric #defines (limits, status codes) agree with it."""
    import re
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")).read()
    found = dict(re.findall(r"^#define\s+(MOE_[A-Z0-9_]+)\s+\(?(-?\d+)\)?\s*$", text, flags=re.M))
    assert {"MOE_MAX_TOP_K", "MOE_MAX_EXPERTS", "MOE_PREFILL_MIN_TOKENS", "MOE_OK"} <= set(found)
    for name, value in found.items():
        assert hasattr(bq, name), name
        assert getattr(bq, name) == int(value), name


def test_layer_plan_validation():
    """moe_layer_plan: argument errors before any HIP call; the prefill from MOE_PREFILL_MIN_TOKENS
    tokens; the chain for several decode tokens and whenever MOE_FLAG_DECODE_CHAIN is set."""
    L = bq.lib()
    assert L.moe_layer_plan(None, 1) == bq.MOE_EINVAL
    assert L.moe_layer_plan(ctypes.byref(_layer(bits=3)), 1) == bq.MOE_EUNSUPPORTED
    assert L.moe_layer_plan(ctypes.byref(_layer()), 0) == bq.MOE_EINVAL
    assert L.moe_layer_plan(ctypes.byref(_layer()), -3) == bq.MOE_EINVAL
    assert bq.moe_layer_plan(_layer(), bq.MOE_PREFILL_MIN_TOKENS) == bq.MOE_PLAN_PREFILL
    assert bq.moe_layer_plan(_layer(), 2) == bq.MOE_PLAN_CHAIN
    assert bq.moe_layer_plan(_layer(flags=bq.MOE_FLAG_DECODE_CHAIN), 1) == bq.MOE_PLAN_CHAIN
    # shapes the first kernel does not take stay on the chain, on any device
    for kw in (dict(hidden=2048), dict(inter=512, expert_stride=bq.moe_blob_bytes(4096, 512, 4)),
               dict(top_k=2), dict(shared_blob=None, shared_gate=None), dict(flags=bq.MOE_FLAG_DEQUANT_NAIVE)):
        kw2 = dict(kw)
        if kw2.pop("shared_blob", 1) is None:
            lay = bq.make_layer(4096, 1024, 512, 3, 4, FAKE, 7_077_888, FAKE)
        else:
            lay = _layer(**kw)
        assert bq.moe_layer_plan(lay, 1) == bq.MOE_PLAN_CHAIN, kw


def test_workspace_holds_the_sync_region():
    """Every workspace starts with the MOE_WS_SYNC_BYTES sync region, before the per-token buffers."""
    lay = _layer()
    n1, n2 = bq.moe_workspace_bytes(lay, 1), bq.moe_workspace_bytes(lay, 2)
    per_token = n2 - n1
    assert n1 - per_token >= bq.MOE_WS_SYNC_BYTES
    assert bq.moe_stack_workspace_bytes(lay, 1) > n1


def test_workspace_init_validation():
    """moe_workspace_init refuses a NULL or misaligned workspace and one smaller than the sync
    region, before any HIP call."""
    L = bq.lib()
    assert L.moe_workspace_init(None, 1 << 20, None) == bq.MOE_EINVAL
    assert L.moe_workspace_init(FAKE + 16, 1 << 20, None) == bq.MOE_EINVAL
    assert L.moe_workspace_init(FAKE, bq.MOE_WS_SYNC_BYTES - 256, None) == bq.MOE_ENOSPC


def test_build_flags():
    """Every HIP source is built for gfx950 without packed-fp32 instructions, and with the leading
    kernel arguments preloaded into SGPRs (the decode kernels' first requests depend on it)."""
    import bit_quantized_expert_gemv_amd._build as B
    f = B.HIP_FLAGS
    assert "--offload-arch=gfx950" in f
    i = f.index("-packed-fp32-ops")
    assert f[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
    assert any(x.startswith("-amdgpu-kernarg-preload-count=") for x in f)
    j = next(k for k, x in enumerate(f) if x.startswith("-amdgpu-kernarg-preload-count="))
    assert f[j - 1] == "-mllvm"
