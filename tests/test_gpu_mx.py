"""GPU parity of MXFP4 expert layers (E2M1 codes, one E8M0 scale per 32, top-6 routing) against the
fp64 oracle, through the C ABI on an MI355X. From 48 tokens the layer runs the grouped path on the
scaled MX MFMA, with the activations as 3-term MXFP8 expansions.

Bar as for the affine layers: bit-exact top-K indices and dequantised weights; outputs within
2e-3*max|oracle| + 1e-5 per token vector.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_quantized_expert_gemv_amd as bq
import oracle
import synth
from synth.gpu_layers import DeviceLayer
from tests._ref import Reference, assert_close, check_topk_all, spread

pytestmark = pytest.mark.gpu

TINYMX, DECMX = synth.WORKLOADS["tinymx"], synth.WORKLOADS["decodemx"]


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def tinymx(gpu_device):
    _log("build tinymx layer")
    return DeviceLayer(TINYMX), Reference(TINYMX)


@pytest.fixture(scope="module")
def decmx(gpu_device):
    _log("build decodemx layer (512 MXFP4 experts)")
    L = DeviceLayer(DECMX)
    torch.cuda.synchronize()
    return L, Reference(DECMX)


def _ws(desc, T):
    n = bq.moe_workspace_bytes(desc, T)
    return torch.zeros(n, dtype=torch.uint8, device="cuda"), n


def _x(w, t0, n):
    return torch.from_numpy(synth.tokens_x(w, t0, n)).cuda()


@pytest.mark.parametrize("which", ["tinymx", "decmx"])
def test_mx_device_generation_and_pack_match_host(which, request):
    L, _ = request.getfixturevalue(which)
    w = L.w
    for e in [0, w.n_experts - 1, synth.SHARED] + ([137] if w.n_experts > 137 else []):
        ex = synth.expert_arrays(w, 0, e)
        blob = np.zeros(L.blob_bytes, dtype=np.uint8)
        bq.moe_pack_expert(w.hidden, w.inter, 4, 32, [m.q for m in ex.mats], [m.scale for m in ex.mats],
                           [None] * 3, blob)
        assert np.array_equal(L.expert_blob(e).cpu().numpy(), blob), f"expert {e}"


@pytest.mark.parametrize("which", ["tinymx", "decmx"])
def test_mx_dequant_bit_exact(which, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    for e in (0, 5, synth.SHARED):
        ex = ref.shared if e == synth.SHARED else ref.expert(e)
        for m, mat in enumerate(ex.mats):
            rows, cols = w.matrix_shape(m)
            W = oracle.dequant_mx(mat.q, mat.scale)
            out = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
            bq.moe_dequant(L.desc, e, m, 0, out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().astype(np.float64), W), f"expert {e} matrix {m}"


@pytest.mark.parametrize("which,T", [("tinymx", 4), ("decmx", 3)])
def test_mx_expert_ffn_and_combine(which, T, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    x = _x(w, 100, T)
    rng = np.random.default_rng(11)
    idx_np = rng.integers(0, w.n_experts, size=(T, w.top_k)).astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    NE = w.top_k + 1
    y = torch.empty(T, NE, w.hidden, dtype=torch.float32, device="cuda")
    ws, n = _ws(L.desc, T)
    bq.moe_expert_ffn(L.desc, x, T, idx, y, ws, n)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    yn = y.cpu().numpy()
    for t in range(T):
        for k, e in enumerate(list(idx_np[t]) + [synth.SHARED]):
            assert_close(yn[t, k], ref.expert_out(xs[t], int(e)), f"y[{t}][{k}]")


@pytest.mark.parametrize("which,t0,T", [("tinymx", 0, 1), ("tinymx", 1, 24), ("tinymx", 30, 64), ("tinymx", 3, 200),
                                         ("decmx", 0, 1), ("decmx", 500, 4), ("decmx", 700, 64), ("decmx", 0, 2048)])
def test_mx_layer_forward(which, t0, T, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    _log(f"{w.name}: layer forward tokens [{t0}, {t0 + T})")
    x = _x(w, t0, T)
    ws, n = _ws(L.desc, T)
    out = torch.empty_like(x)
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x, T, out, idx, ws, n)
    torch.cuda.synchronize()
    on, ix, xs = out.cpu().numpy(), idx.cpu().numpy(), x.cpu().numpy().astype(np.float64)
    check_topk_all(ref, xs, ix)
    for t in (range(T) if T <= 24 else spread(T, 16)):
        r = ref.token(xs[t])
        assert_close(on[t], r.out, f"out[{t0 + t}]")


def test_mx_decode_sequence_graph(decmx):
    """The benchmark's launch configuration: back-to-back T=1 calls in one HIP graph. Every token's
    top-K against the oracle's, outputs on 32 spread tokens, and two replays agree bitwise."""
    L, ref = decmx
    w = L.w
    N = w.tokens
    X = _x(w, 0, N)
    out = torch.empty_like(X)
    idx = torch.empty(N, w.top_k, dtype=torch.int32, device="cuda")
    ws, n = _ws(L.desc, 1)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for t in range(N):
            bq.moe_layer_forward(L.desc, X[t], X[t], 1, out[t], idx[t], ws, n, stream=s)
    g.replay()
    torch.cuda.synchronize()
    first, first_idx = out.clone(), idx.clone()
    out.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, first) and torch.equal(idx, first_idx), "replays differ"
    xs = X.cpu().numpy().astype(np.float64)
    on, ix = out.cpu().numpy(), idx.cpu().numpy()
    check_topk_all(ref, xs, ix)
    for t in spread(N, 32):
        r = ref.token(xs[t])
        assert_close(on[t], r.out, f"out[{t}]")
