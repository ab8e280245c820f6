"""GPU parity of layers without a shared expert (has_shared = 0) against the fp64 oracle.

The shared expert changes slot counts, the router's extra gate row, the combine and the
grouping's shared tiles, so every path runs here once without it: decode (one token and a
ragged handful), the router and expert entry points, and prefill with each of its three routers
(per-token rows below 96 tokens, the fp64 GEMM from 96, the certified bf16 router from 512, each
with a ragged last token tile), for the affine 4-bit format and for MXFP4. Bar as elsewhere: bit-exact top-K indices; outputs within
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
from tests._ref import Reference, assert_close

pytestmark = pytest.mark.gpu

NS4 = synth.Workload("noshared4", 256, 8, 128, 2, bits=4, has_shared=False, weight_family=9, x_family=9,
                     scale_range=(0.001, 0.01), bias_range=(-0.08, -0.005))
NSMX = synth.Workload("nosharedmx", 256, 8, 128, 3, bits=4, group=32, fmt="mxfp4", has_shared=False,
                      weight_family=10, x_family=10)


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def ns4(gpu_device):
    _log("build a 4-bit layer without a shared expert")
    return DeviceLayer(NS4), Reference(NS4)


@pytest.fixture(scope="module")
def nsmx(gpu_device):
    _log("build an MXFP4 layer without a shared expert")
    return DeviceLayer(NSMX), Reference(NSMX)


def _x(w, t0, n):
    return torch.from_numpy(synth.tokens_x(w, t0, n)).cuda()


def _forward(L, x):
    T = x.shape[0]
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(T, L.w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def test_descriptor_has_no_shared_expert(ns4, nsmx):
    for L, _ in (ns4, nsmx):
        assert L.desc.has_shared == 0 and L.shared is None and L.shared_gate is None


@pytest.mark.parametrize("which", ["ns4", "nsmx"])
@pytest.mark.parametrize("t0,T", [(0, 1), (3, 7), (20, 70), (100, 130), (300, 600)])
def test_layer_forward(which, t0, T, request):
    """T = 1 and 7 run the decode path, 70 the prefill path with per-token router rows, 130 the
    prefill path with the fp64 router GEMM (four full token tiles and a ragged one of 2), and 600
    the prefill path with the certified router (no shared-gate row to recompute)."""
    L, ref = request.getfixturevalue(which)
    w = L.w
    _log(f"{w.name}: layer forward tokens [{t0}, {t0 + T})")
    x = _x(w, t0, T)
    out, idx = _forward(L, x)
    xs = x.cpu().numpy().astype(np.float64)
    check = range(T) if T <= 16 else sorted({0, 1, 31, 32, T // 2, T - 2, T - 1})
    for t in check:
        r = ref.token(xs[t])
        assert np.isnan(r.g)
        assert list(idx[t]) == list(r.idx), f"token {t0 + t}: idx {idx[t]} vs {r.idx} (margin {r.margin:.3e})"
        assert_close(out[t], r.out, f"out[{t0 + t}]")
    if T > 16:  # every token's routing, not only the sampled outputs
        for t in range(T):
            l_ref = oracle.router_logits(ref.router, xs[t])
            assert list(idx[t]) == list(oracle.topk(l_ref, w.top_k)), f"token {t0 + t}"


def test_router_without_shared_gate(ns4):
    L, ref = ns4
    w = L.w
    T = 5
    x = _x(w, 40, T)
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.top_k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, w.n_experts, dtype=torch.float64, device="cuda")
    bq.moe_router(L.desc, x, T, idx, wt, None, lg, ws, n)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    for t in range(T):
        l_ref = oracle.router_logits(ref.router, xs[t])
        assert np.allclose(lg[t].cpu().numpy(), l_ref, rtol=1e-12, atol=1e-12)
        i_ref = oracle.topk(l_ref, w.top_k)
        assert list(idx[t].cpu().numpy()) == list(i_ref)
        w_ref = oracle.route_weights(l_ref, i_ref)
        assert np.max(np.abs(wt[t].cpu().numpy() - w_ref)) <= 2e-3 * np.max(w_ref) + 1e-5


@pytest.mark.parametrize("T", [3, 64])
def test_expert_ffn_and_combine_without_shared(ns4, T):
    """K slots per token and no shared slot, through the decode (T = 3) and grouped (T = 64) paths;
    the combine takes no shared gate."""
    L, ref = ns4
    w = L.w
    x = _x(w, 200, T)
    rng = np.random.default_rng(11)
    idx_np = np.stack([rng.choice(w.n_experts, size=w.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    y = torch.empty(T, w.top_k, w.hidden, dtype=torch.float32, device="cuda")
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    bq.moe_expert_ffn(L.desc, x, T, idx, y, ws, n)
    wts = torch.from_numpy(rng.dirichlet(np.ones(w.top_k), size=T).astype(np.float32)).cuda()
    out = torch.empty(T, w.hidden, dtype=torch.float32, device="cuda")
    bq.moe_combine(L.desc, x, y, wts, None, T, out)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    yn = y.cpu().numpy()
    for t in (range(T) if T <= 8 else (0, 1, T // 2, T - 1)):
        ys = [ref.expert_out(xs[t], int(e)) for e in idx_np[t]]
        for k in range(w.top_k):
            assert_close(yn[t, k], ys[k], f"y[{t}][{k}]")
        o_ref = oracle.combine(xs[t], np.stack(ys), wts[t].cpu().numpy(), 0.0, None)
        assert_close(out[t].cpu().numpy(), o_ref, f"combine[{t}]")
