"""GPU parity of the decode stack (moe_stack_forward) against the fp64 oracle's stack.

Between layers the stack applies a unit-weight RMS norm (eps 1e-6); layer 0 reads the raw input.
Every layer's top-K must match the oracle's bit for bit; a mismatch fails and names the oracle's
fp64 margin (K-th minus (K+1)-th logit) at that layer. The oracle takes nothing from the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_quantized_expert_gemv_amd as bq
import oracle
import synth
from synth.gpu_layers import DeviceLayer
from tests._ref import STACK_EPS, Reference, assert_close, spread, stack_oracle_parallel

pytestmark = pytest.mark.gpu

EPS = STACK_EPS
TINYSTACK = synth.Workload("tinystack", 256, 8, 128, 2, bits=4, tokens=8, layers=4, weight_family=5, x_family=5)


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _oracle_layers(refs):
    return [(r.router, r.gate, r.expert, r.shared) for r in refs]


def _check_stack_token(t, ix_t, out_t, r, what):
    """ix_t [L][K] GPU choices, out_t [H]; r the oracle's StackResult for the same token."""
    for l in range(r.idx.shape[0]):
        assert list(ix_t[l]) == list(r.idx[l]), (
            f"{what} token {t} layer {l}: gpu {list(ix_t[l])} oracle {list(r.idx[l])} "
            f"fp64 margin {r.margin[l]:.3e}")
    assert_close(out_t, r.out, f"{what} out[{t}]")


def _run_stack(layers, x, T):
    w = layers[0].w
    n = bq.moe_stack_workspace_bytes(layers[0].desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(len(layers), T, w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_stack_forward([L.desc for L in layers], EPS, x, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


def test_stack_tiny(gpu_device):
    w = TINYSTACK
    layers = [DeviceLayer(w, l) for l in range(w.layers)]
    refs = [Reference(w, l) for l in range(w.layers)]
    x = torch.from_numpy(synth.tokens_x(w, 0, w.tokens)).cuda()
    out, idx = _run_stack(layers, x, w.tokens)
    xs = x.cpu().numpy()
    for t in range(w.tokens):
        r = oracle.stack(xs[t], _oracle_layers(refs), w.top_k, w.group, EPS)
        _check_stack_token(t, idx[:, t, :], out[t], r, "tinystack")


def test_stack_single_layer_equals_layer_forward(gpu_device):
    """Layer 0 of the stack reads the raw input, so a one-layer stack is exactly moe_layer_forward."""
    w = synth.WORKLOADS["decode4"]
    L = DeviceLayer(w)
    x = torch.from_numpy(synth.tokens_x(w, 0, 3)).cuda()
    out_s, idx_s = _run_stack([L], x, 3)
    n = bq.moe_workspace_bytes(L.desc, 3)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(3, w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x, 3, out, idx, ws, n)
    torch.cuda.synchronize()
    assert np.array_equal(out_s, out.cpu().numpy()) and np.array_equal(idx_s[0], idx.cpu().numpy())


def test_stack_graph_replays_match_oracle(gpu_device):
    """The stack captured in a HIP graph: every replay, with eager work between replays, matches the
    oracle's stack and the eager call's bits."""
    w = TINYSTACK
    layers = [DeviceLayer(w, l) for l in range(w.layers)]
    refs = [Reference(w, l) for l in range(w.layers)]
    x = torch.from_numpy(synth.tokens_x(w, 0, w.tokens)).cuda()
    xs = x.cpu().numpy()
    want = [oracle.stack(xs[t], _oracle_layers(refs), w.top_k, w.group, EPS) for t in range(w.tokens)]
    out0, idx0 = _run_stack(layers, x, w.tokens)
    n = bq.moe_stack_workspace_bytes(layers[0].desc, w.tokens)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(len(layers), w.tokens, w.top_k, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bq.moe_stack_forward([L.desc for L in layers], EPS, x, w.tokens, out, idx, ws, n, stream=s)
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        on, ix = out.cpu().numpy(), idx.cpu().numpy()
        for t in range(w.tokens):
            _check_stack_token(t, ix[:, t, :], on[t], want[t], f"replay {rep}")
        assert np.array_equal(on, out0) and np.array_equal(ix, idx0), f"replay {rep}"
        _run_stack(layers, x, w.tokens)  # eager work between replays


@pytest.mark.timeout(900)
def test_stack60_sequence(gpu_device):
    """The full 60-layer stack with every expert resident (about 218 GB), as 128 sequential
    single-token calls in one graph. 16 tokens spread over the 128 are checked against the oracle's
    stack: every layer's top-K and the output. The oracle runs in CPU worker processes while the
    GPU builds and runs the stack."""
    w = synth.WORKLOADS["stack60"]
    free, _ = torch.cuda.mem_get_info()
    need = w.layers * (w.n_experts + 1) * bq.moe_blob_bytes(w.hidden, w.inter, w.bits) + (8 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB free, have {free / 2**30:.0f} GiB")
    N = w.tokens
    xs = synth.tokens_x(w, 0, N)
    check = spread(N, 16)
    pool, futs = stack_oracle_parallel(w.name, w.layers, xs[check], workers=16)
    try:
        layers = []
        for l in range(w.layers):
            layers.append(DeviceLayer(w, l))
            if l % 10 == 9:
                torch.cuda.synchronize()
                _log(f"stack60: built {l + 1} layers")
        X = torch.from_numpy(xs).cuda()
        out = torch.empty_like(X)
        idx = torch.empty(N, w.layers, w.top_k, dtype=torch.int32, device="cuda")
        n = bq.moe_stack_workspace_bytes(layers[0].desc, 1)
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        descs = [L.desc for L in layers]
        s = torch.cuda.Stream()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for t in range(N):
                bq.moe_stack_forward(descs, EPS, X[t], 1, out[t], idx[t], ws, n, stream=s)
        g.replay()
        torch.cuda.synchronize()
        _log("stack60: graph replayed")
        on, ix = out.cpu().numpy(), idx.cpu().numpy()
        for t, f in zip(check, futs):
            r = f.result()
            _check_stack_token(t, ix[t], on[t], r, "stack60")
            _log(f"stack60: token {t} matches (min fp64 margin {r.margin.min():.2e})")
    finally:
        pool.shutdown(cancel_futures=True)
