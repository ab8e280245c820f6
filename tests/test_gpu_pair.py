"""The two-launch decode of one token (router, top-K and gate/up + SwiGLU in one kernel, whose
blocks hand the logits to each other inside the launch; then the down + combine kernel) against
the three-kernel chain, bit for bit, and against the fp64 oracle.

Both paths add the same products in the same order, so their outputs and indices must be equal
bitwise; the oracle bar is the usual one (bit-exact top-K, outputs within 2e-3*max|oracle| + 1e-5).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_quantized_expert_gemv_amd as bq
import synth
from synth.gpu_layers import DeviceLayer
from tests._ref import Reference, assert_close, spread

pytestmark = pytest.mark.gpu

DEC4, DEC2 = synth.WORKLOADS["decode4"], synth.WORKLOADS["decode2"]


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def dec4(gpu_device):
    _log("build decode4 layer (512 experts, 4-bit)")
    L = DeviceLayer(DEC4)
    torch.cuda.synchronize()
    return L, Reference(DEC4)


@pytest.fixture(scope="module")
def dec2(gpu_device):
    _log("build decode2 layer (512 experts, 2-bit)")
    L = DeviceLayer(DEC2)
    torch.cuda.synchronize()
    return L, Reference(DEC2)


def _chain(desc):
    d = bq.moe_layer_t.from_buffer_copy(desc)
    d.flags |= bq.MOE_FLAG_DECODE_CHAIN
    return d


def _run_tokens(desc, X, ws, n):
    N = X.shape[0]
    out = torch.empty_like(X)
    idx = torch.empty(N, desc.top_k, dtype=torch.int32, device="cuda")
    for t in range(N):
        bq.moe_layer_forward(desc, X[t], X[t], 1, out[t], idx[t], ws, n)
    torch.cuda.synchronize()
    return out, idx


@pytest.mark.parametrize("which", ["dec4", "dec2"])
def test_plan(which, request):
    L, _ = request.getfixturevalue(which)
    assert bq.moe_layer_plan(L.desc, 1) == bq.MOE_PLAN_PAIR
    assert bq.moe_layer_plan(_chain(L.desc), 1) == bq.MOE_PLAN_CHAIN
    assert bq.moe_layer_plan(L.desc, 2) == bq.MOE_PLAN_CHAIN
    assert bq.moe_layer_plan(L.desc, bq.MOE_PREFILL_MIN_TOKENS) == bq.MOE_PLAN_PREFILL


@pytest.mark.parametrize("which", ["dec4", "dec2"])
def test_pair_equals_chain_and_oracle(which, request):
    """128 tokens spread over the workload's 1000, each as a single-token call through both paths on
    their own workspaces: equal bit for bit; 8 of them against the oracle."""
    L, ref = request.getfixturevalue(which)
    w = L.w
    toks = spread(w.tokens, 128)
    X = torch.from_numpy(np.stack([synth.tokens_x(w, t, 1)[0] for t in toks])).cuda()
    n = bq.moe_workspace_bytes(L.desc, 1)
    ws_a = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros(n, dtype=torch.uint8, device="cuda")
    _log(f"{w.name}: {len(toks)} tokens, two launches and the chain")
    out_a, idx_a = _run_tokens(L.desc, X, ws_a, n)
    out_b, idx_b = _run_tokens(_chain(L.desc), X, ws_b, n)
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), "outputs differ in some bit"
    # the sync region's call counter advanced once per two-launch call
    assert int(ws_a[:4].view(torch.int32).item()) == len(toks)
    xs = X.cpu().numpy().astype(np.float64)
    on, ix = out_a.cpu().numpy(), idx_a.cpu().numpy()
    for i in spread(len(toks), 8):
        r = ref.token(xs[i])
        assert list(ix[i]) == list(r.idx), f"token {toks[i]}"
        assert_close(on[i], r.out, f"out[{toks[i]}]")


def test_pair_graph_replays(dec4):
    """32 calls captured in a HIP graph, replayed 3 times with eager two-launch calls on the same
    workspace in between: every replay equals the chain's results."""
    L, _ = dec4
    w = L.w
    N = 32
    X = torch.from_numpy(synth.tokens_x(w, 500, N)).cuda()
    n = bq.moe_workspace_bytes(L.desc, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    want, want_idx = _run_tokens(_chain(L.desc), X, torch.zeros(n, dtype=torch.uint8, device="cuda"), n)
    out = torch.empty_like(X)
    idx = torch.empty(N, w.top_k, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for t in range(N):
            bq.moe_layer_forward(L.desc, X[t], X[t], 1, out[t], idx[t], ws, n, stream=s)
    for rep in range(3):
        out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), want.view(torch.int32)) and torch.equal(idx, want_idx), f"replay {rep}"
        eager, _ = _run_tokens(L.desc, X[:4], ws, n)  # eager calls between replays advance the counter
        assert torch.equal(eager.view(torch.int32), want[:4].view(torch.int32))


def test_marked_sync_region_writes_nan_until_zeroed(dec4):
    """A sync region marked by a call that gave up (the mark set here from the host) makes every
    two-launch call write NaN and nothing else; zeroing the region restores normal calls."""
    L, _ = dec4
    w = L.w
    X = torch.from_numpy(synth.tokens_x(w, 7, 2)).cuda()
    n = bq.moe_workspace_bytes(L.desc, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    want, want_idx = _run_tokens(_chain(L.desc), X, torch.zeros(n, dtype=torch.uint8, device="cuda"), n)
    ws[128:132].view(torch.int32).fill_(1)
    out = torch.zeros_like(X)
    idx = torch.full((2, w.top_k), -7, dtype=torch.int32, device="cuda")
    for t in range(2):
        bq.moe_layer_forward(L.desc, X[t], X[t], 1, out[t], idx[t], ws, n)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    assert (idx == -7).all()
    ws[:bq.MOE_WS_SYNC_BYTES].zero_()
    got, got_idx = _run_tokens(L.desc, X, ws, n)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)) and torch.equal(got_idx, want_idx)


def test_pair_mxfp4_equals_chain_and_oracle(gpu_device):
    """The MXFP4 top-6 layer (decodemx): 64 spread tokens through both plans, equal bit for bit; 6 of
    them against the oracle."""
    w = synth.WORKLOADS["decodemx"]
    _log("build decodemx layer (512 experts, MXFP4)")
    L = DeviceLayer(w)
    ref = Reference(w)
    assert bq.moe_layer_plan(L.desc, 1) == bq.MOE_PLAN_PAIR
    toks = spread(w.tokens, 64)
    X = torch.from_numpy(np.stack([synth.tokens_x(w, t, 1)[0] for t in toks])).cuda()
    n = bq.moe_workspace_bytes(L.desc, 1)
    out_a, idx_a = _run_tokens(L.desc, X, torch.zeros(n, dtype=torch.uint8, device="cuda"), n)
    out_b, idx_b = _run_tokens(_chain(L.desc), X, torch.zeros(n, dtype=torch.uint8, device="cuda"), n)
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32)), "outputs differ in some bit"
    xs = X.cpu().numpy().astype(np.float64)
    on, ix = out_a.cpu().numpy(), idx_a.cpu().numpy()
    for i in spread(len(toks), 6):
        r = ref.token(xs[i])
        assert list(ix[i]) == list(r.idx), f"token {toks[i]}"
        assert_close(on[i], r.out, f"out[{toks[i]}]")


def test_pair_stack_equals_chain_and_oracle(gpu_device):
    """Three layers at the 60-layer stack's shapes (RMS norm before layers 1 and 2): 6 single-token
    stack calls through both plans, equal bit for bit in every layer's indices and the output; 2 of
    them against the oracle's stack."""
    import oracle
    from tests._ref import STACK_EPS

    w = synth.WORKLOADS["stack60"]
    nl = 3
    _log(f"build {nl} layers at stack60 shapes")
    layers = [DeviceLayer(w, l) for l in range(nl)]
    descs = [L.desc for L in layers]
    chains = [_chain(d) for d in descs]
    X = torch.from_numpy(synth.tokens_x(w, 0, 6)).cuda()
    n = bq.moe_stack_workspace_bytes(descs[0], 1)
    res = []
    for ds in (descs, chains):
        ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(X)
        idx = torch.empty(6, nl, 1, w.top_k, dtype=torch.int32, device="cuda")
        for t in range(6):
            bq.moe_stack_forward(ds, STACK_EPS, X[t], 1, out[t], idx[t], ws, n)
        torch.cuda.synchronize()
        res.append((out, idx))
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][0].view(torch.int32), res[1][0].view(torch.int32)), "outputs differ in some bit"
    refs = [Reference(w, l) for l in range(nl)]
    xs = X.cpu().numpy().astype(np.float64)
    for t in (0, 5):
        r = oracle.stack(xs[t], [(q.router, q.gate, q.expert, q.shared) for q in refs], w.top_k, w.group, STACK_EPS)
        for l in range(nl):
            assert list(res[0][1][t, l, 0].cpu().numpy()) == list(r.idx[l]), f"token {t} layer {l}"
        assert_close(res[0][0][t].cpu().numpy(), r.out, f"stack out[{t}]")


def test_workspace_init_clears_a_garbage_region(dec4):
    """A workspace filled with garbage, cleared by moe_workspace_init: the same results as a
    workspace allocated zeroed."""
    L, _ = dec4
    w = L.w
    X = torch.from_numpy(synth.tokens_x(w, 3, 4)).cuda()
    n = bq.moe_workspace_bytes(L.desc, 1)
    want, want_idx = _run_tokens(L.desc, X, torch.zeros(n, dtype=torch.uint8, device="cuda"), n)
    ws = torch.full((n,), 0xA7, dtype=torch.uint8, device="cuda")
    bq.moe_workspace_init(ws, n)
    got, got_idx = _run_tokens(L.desc, X, ws, n)
    assert torch.equal(got_idx, want_idx)
    assert torch.equal(got.view(torch.int32), want.view(torch.int32))
    assert int(ws[:bq.MOE_WS_SYNC_BYTES].count_nonzero().item()) > 0  # the calls use the region again
