"""GPU parity of the prefill (grouped, MFMA) path against the fp64 oracle.

Prefill runs when T >= MOE_PREFILL_MIN_TOKENS. Its bar is the decode path's bar:
- bit-exact top-K for every token;
- outputs within 2e-3*max|oracle| + 1e-5 per token;
- a prefill row equals the decode of the same token within the same tolerance.
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

TINY, DEC2, PRE4 = synth.WORKLOADS["tiny"], synth.WORKLOADS["decode2"], synth.WORKLOADS["prefill4"]


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def tiny(gpu_device):
    return DeviceLayer(TINY), Reference(TINY)


@pytest.fixture(scope="module")
def pre4(gpu_device):
    _log("build the 4-bit layer (512 experts) for prefill")
    L = DeviceLayer(PRE4)
    torch.cuda.synchronize()
    return L, Reference(PRE4)


def _forward(L, x, res=None):
    T = x.shape[0]
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(T, L.w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x if res is None else res, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("T", [bq.MOE_PREFILL_MIN_TOKENS, 100, 300, bq.MOE_ROUTER_CERTIFIED_MIN_TOKENS + 88])
def test_prefill_tiny_all_tokens(tiny, T):
    """Every token against the oracle, through each prefill router: per-token rows (48), the fp64
    GEMM (100, 300) and the certified router (600, with 8 experts: one 32-row tile, mostly
    clamped rows)."""
    L, ref = tiny
    x = torch.from_numpy(synth.tokens_x(TINY, 7, T)).cuda()
    out, idx = _forward(L, x)
    xs = x.cpu().numpy()
    for t in range(T):
        r = ref.token(xs[t])
        assert list(idx[t]) == list(r.idx), f"token {t}"
        assert_close(out[t], r.out, f"out[{t}]")
    counts = np.bincount(idx.reshape(-1), minlength=TINY.n_experts)
    assert counts.sum() == T * TINY.top_k


# token t -> factor applied to its synthetic x: far above fp16's largest value (65504), large
# enough that the SwiGLU outputs pass it while x does not, and far below fp16's normal range
_RANGE_SCALES = {0: 1e6, 1: 3e3, 2: 1e-6, 5: 2.5e4, 9: 1e-3}


@pytest.mark.parametrize("which,T", [("tiny", 64), ("pre4", 100), ("pre4", bq.MOE_ROUTER_CERTIFIED_MIN_TOKENS + 88)])
def test_prefill_fp16_range(which, T, request):
    """Prefill casts activations and SwiGLU outputs to fp16 for the MFMAs. Tokens whose x, or whose
    SwiGLU outputs, lie far outside fp16's range (or deep in its subnormals) must still meet the
    oracle's bar: every token's top-K, and outputs of the scaled tokens and 16 spread ones."""
    L, ref = request.getfixturevalue(which)
    w = L.w
    _log(f"{w.name}: fp16 range, T={T}")
    xs = synth.tokens_x(w, 3, T).copy()
    for t, f in _RANGE_SCALES.items():
        xs[t] *= np.float32(f)
    x = torch.from_numpy(xs).cuda()
    out, idx = _forward(L, x)
    x64 = xs.astype(np.float64)
    check_topk_all(ref, x64, idx)
    big_h = 0.0
    for t in sorted(set(_RANGE_SCALES) | set(spread(T, 16))):
        r = ref.token(x64[t])
        assert np.all(np.isfinite(r.out))
        if t == 1:
            ex = ref.expert(int(r.idx[0]))
            big_h = float(np.max(np.abs(oracle.expert(x64[t], ex, w.group, want_h=True)[1])))
        assert_close(out[t], r.out, f"out[{t}] (x scaled by {_RANGE_SCALES.get(t, 1.0):g})")
    assert np.max(np.abs(xs[1])) < 65504 < big_h, "token 1 must keep x inside fp16 and push h past it"


def test_prefill_tiny_residual_and_determinism(tiny):
    L, ref = tiny
    x = torch.from_numpy(synth.tokens_x(TINY, 0, 128)).cuda()
    res = torch.randn_like(x)
    a, ia = _forward(L, x, res)
    b, ib = _forward(L, x, res)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)
    for t in (0, 41, 127):
        r = ref.token(x[t].cpu().numpy(), res[t].cpu().numpy())
        assert_close(a[t], r.out)


def test_prefill4_full(pre4):
    """2048 tokens through the 4-bit layer: every token's top-K against the oracle's fp64 routing,
    outputs of 64 spread tokens (and the tile edges) against the oracle, and prefill rows against
    the decode path's rows."""
    L, ref = pre4
    T = PRE4.tokens
    x = torch.from_numpy(synth.tokens_x(PRE4, 0, T)).cuda()
    _log("prefill4: 2048-token forward")
    out, idx = _forward(L, x)
    xs = x.cpu().numpy().astype(np.float64)
    _log("prefill4: oracle routing for every token")
    check_topk_all(ref, xs, idx)
    counts = np.bincount(idx.reshape(-1), minlength=PRE4.n_experts)
    _log(f"prefill4: tokens per expert min {counts.min()} mean {counts.mean():.1f} max {counts.max()}, "
         f"untouched {(counts == 0).sum()}")
    assert counts.sum() == T * PRE4.top_k
    sample = [0, 1, 17, 500, 1023, 1024, 2046, 2047]
    _log("prefill4: oracle outputs of 64 spread tokens")
    for t in sorted(set(sample) | set(spread(T, 64))):
        r = ref.token(xs[t])
        assert_close(out[t], r.out, f"prefill out[{t}]")
    # the same tokens through the decode path (T=1 calls)
    n = bq.moe_workspace_bytes(L.desc, 1)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for t in sample:
        o1 = torch.empty(1, PRE4.hidden, device="cuda")
        bq.moe_layer_forward(L.desc, x[t:t + 1], x[t:t + 1], 1, o1, None, ws, n)
        torch.cuda.synchronize()
        assert_close(out[t], o1[0].cpu().numpy(), f"prefill vs decode [{t}]")


def test_prefill_expert_ffn_and_router(pre4):
    L, ref = pre4
    T = 96
    x = torch.from_numpy(synth.tokens_x(PRE4, 3000, T)).cuda()
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, PRE4.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, PRE4.top_k, device="cuda")
    g = torch.empty(T, device="cuda")
    bq.moe_router(L.desc, x, T, idx, wt, g, None, ws, n)
    y = torch.empty(T, PRE4.top_k + 1, PRE4.hidden, device="cuda")
    bq.moe_expert_ffn(L.desc, x, T, idx, y, ws, n)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    ix, yn = idx.cpu().numpy(), y.cpu().numpy()
    for t in range(T):
        lg = oracle.router_logits(ref.router, xs[t])
        assert list(ix[t]) == list(oracle.topk(lg, PRE4.top_k)), f"token {t}"
    for t in (0, 50, 95):
        for k, e in enumerate(list(ix[t]) + [synth.SHARED]):
            assert_close(yn[t, k], ref.expert_out(xs[t], int(e)), f"y[{t}][{k}]")


def test_prefill_2bit(gpu_device):
    L = DeviceLayer(DEC2)
    ref = Reference(DEC2)
    T = 128
    x = torch.from_numpy(synth.tokens_x(DEC2, 0, T)).cuda()
    out, idx = _forward(L, x)
    xs = x.cpu().numpy()
    for t in (0, 63, 127):
        r = ref.token(xs[t])
        assert list(idx[t]) == list(r.idx)
        assert_close(out[t], r.out, f"2-bit prefill out[{t}]")


def test_prefill_duplicate_router_rows_tie_to_lower_index(gpu_device):
    """Equal router rows give bitwise-equal fp64 logits in the router GEMM, and the top-K keeps the
    lower expert index, as the oracle's sort does, for every token of a prefill batch."""
    L = DeviceLayer(TINY)
    ref = Reference(TINY)
    T = bq.MOE_PREFILL_MIN_TOKENS
    x = torch.from_numpy(synth.tokens_x(TINY, 11, T)).cuda()
    xs = x.cpu().numpy().astype(np.float64)
    best = int(np.argmax(oracle.router_logits(ref.router, xs[0])))
    R = ref.router.copy()
    for r in (2, 5):
        R[r] = R[best]
    ref.router = R
    L.router.copy_(torch.from_numpy(R.view(np.int16)))
    out, idx = _forward(L, x)
    tied_tokens = 0
    for t in range(T):
        want = oracle.topk(oracle.router_logits(R, xs[t]), TINY.top_k)
        assert list(idx[t]) == list(want), f"token {t}"
        tied_tokens += len({best, 2, 5} & set(want)) >= 2
    assert tied_tokens >= 1  # the tie decides at least token 0's choice
    for t in (0, 31, T - 1):
        assert_close(out[t], ref.token(xs[t]).out, f"out[{t}]")


@pytest.mark.parametrize("which,T", [("tiny", bq.MOE_ROUTER_CERTIFIED_MIN_TOKENS + 88),
                                     ("pre4", bq.MOE_ROUTER_CERTIFIED_MIN_TOKENS)])
def test_prefill_graph_replays_match_eager(which, T, request):
    """One prefill call captured in a HIP graph: its shared expert runs on the library's side stream,
    forked from and joined back to the caller's stream, so the capture holds both. Three replays,
    with eager work on the device between them, each equal the eager call bit for bit."""
    L, _ = request.getfixturevalue(which)
    w = L.w
    _log(f"{w.name}: graph of one {T}-token prefill call")
    x = torch.from_numpy(synth.tokens_x(w, 4000, T)).cuda()
    eager, eager_idx = _forward(L, x)
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bq.moe_layer_forward(L.desc, x, x, T, out, idx, ws, n, stream=s)
    for rep in range(3):
        out.fill_(float(rep + 1))
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {rep}"
        assert np.array_equal(idx.cpu().numpy(), eager_idx), f"replay {rep}"
        _forward(L, x[: T // 2].contiguous())  # eager work between replays
