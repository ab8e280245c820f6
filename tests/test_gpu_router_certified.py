"""GPU parity of the certified router: many tokens, no logits requested.

From MOE_ROUTER_CERTIFIED_MIN_TOKENS tokens, moe_router without a logits buffer takes approximate
logits from bf16 MFMAs, and so does moe_layer_forward's prefill. Every row that the approximation's
error bound cannot rule out is then recomputed in fp64. The choice must be the top-K of the fp64
logits, so the bar is exact:
- the indices equal, for every token, those of the same entry point's fp64 path (moe_router with a
  logits buffer) and those of the oracle's top-K;
- the weights and the shared gate agree with the fp64 path to fp32 rounding.

The inputs are built to defeat the approximation:
- router rows in pairs one bf16 ulp apart in one element, so the logits are far closer than the
  bound;
- exact duplicate rows, where ties go to the lower index;
- a zero token, where every row ties and every row is recomputed;
- a token near the fp32 maximum, whose bf16 split overflows, so every row takes the non-finite
  fallback.
The shapes are ragged or at the edges: T not a multiple of the 32-token tile, E not a multiple of
the 128-row tile, hidden 256 (half a wave of chunks), hidden 8192 and 1024 experts with top-8.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_quantized_expert_gemv_amd as bq
import oracle
import synth
from synth.gpu_layers import DeviceLayer

pytestmark = pytest.mark.gpu

_4 = dict(bits=4, scale_range=(0.001, 0.01), bias_range=(-0.08, -0.005))
SHAPES = {
    "c4096": synth.Workload("c4096", 4096, 512, 64, 3, weight_family=21, x_family=21, **_4),
    "c1024e200": synth.Workload("c1024e200", 1024, 200, 64, 4, weight_family=22, x_family=22, **_4),
    "c256": synth.Workload("c256", 256, 16, 64, 2, has_shared=False, weight_family=23, x_family=23, **_4),
    "c8192": synth.Workload("c8192", 8192, 64, 64, 2, weight_family=24, x_family=24, **_4),
    "c512e1024": synth.Workload("c512e1024", 512, 1024, 64, 8, weight_family=25, x_family=25, **_4),
}
MIN_T = bq.MOE_ROUTER_CERTIFIED_MIN_TOKENS


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def layers(gpu_device):
    built = {}

    def get(name):
        if name not in built:
            _log(f"build layer {name}")
            built[name] = DeviceLayer(SHAPES[name])
            torch.cuda.synchronize()
        return built[name]

    yield get
    built.clear()
    torch.cuda.empty_cache()


def _route(L, x, with_logits):
    w = L.w
    T = x.shape[0]
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.top_k, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda") if w.has_shared else None
    lg = torch.empty(T, w.n_experts, dtype=torch.float64, device="cuda") if with_logits else None
    bq.moe_router(L.desc, x, T, idx, wt, g, lg, ws, n)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), wt.cpu().numpy(), None if g is None else g.cpu().numpy(),
            None if lg is None else lg.cpu().numpy())


def _check(L, x, router_u16, sample):
    """Certified vs fp64 path for every token; vs the oracle's top-K on the sampled tokens."""
    T = x.shape[0]
    i_c, w_c, g_c, _ = _route(L, x, with_logits=False)
    i_f, w_f, g_f, lg = _route(L, x, with_logits=True)
    for t in range(T):
        assert list(i_c[t]) == list(i_f[t]), f"token {t}: certified {i_c[t]} vs fp64 {i_f[t]}"
    assert np.max(np.abs(w_c - w_f)) <= 1e-6
    if g_c is not None:
        assert np.max(np.abs(g_c - g_f)) <= 1e-6
    xs = x.cpu().numpy().astype(np.float64)
    for t in sample:
        l_ref = oracle.router_logits(router_u16, xs[t])
        assert list(i_c[t]) == list(oracle.topk(l_ref, L.w.top_k)), f"token {t} vs oracle"
    return i_c, w_c


def _router_u16(L):
    return L.router.cpu().numpy().view(np.uint16).reshape(L.w.n_experts, L.w.hidden)


@pytest.mark.parametrize("name,T", [
    ("c4096", MIN_T), ("c4096", MIN_T + 1), ("c4096", 1000), ("c4096", 2048),
    ("c1024e200", MIN_T + 18), ("c256", MIN_T + 4), ("c8192", MIN_T + 4), ("c512e1024", MIN_T),
])
def test_certified_router_matches_fp64(layers, name, T):
    L = layers(name)
    _log(f"{name}: {T} tokens, certified vs fp64 router")
    x = torch.from_numpy(synth.tokens_x(L.w, 0, T)).cuda()
    sample = sorted({0, 1, 31, 32, T // 2, T - 2, T - 1})
    _check(L, x, _router_u16(L), sample)


@pytest.mark.parametrize("name", ["c4096", "c1024e200", "c512e1024"])
def test_certified_router_near_ties_and_duplicates(layers, name):
    """Rows 2i+1 copy rows 2i with one element one bf16 ulp apart (a logit gap of ~1e-4, far
    below the approximation's bound); the last 32 rows are exact copies of the 32 before them."""
    L = layers(name)
    w = L.w
    E, H = w.n_experts, w.hidden
    orig = L.router.clone()
    try:
        R = _router_u16(L).copy()
        rng = np.random.default_rng(5)
        for i in range(0, E - 1, 2):
            R[i + 1] = R[i]
            j = int(rng.integers(H))
            v = int(R[i, j])
            R[i + 1, j] = v + 1 if v & 0x7F != 0x7F else v - 1  # one ulp, same sign and exponent
        R[E - 32:] = R[E - 64:E - 32]
        L.router.copy_(torch.from_numpy(R.view(np.int16)).to(L.router.device))
        T = MIN_T + 32
        _log(f"{name}: near-tie router, {T} tokens")
        x = torch.from_numpy(synth.tokens_x(w, 500, T)).cuda()
        i_c, _ = _check(L, x, R, range(0, T, 9))
        for t in range(T):
            for e in i_c[t]:
                if e >= E - 32:  # a winning copy implies its twin (a lower index) won first
                    assert e - 32 in i_c[t] and list(i_c[t]).index(e - 32) < list(i_c[t]).index(e)
    finally:
        L.router.copy_(orig)
        torch.cuda.synchronize()


def test_certified_router_degenerate_tokens(layers):
    """A zero token (every logit 0: every row recomputed, the first K rows chosen with equal
    weights) and a token with one value near the fp32 maximum (its bf16 split overflows, so the
    token falls back to fp64 for every row), inside a batch of ordinary tokens."""
    L = layers("c4096")
    w = L.w
    T = MIN_T
    x_np = synth.tokens_x(w, 900, T)
    x_np[10] = 0.0
    x_np[77, 5] = np.float32(3.4e38)
    x = torch.from_numpy(x_np).cuda()
    _log(f"c4096: zero and overflow tokens in a batch of {T}")
    i_c, w_c = _check(L, x, _router_u16(L), [0, 10, 11, 76, 77, 78, T - 1])
    assert list(i_c[10]) == list(range(w.top_k))
    assert np.allclose(w_c[10], 1.0 / w.top_k, atol=1e-7)


def test_certified_router_bitwise_repeatable(layers):
    """Two calls on the same inputs give the same indices, weights and gate bit for bit: the
    approximation's partial sums, the candidate list and the fp64 recomputation all run in a fixed
    order."""
    L = layers("c4096")
    x = torch.from_numpy(synth.tokens_x(L.w, 3000, 1024)).cuda()
    _log("c4096: certified router twice on 1024 tokens")
    a = _route(L, x, with_logits=False)
    b = _route(L, x, with_logits=False)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("name", ["prefill4", "prefillmx"])
def test_certified_bound_margin(gpu_device, name):
    """The certified top-K trusts |approx - exact| <= kc |r_e| |x_t| + (|r_e| + 1) 2^-100. Over
    every token and every row of the 2048-token workloads, the measured error must stay below a
    quarter of that bound (exact = the oracle's fp64 logits)."""
    w = synth.WORKLOADS[name]
    L = DeviceLayer(w)
    T, E = w.tokens, w.n_experts
    xs = synth.tokens_x(w, 0, T)
    x = torch.from_numpy(xs).cuda()
    lg = torch.full((T, E + 1), float("nan"), dtype=torch.float64, device="cuda")
    kc = bq.moe_router_approx_logits(L.desc, x, T, lg)
    torch.cuda.synchronize()
    approx = lg.cpu().numpy()[:, :E]
    R = synth.router_weights(w, 0)
    x64 = xs.astype(np.float64)
    exact = np.stack([oracle.router_logits(R, x64[t]) for t in range(T)])
    rn = np.linalg.norm(synth.bf16_to_f32(R).astype(np.float64), axis=1)
    xn = np.linalg.norm(x64, axis=1)
    bound = kc * xn[:, None] * rn[None, :] + (rn[None, :] + 1.0) * 2.0 ** -100
    ratio = np.abs(approx - exact) / bound
    t, e = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    _log(f"{name}: kc {kc:.3e}; max |approx - exact| / bound = {ratio[t, e]:.4f} at token {t} row {e}; "
         f"mean {ratio.mean():.2e}; 99.99th percentile {np.quantile(ratio, 0.9999):.4f}")
    assert np.all(np.isfinite(approx))
    assert ratio.max() < 0.25
