"""GPU parity of the decode path (router, experts, combine, fused layer) against the fp64 oracle.

Bar: bit-exact top-K indices and dequantised weights, outputs within
2e-3*max|oracle| + 1e-5 per token vector. Runs through the C ABI on an MI355X.
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

TINY, DEC4, DEC2 = synth.WORKLOADS["tiny"], synth.WORKLOADS["decode4"], synth.WORKLOADS["decode2"]


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def tiny(gpu_device):
    _log("build tiny layer")
    return DeviceLayer(TINY), Reference(TINY)


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


def _ws(desc, T):
    n = bq.moe_workspace_bytes(desc, T)
    return torch.zeros(n, dtype=torch.uint8, device="cuda"), n


def _x(w, t0, n):
    return torch.from_numpy(synth.tokens_x(w, t0, n)).cuda()


def _forward(L, x, res=None):
    T = x.shape[0]
    ws, n = _ws(L.desc, T)
    out = torch.empty_like(x)
    idx = torch.empty(T, L.w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x if res is None else res, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


# ---- inputs and formats -----------------------------------------------------------------------

@pytest.mark.parametrize("which", ["tiny", "dec4", "dec2"])
def test_device_generation_and_pack_match_host(which, request):
    L, _ = request.getfixturevalue(which)
    w = L.w
    experts = [0, w.n_experts - 1, synth.SHARED] + ([137] if w.n_experts > 137 else [])
    for e in experts:
        _log(f"{w.name}: blob of expert {e}")
        ex = synth.expert_arrays(w, 0, e)
        blob = np.zeros(L.blob_bytes, dtype=np.uint8)
        bq.moe_pack_expert(w.hidden, w.inter, w.bits, w.group, [m.q for m in ex.mats],
                           [m.scale for m in ex.mats], [m.bias for m in ex.mats], blob)
        assert np.array_equal(L.expert_blob(e).cpu().numpy(), blob), f"expert {e}"


@pytest.mark.parametrize("which", ["tiny", "dec4", "dec2"])
def test_dequant_bit_exact(which, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    for e in (0, 5, synth.SHARED):
        ex = ref.shared if e == synth.SHARED else ref.expert(e)
        for m, mat in enumerate(ex.mats):
            rows, cols = w.matrix_shape(m)
            W = oracle.dequant(mat.q, mat.scale, mat.bias, w.group)
            assert np.array_equal(W.astype(np.float32).astype(np.float64), W)  # exact in fp32
            out = torch.empty(rows, cols, dtype=torch.float32, device="cuda")
            bq.moe_dequant(L.desc, e, m, 0, out)
            o16 = torch.empty(rows, cols, dtype=torch.int16, device="cuda")
            bq.moe_dequant(L.desc, e, m, 1, o16)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().astype(np.float64), W), f"expert {e} matrix {m}"
            rne = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
            assert torch.equal(o16.cpu(), rne), f"bf16 expert {e} matrix {m}"


# ---- step by step ------------------------------------------------------------------------------

@pytest.mark.parametrize("which,T", [("tiny", 16), ("dec4", 8), ("dec2", 8)])
def test_router(which, T, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    x = _x(w, 0, T)
    ws, n = _ws(L.desc, T)
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.top_k, dtype=torch.float32, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, w.n_experts, dtype=torch.float64, device="cuda")
    bq.moe_router(L.desc, x, T, idx, wt, g, lg, ws, n)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    for t in range(T):
        l_ref = oracle.router_logits(ref.router, xs[t])
        assert np.allclose(lg[t].cpu().numpy(), l_ref, rtol=1e-12, atol=1e-12)
        i_ref = oracle.topk(l_ref, w.top_k)
        assert list(idx[t].cpu().numpy()) == list(i_ref), f"token {t}"
        w_ref = oracle.route_weights(l_ref, i_ref)
        assert np.max(np.abs(wt[t].cpu().numpy() - w_ref)) <= 2e-3 * np.max(w_ref) + 1e-5
        assert abs(wt[t].sum().item() - 1.0) < 1e-6
        g_ref = oracle.shared_gate(ref.gate, xs[t])
        assert abs(g[t].item() - g_ref) <= 2e-3 * g_ref + 1e-5


@pytest.mark.parametrize("which,T", [("tiny", 4), ("dec4", 3), ("dec2", 3)])
def test_expert_ffn_and_combine(which, T, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    x = _x(w, 100, T)
    rng = np.random.default_rng(7)
    idx_np = rng.integers(0, w.n_experts, size=(T, w.top_k)).astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    NE = w.top_k + 1
    y = torch.empty(T, NE, w.hidden, dtype=torch.float32, device="cuda")
    ws, n = _ws(L.desc, T)
    bq.moe_expert_ffn(L.desc, x, T, idx, y, ws, n)
    wts = torch.from_numpy(rng.dirichlet(np.ones(w.top_k), size=T).astype(np.float32)).cuda()
    g = torch.rand(T, device="cuda")
    out = torch.empty(T, w.hidden, dtype=torch.float32, device="cuda")
    bq.moe_combine(L.desc, x, y, wts, g, T, out)
    torch.cuda.synchronize()
    xs = x.cpu().numpy().astype(np.float64)
    yn = y.cpu().numpy()
    for t in range(T):
        ys = [ref.expert_out(xs[t], int(e)) for e in idx_np[t]] + [ref.expert_out(xs[t], synth.SHARED)]
        for k in range(NE):
            assert_close(yn[t, k], ys[k], f"y[{t}][{k}]")
        o_ref = oracle.combine(xs[t], np.stack(ys[:-1]), wts[t].cpu().numpy(), g[t].item(), ys[-1])
        assert_close(out[t].cpu().numpy(), o_ref, f"combine[{t}]")


def test_expert_ffn_invalid_index_is_nan_not_a_fault(tiny):
    L, _ = tiny
    w = L.w
    x = _x(w, 0, 1)
    idx = torch.tensor([[1, w.n_experts + 5]], dtype=torch.int32, device="cuda")
    y = torch.empty(1, w.top_k + 1, w.hidden, dtype=torch.float32, device="cuda")
    ws, n = _ws(L.desc, 1)
    bq.moe_expert_ffn(L.desc, x, 1, idx, y, ws, n)
    torch.cuda.synchronize()
    assert torch.isfinite(y[0, 0]).all() and torch.isnan(y[0, 1]).all() and torch.isfinite(y[0, 2]).all()


@pytest.mark.parametrize("T", [1, 64, 2048])
def test_expert_ffn_checked_error_word(dec4, T):
    """moe_expert_ffn_checked: out-of-range indices (past E and negative) set the caller's error
    word to MOE_EINVAL and give NaN outputs in their slots only; the other slots, and a clean call,
    match the oracle with the word left at zero. T=1 takes the decode kernels, 64 and 2048 the
    prefill path."""
    L, ref = dec4
    w = L.w
    _log(f"{w.name}: checked expert FFN, T={T}")
    x = _x(w, 0, T)
    xs = x.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(T)
    idx_np = np.stack([rng.choice(w.n_experts, w.top_k, replace=False) for _ in range(T)]).astype(np.int32)
    bad = {(0, 1): w.n_experts + 5}
    if T > 1:
        bad[(T // 2, 0)] = -1
        bad[(T - 1, 2)] = 1 << 30
    idx_bad = idx_np.copy()
    for (t, k), v in bad.items():
        idx_bad[t, k] = v
    ws, n = _ws(L.desc, T)
    NE = w.top_k + 1
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty(T, NE, w.hidden, dtype=torch.float32, device="cuda")
    bq.moe_expert_ffn_checked(L.desc, x, T, torch.from_numpy(idx_np).cuda(), y, ws, n, err)
    torch.cuda.synchronize()
    assert err.item() == 0
    y_clean = y.cpu().numpy()
    err.zero_()
    y.fill_(0.0)
    bq.moe_expert_ffn_checked(L.desc, x, T, torch.from_numpy(idx_bad).cuda(), y, ws, n, err)
    torch.cuda.synchronize()
    assert err.item() == bq.MOE_EINVAL
    yb = y.cpu().numpy()
    for (t, k) in bad:
        assert np.isnan(yb[t, k]).all(), f"slot ({t}, {k}) not NaN"
    good = np.ones((T, NE), dtype=bool)
    for (t, k) in bad:
        good[t, k] = False
    assert np.isfinite(yb[good]).all()
    assert np.array_equal(yb[good], y_clean[good]), "valid slots changed when another slot was invalid"
    for t in sorted({0, T // 2, T - 1}):
        for k in range(NE):
            e = synth.SHARED if k == w.top_k else int(idx_np[t, k])
            assert_close(y_clean[t, k], ref.expert_out(xs[t], e), f"y[{t}][{k}]")


# ---- the fused layer -----------------------------------------------------------------------------

@pytest.mark.parametrize("which,t0,T", [("tiny", 0, 1), ("tiny", 1, 24), ("dec4", 0, 1), ("dec4", 500, 4),
                                         ("dec2", 0, 1), ("dec2", 900, 4)])
def test_layer_forward(which, t0, T, request):
    L, ref = request.getfixturevalue(which)
    w = L.w
    _log(f"{w.name}: layer forward tokens [{t0}, {t0 + T})")
    x = _x(w, t0, T)
    out, idx = _forward(L, x)
    xs = x.cpu().numpy().astype(np.float64)
    for t in range(T):
        r = ref.token(xs[t])
        assert list(idx[t]) == list(r.idx), f"token {t0 + t}: idx {idx[t]} vs {r.idx} (margin {r.margin:.3e})"
        assert_close(out[t], r.out, f"out[{t0 + t}]")


def test_layer_forward_residual_separate(tiny):
    L, ref = tiny
    x = _x(L.w, 3, 2)
    res = torch.randn_like(x)
    out, idx = _forward(L, x, res)
    for t in range(2):
        r = ref.token(x[t].cpu().numpy(), res[t].cpu().numpy())
        assert_close(out[t], r.out)


@pytest.mark.parametrize("which", ["dec4", "dec2"])
def test_decode_sequence_graph(which, request):
    """The benchmark's launch configuration: the tokens as back-to-back T=1 calls captured in one
    HIP graph. Every token's top-K is checked against the oracle's, outputs on 32 spread tokens, and
    two replays must agree bitwise."""
    L, ref = request.getfixturevalue(which)
    w = L.w
    N = w.tokens
    _log(f"{w.name}: graph of {N} single-token calls")
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
    first = out.clone()
    first_idx = idx.clone()
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


# ---- edge cases ------------------------------------------------------------------------------------

def test_empty_calls_touch_nothing(tiny):
    """T = 0 through every compute entry point: MOE_OK, nothing enqueued, every output untouched."""
    L, _ = tiny
    w = L.w
    x = _x(w, 0, 2)
    ws, n = _ws(L.desc, 2)
    out = torch.full_like(x, 7.0)
    idx = torch.full((2, w.top_k), -7, dtype=torch.int32, device="cuda")
    wt = torch.full((2, w.top_k), 7.0, device="cuda")
    g = torch.full((2,), 7.0, device="cuda")
    y = torch.full((2, w.top_k + 1, w.hidden), 7.0, device="cuda")
    err = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    sn = bq.moe_stack_workspace_bytes(L.desc, 2)
    sws = torch.zeros(sn, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    bq.moe_layer_forward(L.desc, x, x, 0, out, idx, ws, n)
    bq.moe_layer_forward_noalloc(L.desc, x, x, 0, out, idx)
    bq.moe_router(L.desc, x, 0, idx, wt, g, None, ws, n)
    bq.moe_expert_ffn(L.desc, x, 0, idx, y, ws, n)
    bq.moe_expert_ffn_checked(L.desc, x, 0, idx, y, ws, n, err)
    bq.moe_combine(L.desc, x, y, wt, g, 0, out)
    bq.moe_stack_forward([L.desc, L.desc], 1e-6, x, 0, out, None, sws, sn)
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (idx == -7).all() and (wt == 7.0).all() and (g == 7.0).all()
    assert (y == 7.0).all() and err.item() == 7


def test_zero_input_gives_residual(tiny):
    L, _ = tiny
    w = L.w
    x = torch.zeros(2, w.hidden, device="cuda")
    res = _x(w, 0, 2)
    out, idx = _forward(L, x, res)
    assert np.array_equal(out, res.cpu().numpy())
    assert (idx == np.arange(w.top_k)).all()


def test_zero_codes_bias_only(gpu_device):
    """All codes zero: every weight is its group bias (closed form in the oracle pins)."""
    w = TINY
    L = DeviceLayer(w)
    ref = Reference(w)
    H, I = w.hidden, w.inter
    for e in list(range(w.n_experts)) + [synth.SHARED]:
        ex = ref.expert(e) if e != synth.SHARED else ref.shared
        for m in ex.mats:
            m.q[:] = 0
        blob = np.zeros(L.blob_bytes, dtype=np.uint8)
        bq.moe_pack_expert(H, I, w.bits, w.group, [m.q for m in ex.mats], [m.scale for m in ex.mats],
                           [m.bias for m in ex.mats], blob)
        L.expert_blob(e).copy_(torch.from_numpy(blob))
    x = _x(w, 0, 3)
    out, idx = _forward(L, x)
    for t in range(3):
        r = ref.token(x[t].cpu().numpy())
        assert list(idx[t]) == list(r.idx)
        assert_close(out[t], r.out)


def test_duplicate_router_rows_tie_to_lower_index(gpu_device):
    w = TINY
    L = DeviceLayer(w)
    ref = Reference(w)
    x = _x(w, 0, 1)
    lg = oracle.router_logits(ref.router, x[0].cpu().numpy())
    best = int(np.argmax(lg))
    R = ref.router.copy()
    for r in (2, 5):
        R[r] = R[best]
    ref.router = R
    L.router.copy_(torch.from_numpy(R.view(np.int16)))
    out, idx = _forward(L, x)
    r = ref.token(x[0].cpu().numpy())
    tied = sorted({best, 2, 5})
    assert list(r.idx) == tied[:2] and list(idx[0]) == tied[:2]
    assert_close(out[0], r.out)


@pytest.mark.parametrize("T", [1, 4, 64])
def test_topk_low_bit_tie_break(gpu_device, T):
    """Logits equal in their upper 32 bits: row a is row b with one bf16 ulp more at an element
    where x is 1e-10, so the two fp64 logits differ only far below 2^-20 relative; row c duplicates
    row b exactly. The order must be a, then the lower of b and c (T=1 and T=4 take the decode
    routers, T=64 the prefill router)."""
    w = TINY
    L = DeviceLayer(w)
    ref = Reference(w)
    x = _x(w, 0, 1)[0].cpu().numpy().copy()
    R = ref.router.copy()
    lg = oracle.router_logits(R, x.astype(np.float64))
    b = int(np.argmax(lg))
    a_row, c_row = [r for r in range(w.n_experts) if r != b][:2]
    Rb = synth.bf16_to_f32(R[b])
    j = int(np.flatnonzero(Rb > 0)[0])
    x[j] = np.float32(1e-10)
    R[a_row] = R[b]
    R[a_row, j] = R[b, j] + 1  # one ulp larger in magnitude, and positive
    R[c_row] = R[b]
    ref.router = R
    L.router.copy_(torch.from_numpy(R.view(np.int16)))
    xd = x.astype(np.float64)
    lg = oracle.router_logits(R, xd)
    hi = lambda v: np.float64(v).view(np.uint64) >> np.uint64(32)
    assert lg[a_row] > lg[b] == lg[c_row] and hi(lg[a_row]) == hi(lg[b]), "the case must tie in the upper 32 bits"
    want = [a_row, min(b, c_row)]
    r = ref.token(xd)
    assert list(r.idx) == want
    X = torch.from_numpy(np.tile(x, (T, 1))).cuda()
    out, idx = _forward(L, X)
    for t in range(T):
        assert list(idx[t]) == want, f"token {t}: {list(idx[t])} vs {want}"
        assert_close(out[t], r.out, f"out[{t}]")


def test_bitwise_determinism(dec4):
    L, _ = dec4
    x = _x(L.w, 10, 2)
    a, ia = _forward(L, x)
    b, ib = _forward(L, x)
    assert np.array_equal(a, b) and np.array_equal(ia, ib)


# ---- per-element dequant forms (the pages' rewrite and the form it replaced), an A/B ablation ------

@pytest.mark.parametrize("flag", ["MOE_FLAG_DEQUANT_LITERAL", "MOE_FLAG_DEQUANT_NAIVE"])
@pytest.mark.parametrize("which,tokens", [("tiny", 4), ("dec4", 6), ("dec2", 6)])
def test_per_element_dequant_forms_parity(which, tokens, flag, request):
    """The decode GEMVs in the pages' fma(q, s*x, b*x) form, and in the naive (q*s + b)*x form, meet
    the default form's bar: bit-exact routing, outputs within tolerance of the oracle, and within
    rounding of the default form."""
    L, ref = request.getfixturevalue(which)
    w = L.w
    x = _x(w, 40, tokens)
    base_out, base_idx = _forward(L, x)
    L.desc.flags = getattr(bq, flag)
    try:
        out, idx = _forward(L, x)
    finally:
        L.desc.flags = 0
    xs = x.cpu().numpy()
    for t in range(tokens):
        r = ref.token(xs[t])
        assert list(idx[t]) == list(r.idx) == list(base_idx[t]), f"{w.name} token {t}"
        assert_close(out[t], r.out, f"{w.name} literal out[{t}]")
        assert_close(out[t], base_out[t], f"{w.name} literal vs default out[{t}]")



@pytest.mark.parametrize("which,T", [("tiny", 9), ("dec4", 8), ("dec2", 6)])
def test_router_token_groups_bitwise(which, T, request):
    """Several tokens per call read each router row once for a group of tokens; every token's
    logits are summed in the single-token order, so they equal one-token calls bitwise (T not a
    multiple of the group size leaves a partial group)."""
    L, _ = request.getfixturevalue(which)
    w = L.w
    x = _x(w, 60, T)
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(T, w.top_k, dtype=torch.int32, device="cuda")
    wt = torch.empty(T, w.top_k, dtype=torch.float32, device="cuda")
    lg = torch.empty(T, w.n_experts, dtype=torch.float64, device="cuda")
    bq.moe_router(L.desc, x, T, idx, wt, None, lg, ws, n)
    one = torch.empty(1, w.n_experts, dtype=torch.float64, device="cuda")
    i1 = torch.empty(1, w.top_k, dtype=torch.int32, device="cuda")
    w1 = torch.empty(1, w.top_k, dtype=torch.float32, device="cuda")
    n1 = bq.moe_workspace_bytes(L.desc, 1)
    ws1 = torch.zeros(n1, dtype=torch.uint8, device="cuda")
    for t in range(T):
        bq.moe_router(L.desc, x[t:t + 1].contiguous(), 1, i1, w1, None, one, ws1, n1)
        torch.cuda.synchronize()
        assert torch.equal(lg[t], one[0]), f"token {t}"
        assert torch.equal(idx[t], i1[0]) and torch.equal(wt[t], w1[0])
