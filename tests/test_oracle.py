"""Pins of the fp64 oracle to things other than itself (CPU only).

Each pin checks one oracle function against a different route to the same value:
- numpy brute force on tiny inputs;
- textbook routines (Python's sorted, scipy's softmax and expit);
- closed forms for special inputs;
- invariants;
- exact rational arithmetic;
- the figures the pages print.

The pins are plain functions, so ``test_mutants_are_caught`` can rerun them against
deliberately broken builds of ``oracle.c`` and show that each plausible mistake is caught.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import scipy.special as sp

import oracle
import synth

TINY = synth.WORKLOADS["tiny"]
G = TINY.group


def _bf(h):
    return synth.bf16_to_f32(np.asarray(h, dtype=np.uint16)).astype(np.float64)


def _dense_np(m, group=G):
    """Independent dense dequantisation: scales/biases broadcast along the group axis."""
    s = np.repeat(_bf(m.scale), group, axis=1)
    b = np.repeat(_bf(m.bias), group, axis=1)
    return s * m.q.astype(np.float64) + b


def _bf16_bits(v):
    """Exact bf16 bit pattern of a value representable in bf16."""
    f = np.float32(v)
    u = f.view(np.uint32)
    assert (u & 0xFFFF) == 0, v
    return np.uint16(u >> 16)


# ---- pins -------------------------------------------------------------------------------------

def pin_dequant_special_cases():
    # scale 1.0 (0x3F80), bias 0 -> W equals the code; bias -2 (0xC000) shifts every element by -2.
    rows, cols = 3, 2 * G
    q = (np.arange(rows * cols) % 16).astype(np.uint8).reshape(rows, cols)
    s = np.full((rows, cols // G), 0x3F80, dtype=np.uint16)
    b = np.zeros((rows, cols // G), dtype=np.uint16)
    assert np.array_equal(oracle.dequant(q, s, b, G), q.astype(np.float64))
    b[:] = 0xC000
    assert np.array_equal(oracle.dequant(q, s, b, G), q.astype(np.float64) - 2.0)
    # distinct power-of-two scale per (row, group), q = 1, bias 0: element (r, c) must carry group c // G's scale
    q1 = np.ones((rows, cols), dtype=np.uint8)
    sv = np.array([[2.0 ** -(1 + r * 2 + g) for g in range(cols // G)] for r in range(rows)])
    s2 = np.vectorize(_bf16_bits)(sv).astype(np.uint16)
    got = oracle.dequant(q1, s2, np.zeros_like(s2), G)
    for r in range(rows):
        for c in range(cols):
            assert got[r, c] == sv[r, c // G]
    # linearity in the code: W(q+1) - W(q) = scale, for every element
    ex = synth.expert_arrays(TINY, 0, 3)
    m = ex.gate
    qa = np.minimum(m.q, 14)
    d = oracle.dequant(qa + 1, m.scale, m.bias, G) - oracle.dequant(qa, m.scale, m.bias, G)
    assert np.array_equal(d, np.repeat(_bf(m.scale), G, axis=1))


def pin_dequant_bruteforce():
    ex = synth.expert_arrays(TINY, 0, 1)
    for m in ex.mats:
        assert np.array_equal(oracle.dequant(m.q, m.scale, m.bias, G), _dense_np(m))


def pin_matvec_onehot():
    ex = synth.expert_arrays(TINY, 0, 2)
    W = oracle.dequant(ex.up.q, ex.up.scale, ex.up.bias, G)
    for j in (0, 1, G - 1, G, W.shape[1] - 1):
        e = np.zeros(W.shape[1])
        e[j] = 1.0
        assert np.array_equal(oracle.matvec(W, e), W[:, j])
    v = np.random.default_rng(0).standard_normal(W.shape[1])
    assert np.allclose(oracle.matvec(W, v), W @ v, rtol=1e-12, atol=1e-12)


def pin_router_logits():
    R = synth.router_weights(TINY)
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    ref = _bf(R) @ x
    assert np.allclose(oracle.router_logits(R, x), ref, rtol=1e-12, atol=1e-14)
    # logit e depends on row e only: a one-hot x picks column j of R
    e = np.zeros(TINY.hidden)
    e[5] = 1.0
    assert np.array_equal(oracle.router_logits(R, e), _bf(R)[:, 5])


def pin_topk_sorted():
    rng = np.random.default_rng(1)
    logits = np.round(rng.standard_normal(64), 1)  # many exact ties
    for K in (1, 2, 3, 7, 64):
        ref = sorted(range(64), key=lambda e: (-logits[e], e))[:K]
        assert list(oracle.topk(logits, K)) == ref


def pin_topk_duplicate_rows_tie():
    # duplicate router rows give exactly equal logits; the lower index must come first
    R = synth.router_weights(TINY).copy()
    R[6] = R[1]
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    lg = oracle.router_logits(R, x)
    assert lg[1] == lg[6]
    best = int(np.argmax(lg))
    ref_row = R[best].copy()
    for r in (1, 4, 6):
        R[r] = ref_row
    lg = oracle.router_logits(R, x)
    tied = sorted({best, 1, 4, 6})
    assert len({lg[r] for r in tied}) == 1 and lg[tied[0]] == lg.max()
    assert list(oracle.topk(lg, 3)) == tied[:3]


def pin_route_weights():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal(16) * 2
    for K in (1, 3, 16):
        idx = oracle.topk(lg, K)
        w = oracle.route_weights(lg, idx)
        assert abs(w.sum() - 1.0) < 1e-15
        # renormalised full softmax = softmax over the chosen logits
        assert np.allclose(w, sp.softmax(lg[idx]), rtol=1e-14, atol=0)
    assert np.array_equal(oracle.route_weights(lg, oracle.topk(lg, 1)), [1.0])
    idx = np.arange(16, dtype=np.int32)
    assert np.allclose(oracle.route_weights(lg, idx), sp.softmax(lg), rtol=1e-14, atol=0)
    # order of the chosen experts carries over to the weights
    idx = oracle.topk(lg, 4)
    w = oracle.route_weights(lg, idx)
    assert np.all(np.diff(w) <= 0) and abs(w[0] / w[1] - np.exp(lg[idx[0]] - lg[idx[1]])) < 1e-13


def pin_shared_gate():
    gs = synth.shared_gate_weights(TINY)
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    assert abs(oracle.shared_gate(gs, x) - sp.expit(_bf(gs) @ x)) < 1e-15
    assert oracle.shared_gate(gs, np.zeros(TINY.hidden)) == 0.5


def _np_expert(x, ex):
    a = _dense_np(ex.gate) @ x
    c = _dense_np(ex.up) @ x
    h = a * sp.expit(a) * c
    return _dense_np(ex.down) @ h, h


def pin_expert_bruteforce():
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    for e in (0, 5, synth.SHARED):
        ex = synth.expert_arrays(TINY, 0, e)
        y, h = oracle.expert(x, ex, G, want_h=True)
        y_ref, h_ref = _np_expert(x, ex)
        assert np.allclose(h, h_ref, rtol=1e-12, atol=1e-13)
        assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-12)


def pin_expert_bias_only():
    # all codes zero: every weight is its group bias, so a_r = sum_g b[r][g] * S_g(x), S_g = group sum of x
    ex = synth.expert_arrays(TINY, 0, 4)
    for m in ex.mats:
        m.q[:] = 0
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    S = x.reshape(-1, G).sum(axis=1)
    a = _bf(ex.gate.bias) @ S
    c = _bf(ex.up.bias) @ S
    h = a / (1.0 + np.exp(-a)) * c
    y = _bf(ex.down.bias) @ h.reshape(-1, G).sum(axis=1)
    y_got, h_got = oracle.expert(x, ex, G, want_h=True)
    assert np.allclose(h_got, h, rtol=1e-12, atol=1e-14)
    assert np.allclose(y_got, y, rtol=1e-12, atol=1e-13)


def pin_swiglu_points():
    # gate row r reads x_0 only (one-hot x) so a_r = W_gate[r][0], c_r = W_up[r][0]; silu(a) c follows
    ex = synth.expert_arrays(TINY, 0, 6)
    x = np.zeros(TINY.hidden)
    x[0] = 1.0
    _, h = oracle.expert(x, ex, G, want_h=True)
    a = _dense_np(ex.gate)[:, 0]
    c = _dense_np(ex.up)[:, 0]
    assert np.allclose(h, a * sp.expit(a) * c, rtol=1e-13, atol=1e-16)
    # silu(0) = 0 exactly: zero input gives a zero SwiGLU output and a zero expert output
    y0, h0 = oracle.expert(np.zeros(TINY.hidden), ex, G, want_h=True)
    assert not h0.any() and not y0.any()


def pin_combine():
    rng = np.random.default_rng(3)
    H, K = 32, 3
    res, y, ys = rng.standard_normal(H), rng.standard_normal((K, H)), rng.standard_normal(H)
    w = np.array([0.5, 0.3, 0.2])
    out = oracle.combine(res, y, w, 0.25, ys)
    assert np.allclose(out, res + w @ y + 0.25 * ys, rtol=1e-14, atol=1e-14)
    assert np.array_equal(oracle.combine(res, np.zeros((K, H)), w, 0.7, np.zeros(H)), res)
    assert np.allclose(oracle.combine(res, y, w, 0.0, None), res + w @ y, rtol=1e-14, atol=1e-14)


def pin_rmsnorm():
    rng = np.random.default_rng(4)
    h = rng.standard_normal(4096) * 3.0
    u0 = oracle.rmsnorm(h, 0.0)
    assert np.allclose(u0, h * np.sqrt(h.size) / np.linalg.norm(h), rtol=1e-13)
    eps = 1e-6
    u = oracle.rmsnorm(h, eps)
    ms = np.mean(h * h)
    assert abs(np.mean(u * u) - ms / (ms + eps)) < 1e-12
    assert np.all(np.sign(u) == np.sign(h))


def _np_layer(x, res, R, gs, experts, shared, K):
    """Brute force: every expert evaluated densely, then the top-K mask applied."""
    lg = _bf(R) @ x
    order = sorted(range(len(lg)), key=lambda e: (-lg[e], e))
    top = order[:K]
    p = sp.softmax(lg)
    w = p[top] / p[top].sum()
    ys = np.stack([_np_expert(x, ex)[0] for ex in experts])
    mask = np.zeros(len(lg))
    mask[top] = w
    g = sp.expit(_bf(gs) @ x)
    out = res + mask @ ys + g * _np_expert(x, shared)[0]
    return out, np.array(top), w, g


def pin_tiny_layer_bruteforce():
    R = synth.router_weights(TINY)
    gs = synth.shared_gate_weights(TINY)
    experts = [synth.expert_arrays(TINY, 0, e) for e in range(TINY.n_experts)]
    shared = synth.expert_arrays(TINY, 0, synth.SHARED)
    x = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    got = oracle.layer(x, x, R, gs, lambda e: experts[e], TINY.top_k, G, shared_expert=shared)
    out, top, w, g = _np_layer(x, x, R, gs, experts, shared, TINY.top_k)
    assert list(got.idx) == list(top)
    assert np.allclose(got.w, w, rtol=1e-13)
    assert abs(got.g - g) < 1e-15
    assert np.allclose(got.out, out, rtol=1e-12, atol=1e-12)


def pin_zero_input():
    # x = 0: all logits 0, so the tie rule picks experts 0..K-1 with equal weights; g = 1/2; every
    # projection is 0 (silu(0) = 0), so the output is the residual.
    R = synth.router_weights(TINY)
    gs = synth.shared_gate_weights(TINY)
    shared = synth.expert_arrays(TINY, 0, synth.SHARED)
    res = synth.tokens_x(TINY, 0, 1)[0].astype(np.float64)
    got = oracle.layer(np.zeros(TINY.hidden), res, R, gs, lambda e: synth.expert_arrays(TINY, 0, e),
                       TINY.top_k, G, shared_expert=shared)
    assert list(got.idx) == list(range(TINY.top_k))
    assert np.array_equal(got.w, np.full(TINY.top_k, 1.0 / TINY.top_k))
    assert got.g == 0.5
    assert np.array_equal(got.out, res)


# ---- MXFP4 pins --------------------------------------------------------------------------------
# The values E2M1 defines (sign, 2 exponent bits, 1 mantissa bit), written out as the list the
# format specifies rather than derived from bit fields, and E8M0 = 2^(s - 127).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
TINYMX = synth.WORKLOADS["tinymx"]


def _dense_mx(m):
    return np.array(E2M1_TABLE)[m.q] * np.ldexp(1.0, np.repeat(m.scale.astype(np.int64) - 127, 32, axis=1))


def pin_mx_e2m1_table():
    q = np.tile(np.arange(16, dtype=np.uint8), 2).reshape(1, 32)
    W = oracle.dequant_mx(q, np.full((1, 1), 127, np.uint16))
    assert np.array_equal(W[0], np.array(E2M1_TABLE * 2))
    assert np.signbit(W[0, 8]) and not np.signbit(W[0, 0])


def pin_mx_e8m0_scales():
    q = np.full((6, 64), 2, np.uint8)  # E2M1 1.0 everywhere
    s = np.array([[127, 128], [120, 0], [254, 127], [255, 127], [1, 2], [126, 125]], np.uint16)
    W = oracle.dequant_mx(q, s)
    assert W[0, 0] == 1.0 and W[0, 40] == 2.0
    assert W[1, 0] == 2.0 ** -7 and W[1, 40] == 2.0 ** -127
    assert W[2, 0] == 2.0 ** 127 and W[2, 40] == 1.0
    assert np.all(np.isnan(W[3, :32])) and np.all(W[3, 32:] == 1.0)
    assert W[4, 0] == 2.0 ** -126 and W[4, 63] == 2.0 ** -125
    assert W[5, 31] == 0.5 and W[5, 32] == 0.25


def pin_mx_dequant_bruteforce():
    ex = synth.expert_arrays(TINYMX, 0, 3)
    for m in ex.mats:
        assert np.array_equal(oracle.dequant_mx(m.q, m.scale), _dense_mx(m))


def pin_mx_expert_bruteforce():
    ex = synth.expert_arrays(TINYMX, 0, 5)
    x = synth.tokens_x(TINYMX, 0, 1)[0].astype(np.float64)
    Wg, Wu, Wd = (_dense_mx(m) for m in ex.mats)
    a, c = Wg @ x, Wu @ x
    want = Wd @ (a * sp.expit(a) * c)
    got = oracle.expert(x, ex, 32)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def pin_mx_expert_closed_form():
    # every weight 1.0 (code 2, scale 127), x = ones: a = c = H, h = H^2 * sigmoid(H), y = I * h
    H, I = 64, 96
    mk = lambda r, cc: synth.MatrixArrays(np.full((r, cc), 2, np.uint8), np.full((r, cc // 32), 127, np.uint16),
                                          None, "mxfp4")
    ex = synth.ExpertArrays(mk(I, H), mk(I, H), mk(H, I))
    y = oracle.expert(np.ones(H), ex, 32)
    h = H * H * sp.expit(H)
    assert np.allclose(y, I * h, rtol=1e-14)


PINS = [pin_dequant_special_cases, pin_dequant_bruteforce, pin_matvec_onehot, pin_router_logits,
        pin_topk_sorted, pin_topk_duplicate_rows_tie, pin_route_weights, pin_shared_gate,
        pin_expert_bruteforce, pin_expert_bias_only, pin_swiglu_points, pin_combine, pin_rmsnorm,
        pin_tiny_layer_bruteforce, pin_zero_input, pin_mx_e2m1_table, pin_mx_e8m0_scales,
        pin_mx_dequant_bruteforce, pin_mx_expert_bruteforce, pin_mx_expert_closed_form]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---- exact identities behind the GPU's rewrite --------------------------------------------------

def test_fma_rewrite_identity_exact():
    """(q*s + b)*x = q*(s*x) + b*x (GN+ summary, FMA-optimised dequant kernel), and summed over a group
    it is s*sum(q*x) + b*sum(x). Checked in exact rational arithmetic on the tiny workload's values."""
    ex = synth.expert_arrays(TINY, 0, 0)
    x = synth.tokens_x(TINY, 0, 1)[0]
    row = 7
    q, s, b = ex.gate.q[row], _bf(ex.gate.scale[row]), _bf(ex.gate.bias[row])
    for g in range(TINY.hidden // G):
        sF, bF = Fraction(float(s[g])), Fraction(float(b[g]))
        xs = [Fraction(float(v)) for v in x[g * G:(g + 1) * G]]
        qs = [int(v) for v in q[g * G:(g + 1) * G]]
        lhs = sum((qq * sF + bF) * xx for qq, xx in zip(qs, xs))
        assert lhs == sum(qq * (sF * xx) + bF * xx for qq, xx in zip(qs, xs))
        assert lhs == sF * sum(qq * xx for qq, xx in zip(qs, xs)) + bF * sum(xs)


def test_dequant_exact_in_fp32():
    """Every weight of every workload's value ranges is exactly representable in fp32, so a GPU fp32
    dequantisation can match the fp64 definition bit for bit."""
    for name in ("tiny", "decode4", "decode2"):
        w = synth.WORKLOADS[name]
        q = np.arange(2 ** w.bits, dtype=np.float64)
        # extreme bf16 scales/biases of the ranges plus random ones
        rng = np.random.default_rng(5)
        svals = np.concatenate([[w.scale_range[0], w.scale_range[1]], rng.uniform(*w.scale_range, 200)])
        bvals = np.concatenate([[w.bias_range[0], w.bias_range[1]], rng.uniform(*w.bias_range, 200)])
        sb = synth.bf16_to_f32(np.array([synth.host_lib().bq_bf16_rne(float(v)) for v in svals], np.uint16))
        bb = synth.bf16_to_f32(np.array([synth.host_lib().bq_bf16_rne(float(v)) for v in bvals], np.uint16))
        W = sb.astype(np.float64)[:, None, None] * q[None, :, None] + bb.astype(np.float64)[None, None, :]
        assert np.array_equal(W.astype(np.float32).astype(np.float64), W), name


# ---- figures printed on the pages ---------------------------------------------------------------

def test_page_figures_pin_format():
    """Bits per weight: 4-bit codes plus a bf16 (scale, bias) pair per 64 weights makes 6.75 MiB per
    expert; 2-bit experts at 60 layers x 4 experts per token make the quoted 943 MB per token."""
    import json

    fig = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
    H, I, G_ = 4096, 1024, 64

    def expert_bytes(bits):
        weights = 3 * H * I
        return weights * bits // 8 + (weights // G_) * 4

    assert expert_bytes(4) == 7_077_888 == fig["expert_mb_4bit"]["value"] * 2 ** 20
    per_tok = fig["model_shape"]["layers"] * fig["model_shape"]["active_per_token_incl_shared"] * expert_bytes(2)
    assert round(per_tok / 1e6) == 944 and abs(per_tok / 1e6 - fig["io_mb_per_token_k4"]["value"]) < 1.0
    assert abs(fig["io_mb_per_token_k4"]["value"] * fig["io_rate_check"]["tok_per_s"] - fig["io_rate_check"]["mb_per_s"]) < 2


# ---- mutation check: a plausible mistake anywhere in the oracle fails a pin ----------------------

MUTANTS = {
    "group index uses modulo": ("scale[r * ng + c / group]", "scale[r * ng + c % group]"),
    "bias dropped": ("W[r * cols + c] = s * (double)q[r * cols + c] + b;", "W[r * cols + c] = s * (double)q[r * cols + c];"),
    "transposed matvec": ("acc += W[r * cols + c] * v[c];", "acc += W[c * rows + r] * v[c];"),
    "router reads wrong row": ("acc += bf16_value(R[e * H + j]) * x[j];", "acc += bf16_value(R[j * E + e]) * x[j];"),
    "ascending sort": ("if (x->v > y->v) return -1;", "if (x->v < y->v) return -1;"),
    "ties to higher index": ("return (x->e < y->e) ? -1 : (x->e > y->e);", "return (x->e > y->e) ? -1 : (x->e < y->e);"),
    "no renormalisation": ("for (int64_t k = 0; k < K; ++k) w[k] = w[k] / sel;", ""),
    "gate sign flipped": ("return 1.0 / (1.0 + exp(-acc));", "return 1.0 / (1.0 + exp(acc));"),
    "silu sign flipped": ("h[i] = a[i] / (1.0 + exp(-a[i])) * c[i];", "h[i] = a[i] / (1.0 + exp(a[i])) * c[i];"),
    "gate/up swapped in silu": ("h[i] = a[i] / (1.0 + exp(-a[i])) * c[i];", "h[i] = c[i] / (1.0 + exp(-c[i])) * a[i];"),
    "combine drops residual": ("double acc = res[r];", "double acc = 0.0;"),
    "combine transposes y": ("acc += w[k] * y[k * H + r];", "acc += w[k] * y[r * K + k];"),
    "rmsnorm without mean": ("ss / (double)H + eps", "ss + eps"),
    "e2m1 exponent bias 0": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e2m1 no subnormals": ("e == 0 ? 0.5 * m", "e == 0 ? 1.0 * m"),
    "e2m1 sign ignored": ("return sign ? -v : v;", "return v;"),
    "e8m0 bias 128": ("ldexp(1.0, (int)s - 127)", "ldexp(1.0, (int)s - 128)"),
    "mx block of 64": ("scale[r * nb + c / 32]", "scale[r * nb + c / 64]"),
    "mx down uses gate codes": ("oracle_dequant_mx(H, I, q[2], scale[2], Wd);", "oracle_dequant_mx(H, I, q[0], scale[2], Wd);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src_dir = os.path.dirname(oracle.__file__)
    src = open(os.path.join(src_dir, "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    (tmp_path / "oracle.h").write_text(open(os.path.join(src_dir, "oracle.h")).read())
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11", str(tmp_path / "oracle.c"),
                    "-o", str(so), "-lm"], check=True)
    good = oracle._lib
    oracle._lib = None
    real = oracle.lib()  # rebuild the argtypes on the mutant by swapping the path
    mut = ctypes.CDLL(str(so))
    for fname in ("oracle_dequant", "oracle_matvec", "oracle_router_logits", "oracle_topk", "oracle_route_weights",
                  "oracle_shared_gate", "oracle_expert", "oracle_combine", "oracle_rmsnorm", "oracle_dequant_mx",
                  "oracle_expert_mx"):
        getattr(mut, fname).argtypes = getattr(real, fname).argtypes
        getattr(mut, fname).restype = getattr(real, fname).restype
    oracle._lib = mut
    caught = []
    try:
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                caught.append(pin.__name__)
    finally:
        oracle._lib = good
    assert caught, f"mutant '{name}' passed every pin"


# ---- the stack composition ----------------------------------------------------------------------

def test_stack_two_layers_bruteforce():
    """Two tiny layers: h1 = x + MoE0(x), u1 = h1 / rms(h1), out = h1 + MoE1(u1), by numpy brute force."""
    w = synth.Workload("tinystack", 256, 8, 128, 2, bits=4, weight_family=5, x_family=5)
    per = []
    for l in range(2):
        R = synth.router_weights(w, l)
        gs = synth.shared_gate_weights(w, l)
        ex = [synth.expert_arrays(w, l, e) for e in range(w.n_experts)]
        sh = synth.expert_arrays(w, l, synth.SHARED)
        per.append((R, gs, ex, sh))
    x = synth.tokens_x(w, 0, 1)[0].astype(np.float64)
    h1, top0, _, _ = _np_layer(x, x, per[0][0], per[0][1], per[0][2], per[0][3], w.top_k)
    u1 = h1 / np.sqrt(np.mean(h1 * h1) + 1e-6)
    out, top1, _, _ = _np_layer(u1, h1, per[1][0], per[1][1], per[1][2], per[1][3], w.top_k)
    layers = [(R, gs, (lambda ex: (lambda e: ex[e]))(ex), sh) for (R, gs, ex, sh) in per]
    r = oracle.stack(x, layers, w.top_k, w.group, 1e-6)
    assert np.array_equal(r.idx, np.stack([top0, top1]))
    assert np.allclose(r.out, out, rtol=1e-12, atol=1e-12)
    # per-layer margin: the gap between the K-th and (K+1)-th logit of that layer's own input
    u1_lg = np.sort(_bf(per[1][0]) @ u1)[::-1]
    x_lg = np.sort(_bf(per[0][0]) @ x)[::-1]
    K = w.top_k
    assert np.allclose(r.margin, [x_lg[K - 1] - x_lg[K], u1_lg[K - 1] - u1_lg[K]], rtol=1e-12, atol=1e-15)
