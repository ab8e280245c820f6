"""GPU parity at the edges of the supported shapes, against the fp64 oracle.

- 1024 experts (MOE_MAX_EXPERTS), top-8 (MOE_MAX_TOP_K): the decode top-K holds 16 logits per lane.
- top-K = E (every expert routed; the weights are the full softmax) and top-1 (weight 1).
- hidden 8192 x inter 2048, the largest rows the kernels take, in the affine 4-bit, 2-bit and
  MXFP4 formats; hidden 1024 and 2048 (other lane-per-row layouts of the decode GEMVs); MXFP4 with
  inter 64, which stays on the per-token path at every T.
Each runs the decode path and the prefill path. Bar as elsewhere: bit-exact top-K indices;
outputs within 2e-3*max|oracle| + 1e-5 per token vector.
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

_4 = dict(bits=4, scale_range=(0.001, 0.01), bias_range=(-0.08, -0.005))
_2 = dict(bits=2, scale_range=(0.004, 0.04), bias_range=(-0.06, -0.004))
SHAPES = {
    "e1024": synth.Workload("e1024", 256, 1024, 64, 8, weight_family=11, x_family=11, **_4),
    "kall": synth.Workload("kall", 256, 8, 128, 8, weight_family=12, x_family=12, **_4),
    "k1": synth.Workload("k1", 512, 16, 64, 1, weight_family=13, x_family=13, **_2),
    "max4": synth.Workload("max4", 8192, 12, 2048, 3, weight_family=14, x_family=14, **_4),
    "maxmx": synth.Workload("maxmx", 8192, 8, 2048, 6, bits=4, group=32, fmt="mxfp4", weight_family=15,
                            x_family=15),
    "max2": synth.Workload("max2", 8192, 8, 2048, 3, weight_family=16, x_family=16, **_2),
    "mid2": synth.Workload("mid2", 1024, 32, 512, 4, weight_family=17, x_family=17, **_2),
    "mid4": synth.Workload("mid4", 2048, 16, 256, 2, weight_family=18, x_family=18, **_4),
    "mx64": synth.Workload("mx64", 256, 8, 64, 2, bits=4, group=32, fmt="mxfp4", weight_family=19, x_family=19),
}


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def layers(gpu_device):
    built = {}

    def get(name):
        if name not in built:
            _log(f"build layer {name}")
            w = SHAPES[name]
            built[name] = (DeviceLayer(w), Reference(w, cache=16))
            torch.cuda.synchronize()
        return built[name]

    yield get
    built.clear()
    torch.cuda.empty_cache()


def _forward(L, x):
    T = x.shape[0]
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(T, L.w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("name,T,check", [
    ("e1024", 1, (0,)), ("e1024", 5, (0, 2, 4)), ("e1024", 100, (0, 31, 32, 99)),
    ("kall", 2, (0, 1)), ("kall", 70, (0, 35, 69)),
    ("k1", 1, (0,)), ("k1", 4, (0, 1, 2, 3)), ("k1", 64, (0, 63)),
    ("max4", 1, (0,)), ("max4", 64, (0, 63)),
    ("maxmx", 1, (0,)), ("maxmx", 64, (0, 63)),
    ("max2", 1, (0,)), ("max2", 64, (0, 63)),
    ("mid2", 3, (0, 1, 2)), ("mid2", 100, (0, 50, 99)),
    ("mid4", 2, (0, 1)), ("mid4", 64, (0, 33, 63)),
    ("mid4", bq.MOE_PREFILL_MIN_TOKENS - 1, (0, 46)), ("mid4", bq.MOE_PREFILL_MIN_TOKENS, (0, 47)),  # both sides of the threshold
    ("mx64", 1, (0,)), ("mx64", 60, (0, 30, 59)),  # MXFP4 below inter 128 decodes at every T
])
def test_edge_shape_layer_forward(layers, name, T, check):
    L, ref = layers(name)
    w = L.w
    path = "prefill" if T >= bq.MOE_PREFILL_MIN_TOKENS and (w.fmt != "mxfp4" or w.inter >= 128) else "decode"
    _log(f"{name}: {T} tokens ({path})")
    x = torch.from_numpy(synth.tokens_x(w, 0, T)).cuda()
    out, idx = _forward(L, x)
    xs = x.cpu().numpy().astype(np.float64)
    for t in range(T):  # every token's routing
        l_ref = oracle.router_logits(ref.router, xs[t])
        assert list(idx[t]) == list(oracle.topk(l_ref, w.top_k)), f"{name} token {t}"
    for t in check:
        r = ref.token(xs[t])
        if w.top_k == w.n_experts:
            assert sorted(r.idx) == list(range(w.n_experts))
        if w.top_k == 1:
            assert np.array_equal(r.w, [1.0])
        assert_close(out[t], r.out, f"{name} out[{t}]")
