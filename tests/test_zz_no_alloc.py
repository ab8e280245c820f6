"""moe_layer_forward_noalloc (no workspace argument, fixed in-library scratch) against
moe_layer_forward with a caller workspace: two calls in a row, the second smaller, through the C ABI.
Both run the same kernels, so the results must agree bit for bit; sampled tokens are also checked
against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bit_quantized_expert_gemv_amd as bq
import synth
from synth.gpu_layers import DeviceLayer
from tests._ref import Reference, assert_close, check_topk_all

pytestmark = pytest.mark.gpu


def _log(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _with_workspace(L, x, T):
    n = bq.moe_workspace_bytes(L.desc, T)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    idx = torch.empty(T, L.w.top_k, dtype=torch.int32, device="cuda")
    bq.moe_layer_forward(L.desc, x, x, T, out, idx, ws, n)
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("name,sizes", [("decode4", (64, 3)), ("decodemx", (5, 1))])
def test_noalloc_matches_workspace_entry(gpu_device, name, sizes):
    w = synth.WORKLOADS[name]
    _log(f"{name}: build layer")
    L = DeviceLayer(w)
    ref = Reference(w)
    torch.cuda.synchronize()
    for T in sizes:
        assert bq.moe_workspace_bytes(L.desc, T) <= bq.MOE_NOALLOC_SCRATCH_BYTES
        _log(f"{name}: no-alloc call, T={T}")
        x = torch.from_numpy(synth.tokens_x(w, 7, T)).cuda()
        out = torch.full_like(x, float("nan"))
        idx = torch.full((T, w.top_k), -1, dtype=torch.int32, device="cuda")
        bq.moe_layer_forward_noalloc(L.desc, x, x, T, out, idx)
        torch.cuda.synchronize()
        on, ix = out.cpu().numpy(), idx.cpu().numpy()
        want_out, want_idx = _with_workspace(L, x, T)
        assert np.array_equal(ix, want_idx), f"T={T}: indices differ from moe_layer_forward"
        assert np.array_equal(on, want_out), f"T={T}: outputs differ from moe_layer_forward"
        xs = x.cpu().numpy().astype(np.float64)
        check_topk_all(ref, xs, ix)
        for t in sorted({0, T - 1}):
            assert_close(on[t], ref.token(xs[t]).out, f"{name} T={T} out[{t}]")


def test_noalloc_too_large_is_refused(gpu_device):
    L = DeviceLayer(synth.WORKLOADS["tiny"])
    T = 1
    while bq.moe_workspace_bytes(L.desc, T) <= bq.MOE_NOALLOC_SCRATCH_BYTES:
        T *= 2
    x = torch.zeros(T, L.w.hidden, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(bq.MoeError) as e:
        bq.moe_layer_forward_noalloc(L.desc, x, x, T, out, None)
    assert e.value.code == bq.MOE_ENOSPC
