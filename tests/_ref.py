"""Oracle-side helpers for the GPU tests: per-token references from the fp64 oracle, fed by the
host generator (never by the GPU path)."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

RTOL, ATOL = 2e-3, 1e-5  # max|gpu - oracle| <= RTOL * max|oracle| + ATOL, per token vector


def assert_close(gpu, ref, what="output"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    g2 = gpu.reshape(-1, gpu.shape[-1]) if gpu.ndim > 1 else gpu[None]
    r2 = ref.reshape(-1, ref.shape[-1]) if ref.ndim > 1 else ref[None]
    for i, (g, r) in enumerate(zip(g2, r2)):
        err = np.max(np.abs(g - r))
        bound = RTOL * np.max(np.abs(r)) + ATOL
        assert np.all(np.isfinite(g)), f"{what}[{i}]: non-finite values"
        assert err <= bound, f"{what}[{i}]: max err {err:.3e} > bound {bound:.3e} (max|ref| {np.max(np.abs(r)):.3e})"


class Reference:
    """Oracle results for one workload layer, with the canonical arrays of experts cached."""

    def __init__(self, w: synth.Workload, layer: int = 0, cache: int = 24):
        self.w, self.layer = w, layer
        self.router = synth.router_weights(w, layer)
        self.gate = synth.shared_gate_weights(w, layer) if w.has_shared else None
        self._experts = functools.lru_cache(maxsize=cache)(lambda e: synth.expert_arrays(w, layer, e))
        self.shared = self._experts(synth.SHARED) if w.has_shared else None

    def expert(self, e: int):
        return self._experts(e)

    def token(self, x, res=None, force_idx=None) -> oracle.LayerResult:
        x = np.asarray(x, dtype=np.float64)
        res = x if res is None else np.asarray(res, dtype=np.float64)
        return oracle.layer(x, res, self.router, self.gate, self.expert, self.w.top_k, self.w.group,
                            shared_expert=self.shared, force_idx=force_idx)

    def expert_out(self, x, e: int):
        ex = self.shared if e == synth.SHARED else self.expert(e)
        return oracle.expert(np.asarray(x, dtype=np.float64), ex, self.w.group)
