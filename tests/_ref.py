"""Oracle-side helpers for the GPU tests: per-token references from the fp64 oracle, fed by the
host generator (never by the GPU path)."""
from __future__ import annotations

import functools
import multiprocessing
from concurrent.futures import ProcessPoolExecutor

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

    def token(self, x, res=None) -> oracle.LayerResult:
        x = np.asarray(x, dtype=np.float64)
        res = x if res is None else np.asarray(res, dtype=np.float64)
        return oracle.layer(x, res, self.router, self.gate, self.expert, self.w.top_k, self.w.group,
                            shared_expert=self.shared)

    def expert_out(self, x, e: int):
        ex = self.shared if e == synth.SHARED else self.expert(e)
        return oracle.expert(np.asarray(x, dtype=np.float64), ex, self.w.group)


def spread(N: int, n: int) -> list:
    """n token positions spread evenly over 0..N-1, both ends included."""
    return sorted({int(round(v)) for v in np.linspace(0, N - 1, n)})


def check_topk_all(ref: Reference, xs, idx_gpu, what="token"):
    """Every token's top-K against oracle.topk of the oracle's fp64 router logits. A mismatch fails
    and names the fp64 margin (K-th minus (K+1)-th logit) at that decision."""
    K = ref.w.top_k
    bad = []
    for t in range(len(xs)):
        lg = oracle.router_logits(ref.router, np.asarray(xs[t], dtype=np.float64))
        want = oracle.topk(lg, K)
        if list(idx_gpu[t]) != list(want):
            order = np.sort(lg)[::-1]
            margin = float(order[K - 1] - order[K]) if K < len(order) else float("inf")
            bad.append(f"{what} {t}: gpu {list(idx_gpu[t])} oracle {list(want)} fp64 margin {margin:.3e}")
    assert not bad, f"{len(bad)} top-K mismatches: " + "; ".join(bad[:8])


_STACK_REFS = {}


def _one_thread():
    # set before the worker first loads the oracle library, whose OpenMP runtime reads it once
    import os
    os.environ["OMP_NUM_THREADS"] = "1"


def _stack_token(args):
    name, n_layers, x = args
    w = synth.WORKLOADS[name]
    if name not in _STACK_REFS:
        _STACK_REFS[name] = [Reference(w, l, cache=1) for l in range(n_layers)]
    layers = [(r.router, r.gate, r.expert, r.shared) for r in _STACK_REFS[name]]
    return oracle.stack(x, layers, w.top_k, w.group, STACK_EPS)


STACK_EPS = 1e-6


def stack_oracle_parallel(name: str, n_layers: int, xs, workers: int = 8):
    """oracle.stack for several tokens of a named workload, one token per task in single-threaded
    CPU-only worker processes (spawned, so they never touch the GPU). Returns the pool and the
    futures, so the caller can run GPU work meanwhile; it shuts the pool down."""
    ctx = multiprocessing.get_context("spawn")
    pool = ProcessPoolExecutor(max_workers=min(workers, len(xs)), mp_context=ctx, initializer=_one_thread)
    futs = [pool.submit(_stack_token, (name, n_layers, np.asarray(x, dtype=np.float64))) for x in xs]
    return pool, futs
