"""Build a workload's layers in device memory.

Canonical arrays are generated in place on the GPU by the seeded fill kernels, then packed into
blobs by the library's device packer. The result matches, byte for byte, what the host
generator plus the host packer would produce (tests check this on sampled experts). Used by
the GPU tests and the benchmark.
"""
from __future__ import annotations

import numpy as np
import torch

import bit_quantized_expert_gemv_amd as bq
import synth


def _i16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


class DeviceLayer:
    """One MoE layer resident in HBM: E expert blobs, the shared expert, router and shared gate."""

    def __init__(self, w: synth.Workload, layer: int = 0, device="cuda", stream=None):
        self.w, self.layer = w, layer
        H, I, E = w.hidden, w.inter, w.n_experts
        self.blob_bytes = bq.moe_blob_bytes(H, I, w.bits, w.group)
        self.stride = (self.blob_bytes + 255) // 256 * 256
        self.experts = torch.empty(E * self.stride, dtype=torch.uint8, device=device)
        self.shared = torch.empty(self.stride, dtype=torch.uint8, device=device) if w.has_shared else None
        s = bq.stream_handle(stream)
        q = [torch.empty(r * c, dtype=torch.uint8, device=device) for r, c in map(w.matrix_shape, range(3))]
        sc = [torch.empty(r * c // w.group, dtype=torch.int16, device=device) for r, c in map(w.matrix_shape, range(3))]
        bi = [torch.empty_like(t) for t in sc] if w.fmt == "affine" else [None] * 3
        targets = [(e, self.experts.data_ptr() + e * self.stride) for e in range(E)]
        if w.has_shared:
            targets.append((synth.SHARED, self.shared.data_ptr()))
        for e, dst in targets:
            for m in range(3):
                synth.fill_matrix_device(w, layer, e, m, q[m].data_ptr(), sc[m].data_ptr(),
                                         bi[m].data_ptr() if bi[m] is not None else 0, s)
            bq.moe_pack_expert_device(H, I, w.bits, w.group, q, sc, bi, dst, s)
        self.router = _i16(synth.router_weights(w, layer)).to(device)
        self.shared_gate = _i16(synth.shared_gate_weights(w, layer)).to(device) if w.has_shared else None
        self.desc = bq.make_layer(H, I, E, w.top_k, w.bits, self.experts, self.stride, self.router,
                                  self.shared, self.shared_gate, w.group)

    def expert_blob(self, e: int) -> torch.Tensor:
        if e == synth.SHARED:
            return self.shared[: self.blob_bytes]
        return self.experts[e * self.stride: e * self.stride + self.blob_bytes]

    def weight_bytes(self) -> int:
        n = self.experts.numel() + (self.shared.numel() if self.shared is not None else 0)
        return n + self.router.numel() * 2 + (self.shared_gate.numel() * 2 if self.shared_gate is not None else 0)
