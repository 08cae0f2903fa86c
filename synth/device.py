"""Allocate a workload's inputs in device memory (PyTorch) and fill them in place with
the HIP twin of the seeded generator.  Memory plumbing only; no decode arithmetic."""
from __future__ import annotations

import numpy as np
import torch

from . import native, workloads


def _tdtype(d: str):
    return torch.float32 if d == "f32" else torch.bfloat16


class DeviceInputs:
    """Weights (canonical order), K/V caches [layers, batch, kv_heads, capacity, hd],
    tokens, positions and a logits buffer for workload ``w`` on ``device``."""

    def __init__(self, w: "workloads.Workload", device: str = "cuda", fill: bool = True, weights=None):
        """``weights``: reuse another instance's weight tensors (same model shape) and
        allocate only caches, tokens, positions and logits."""
        self.w = w
        self.device = torch.device(device)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        self.weights = []
        if weights is not None:
            specs = w.weight_specs()
            assert len(weights) == len(specs)
            assert all(tuple(t.shape) == tuple(sp[2]) for t, sp in zip(weights, specs))
            self.weights = list(weights)
        for tid, name, shape, mean, std, dtype in (w.weight_specs() if weights is None else []):
            t = torch.empty(shape, dtype=_tdtype(dtype), device=self.device)
            if fill:
                native.gpu_fill_flat(t.data_ptr(), t.numel(), 0, w.seed, tid, mean, std, dtype, stream)
            self.weights.append(t)
        cshape = (w.n_layers,) + w.cache_shape()
        self.kcache = torch.empty(cshape, dtype=_tdtype(w.kv_dtype), device=self.device)
        self.vcache = torch.empty(cshape, dtype=_tdtype(w.kv_dtype), device=self.device)
        if fill:
            self.refill_caches()
        self.tokens = torch.from_numpy(w.tokens()).to(self.device)
        self.positions = torch.from_numpy(w.positions()).to(self.device)
        self.logits = torch.empty((w.batch, w.vocab), dtype=torch.float32, device=self.device)

    def refill_caches(self) -> None:
        """Restore both caches to the seeded pre-filled state."""
        w = self.w
        stream = torch.cuda.current_stream(self.device).cuda_stream
        for l in range(w.n_layers):
            for which, cache in ((workloads.KCACHE, self.kcache), (workloads.VCACHE, self.vcache)):
                native.gpu_fill_cache(cache[l].data_ptr(), w.batch * w.n_kv_heads, w.kv_capacity, w.head_dim,
                                      w.seed, w.tid_layer(l, which), 0.0, workloads.KV_STD, w.kv_dtype, stream)

    def packed_weights(self):
        """The weight list with every matrix (W_qkv, W_o, W_gate_up, W_down, W_lm) copied
        into the library's 16-row tile layout by mk_pack_matrix, for graphs lowered with
        MK_LOWER_PACKED_WEIGHTS; the other tensors are shared, self.weights is unchanged."""
        from task_graph_interpreter_amd import binding as mk

        stream = torch.cuda.current_stream(self.device).cuda_stream
        out = list(self.weights)
        for i in mk.packed_matrix_indices(self.w.n_layers):
            src = self.weights[i]
            dst = torch.empty_like(src)
            mk.mk_pack_matrix(src.data_ptr(), dst.data_ptr(), src.shape[0], src.shape[1], stream)
            out[i] = dst
        return out

    def weight_ptrs(self):
        return [t.data_ptr() for t in self.weights]

    def step_ptrs(self):
        """(tokens, positions, kcache, vcache, logits) device addresses."""
        return (self.tokens.data_ptr(), self.positions.data_ptr(), self.kcache.data_ptr(),
                self.vcache.data_ptr(), self.logits.data_ptr())

    def set_step(self, tokens: np.ndarray, positions: np.ndarray) -> None:
        self.tokens.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.positions.copy_(torch.from_numpy(np.asarray(positions, dtype=np.int32)))
