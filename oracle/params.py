"""Oracle-side view of the seeded weights and caches -- TEST INFRASTRUCTURE ONLY.

Regenerates any tensor (or slice of a cache) from the seeded generator of the
``synth`` package and widens it exactly to float64.  Small workloads use the numpy
generator; large ones the C twin of the same generator (bit-identical, checked by
the tests).  Nothing here comes from the GPU.
"""
from __future__ import annotations

import numpy as np

from synth import gen, workloads


class GeneratedParams:
    def __init__(self, w: "workloads.Workload", backend: str = "auto"):
        self.w = w
        if backend == "auto":
            backend = "numpy" if w.weight_bytes_per_step() < 64 << 20 else "c"
        self.backend = backend
        self.specs = {s[0]: s for s in w.weight_specs()}
        self._small = {}

    def _flat(self, tid: int, n: int, start: int = 0) -> np.ndarray:
        _, _, _, mean, std, dtype = self.specs[tid]
        if self.backend == "numpy":
            return gen.to_f64(gen.fill(self.w.seed, tid, n, mean, std, dtype, start=start), dtype)
        from synth import native
        return native.cpu_fill_flat_f64(n, start, self.w.seed, tid, mean, std, dtype)

    def embedding_row(self, token: int) -> np.ndarray:
        H = self.w.hidden
        return self._flat(2, H, start=token * H)

    def vector(self, tid: int) -> np.ndarray:
        if tid not in self._small:
            shape = self.specs[tid][2]
            self._small[tid] = self._flat(tid, int(np.prod(shape))).reshape(shape)
        return self._small[tid]

    def matrix(self, tid: int) -> np.ndarray:
        shape = self.specs[tid][2]
        return self._flat(tid, int(np.prod(shape))).reshape(shape)

    def cache(self, layer: int, which: int, b: int, g: int, n: int) -> np.ndarray:
        """Pre-filled slots [0, n) of cache ``which`` (0 = K, 1 = V) for sequence b, KV head g."""
        w = self.w
        tid = w.tid_layer(layer, workloads.KCACHE + which)
        bg = b * w.n_kv_heads + g
        if self.backend == "numpy":
            slot, d = np.meshgrid(np.arange(n), np.arange(w.head_dim), indexing="ij")
            idx = gen.cache_index(np.full_like(slot, bg), slot, d, w.head_dim)
            raw = gen.values(w.seed, tid, idx, 0.0, workloads.KV_STD, w.kv_dtype)
        else:
            from synth import native
            raw = native.cpu_fill_cache(bg, 1, 0, n, w.head_dim, w.seed, tid, 0.0, workloads.KV_STD,
                                        w.kv_dtype)[0]
        return gen.to_f64(raw, w.kv_dtype).reshape(n, w.head_dim)
