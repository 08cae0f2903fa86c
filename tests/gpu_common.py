"""Helpers for the GPU parity tests: run the library on a workload through the C ABI
and read back logits and every activation buffer for comparison with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import task_graph_interpreter_amd as mk
from task_graph_interpreter_amd import binding
from oracle import graph as og
from synth.device import DeviceInputs

ATOL, RTOL = 2e-2, 1e-2  # |gpu - ref| <= ATOL + RTOL * |ref|, every element


def check_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance; "
                             f"worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}; max_abs={err.max():.3e}")
    return float(err.max())


def check_tokens(gpu_logits, ref_logits, what="tokens"):
    """Greedy tokens per row: equal to the oracle's, except where the oracle's own
    top-1 logit and the logit of the GPU's pick differ by less than twice the row's
    largest measured logit error (a tie within error: the GPU's pick must then be one of
    the near-tied candidates).  Returns the rows that were ties within error."""
    ties = []
    for b, (g, r) in enumerate(zip(np.asarray(gpu_logits, np.float64), np.asarray(ref_logits, np.float64))):
        tg, tr = int(np.argmax(g)), int(np.argmax(r))
        if tg == tr:
            continue
        err = float(np.max(np.abs(g - r)))
        margin = float(r[tr] - r[tg])
        assert margin <= 2.0 * err, (f"{what}: row {b} picks {tg}, oracle {tr}; oracle margin {margin:.3e} "
                                     f"exceeds twice the row's logit error {err:.3e}")
        ties.append(b)
    if ties:
        print(f"[{what}] tie within error on rows {ties}", flush=True)
    return ties


class MkRun:
    """Inputs on the GPU + an uploaded graph for workload ``w``."""

    def __init__(self, w, inputs: DeviceInputs | None = None):
        self.w = w
        self.inp = inputs or DeviceInputs(w)
        self.cfg, self._keep = mk.make_cfg(**w.mk_fields())
        self.plan = mk.mk_plan(self.cfg)
        self.scratch = torch.zeros(max(self.plan["scratch_bytes"], 256), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream
        self.graph = mk.mk_build_graph(self.cfg, self.inp.weight_ptrs(), self.scratch.data_ptr(), self.stream)
        self.lowered = mk.mk_lower(self.cfg)
        self.bi = og.BufferIndex(w)

    def step(self, path: str = "persistent", check_status: bool = True) -> np.ndarray:
        fn = self.graph.mk_decode_step if path == "persistent" else self.graph.mk_decode_step_per_op
        fn(self.stream, *self.inp.step_ptrs())
        if check_status:
            st = self.graph.mk_status()
            assert st == 0, f"device status 0x{st:08x}"
        torch.cuda.synchronize()
        return self.inp.logits.cpu().numpy().astype(np.float64)

    def activation(self, buf: int) -> np.ndarray:
        off, nb = self.lowered.scratch_span(buf)
        return self.scratch[off:off + nb].view(torch.float32).cpu().numpy().astype(np.float64)

    def activations(self):
        """GPU activations keyed like the oracle's intermediates."""
        w, bi = self.w, self.bi
        out = {"x0": self.activation(bi.x0).reshape(w.batch, w.hidden)}
        names = ["qkv_out", "q_rot", "partials", "att", "h", "gu", "x_out"]
        for l in range(w.n_layers):
            for j, nm in enumerate(names):
                a = self.activation(bi.act(l, j))
                if nm == "partials":
                    a = a.reshape(-1, w.grp, w.head_dim + 2)
                else:
                    a = a.reshape(w.batch, -1)
                out[f"l{l}.{nm}"] = a
        return out

    def close(self):
        self.graph.close()


def slot_index(w, b, g, c):
    base = 0
    for bb in range(b):
        base += w.n_kv_heads * w.chunks(bb)
    return base + g * w.chunks(b) + c


def compare_activations(w, gpu: dict, ref: dict, rows):
    """Every activation buffer of the GPU step against the oracle's, for batch rows ``rows``."""
    worst = {}
    rows = list(rows)
    for name, rv in ref.items():
        if name.endswith("partials"):
            gv = gpu[name]
            for (b, g, c, j), (m, l, o) in rv.items():
                s = gv[slot_index(w, b, g, c), j]
                tag = f"{name}[b{b} g{g} c{c} h{j}]"
                if m == -np.inf:
                    assert s[w.head_dim] == -np.inf and s[w.head_dim + 1] == 0, tag
                    continue
                check_close(s[w.head_dim], m, tag + ".m", atol=1e-3, rtol=1e-4)
                # l and o are sums of e^(s - m); a relative bound in the size of the sum
                check_close(s[w.head_dim + 1], l, tag + ".l", atol=1e-3 * max(1.0, l), rtol=1e-3)
                check_close(s[:w.head_dim], o, tag + ".o", atol=2e-3 * max(1.0, l), rtol=1e-2)
            continue
        worst[name] = check_close(gpu[name][rows], rv, name)
    return worst
