"""Helpers for the GPU parity tests: run the library on a workload through the C ABI
and read back logits and every activation buffer for comparison with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import task_graph_interpreter_amd as mk
from task_graph_interpreter_amd import binding
from oracle import graph as og
from synth.device import DeviceInputs

# The contract on logits: |gpu - ref| <= ATOL + RTOL |ref| for every element (the
# tolerance stated for bf16 weights with fp32 accumulation).
ATOL, RTOL = 2e-2, 1e-2

# Tighter bounds, per arithmetic path, fixed before any run and derived from what
# each path rounds (the oracle is float64 and models the storage roundings of the
# cache rows, so what is left is the path's own arithmetic):
#  * "f32": fp32 weights, cache and activations; every GEMV output is a chain of
#    fp32 FMAs over K <= 512 terms of size ~|x||w|, so its error is a few ulp of the
#    sum of |terms| (~1e-7 relative): 1e-5 leaves two orders of magnitude of room.
#  * "bf16": bf16 weights and cache (exact in fp32), fp32 vector arithmetic: the
#    same fp32 rounding per dot product (K up to 14336), compounded through the
#    layers' residual stream (up to 32 layers): 2e-4 abs and rel (the 8B-class
#    batch-1 step's logits reach 1.7e-5, the tiny bf16 activations 3e-6).
#  * "mfma": the matrix-core GEMV takes its fp32 input as a bf16 hi + lo pair (16
#    significant bits, relative error <= 2^-17 per element), so each dot product
#    carries an extra ~1e-5 relative error on top of the "bf16" path: 5e-3.
TIERS = {"f32": (1e-5, 1e-5), "bf16": (2e-4, 2e-4), "mfma": (5e-3, 5e-3)}


def tier_of(w) -> str:
    if w.weight_dtype == "f32":
        return "f32"
    return "mfma" if w.gemv_config == 2 else "bf16"


def check_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err - bound, -np.inf)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements out of tolerance "
                             f"(atol {atol:g}, rtol {rtol:g}); worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}; "
                             f"max_abs={err.max():.3e}")
    return float(err.max())


def check_logits(gpu, ref, w, what="logits"):
    """Logits against the contract (A17) and against the path's own tighter tier.
    Returns the largest absolute difference."""
    check_close(gpu, ref, what + " (contract)")
    atol, rtol = TIERS[tier_of(w)]
    return check_close(gpu, ref, f"{what} ({tier_of(w)} tier)", atol, rtol)


def tie_bound(ref_row, tol) -> float:
    """Largest oracle top-2 margin that logits within tolerance ``tol`` = (atol,
    rtol) could still reverse: two candidates' logits can each move by atol + rtol
    |logit|, in opposite directions."""
    atol, rtol = tol
    return 2.0 * (atol + rtol * float(np.max(np.abs(ref_row))))


def check_tokens(gpu_logits, ref_logits, tol, what="tokens"):
    """Greedy tokens per row (argmax, lowest index on ties) asserted equal to the
    oracle's.  A row is exempt only when the oracle's own top-2 margin is below
    tie_bound(row, tol), with ``tol`` the tolerance the path's logits are held to
    (fixed before the run, never the measured error): logits inside that tolerance
    could then pick another candidate.  In an exempt row the GPU's pick must still
    be a candidate within the bound of the oracle's top-1 logit.  Every exempt row
    is printed with its margin.  Returns the GPU's tokens and the exempt rows."""
    toks, exempt = [], []
    for b, (g, r) in enumerate(zip(np.asarray(gpu_logits, np.float64), np.asarray(ref_logits, np.float64))):
        tg, tr = int(np.argmax(g)), int(np.argmax(r))
        toks.append(tg)
        tau = tie_bound(r, tol)
        s = np.sort(r)
        margin = float(s[-1] - s[-2])
        if margin >= tau:
            assert tg == tr, (f"{what}: row {b} picks {tg}, oracle {tr}; oracle top-2 margin {margin:.3e} "
                              f">= tie bound {tau:.3e}")
        else:
            gap = float(r[tr] - r[tg])
            assert gap <= tau, (f"{what}: row {b} picks {tg}, oracle {tr}; the pick is {gap:.3e} below the "
                                f"oracle's top-1 logit, beyond the tie bound {tau:.3e}")
            exempt.append(b)
            print(f"[{what}] row {b}: oracle top-2 margin {margin:.3e} < tie bound {tau:.3e}; "
                  f"gpu {tg}, oracle {tr}", flush=True)
    return toks, exempt


class MkRun:
    """Inputs on the GPU + an uploaded graph for workload ``w``."""

    def __init__(self, w, inputs: DeviceInputs | None = None):
        self.w = w
        self.inp = inputs or DeviceInputs(w)
        self.cfg, self._keep = mk.make_cfg(**w.mk_fields())
        self.plan = mk.mk_plan(self.cfg)
        self.scratch = torch.zeros(max(self.plan["scratch_bytes"], 256), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream
        # Packed graphs get their own tile-layout copies of the matrices; inputs shared
        # with a row-major run stay as they are.
        self.weights = self.inp.packed_weights() if w.packed else self.inp.weights
        self.graph = mk.mk_build_graph(self.cfg, [t.data_ptr() for t in self.weights], self.scratch.data_ptr(),
                                       self.stream)
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
            if bi.unfused:
                for j, nm in enumerate(["xn", "o", "hn", "d"]):
                    out[f"l{l}.{nm}"] = self.activation(bi.extra(l, j)).reshape(w.batch, -1)
        if bi.unfused:
            out["xn_final"] = self.activation(bi.extra(w.n_layers, 0)).reshape(w.batch, -1)
        return out

    def close(self):
        self.graph.close()


def slot_index(w, b, g, c):
    base = 0
    for bb in range(b):
        base += w.n_kv_heads * w.chunks(bb)
    return base + g * w.chunks(b) + c


def compare_activations(w, gpu: dict, ref: dict, rows, tol=None):
    """Every activation buffer of the GPU step against the oracle's, for batch rows
    ``rows``, at the path's tier (or ``tol`` = (atol, rtol)).  Partial slots: m to
    atol + rtol |m|; l and o, which are sums of e^(s - m) with up to chunk terms of
    size <= 1, to atol max(1, l) + rtol |value|.  Returns the largest absolute
    difference per activation kind."""
    atol, rtol = tol if tol is not None else TIERS[tier_of(w)]
    worst = {}
    rows = list(rows)

    def note(kind, e):
        worst[kind] = max(worst.get(kind, 0.0), e)

    standard = {"x0"} | {f"l{l}.{nm}" for l in range(w.n_layers)
                         for nm in ("qkv_out", "q_rot", "partials", "att", "h", "gu", "x_out")}
    assert standard <= set(gpu), "the GPU step is missing an activation buffer"
    for name, rv in ref.items():
        if name not in gpu:  # buffers of the unfused graph only
            continue
        kind = name.split(".")[-1]
        if name.endswith("partials"):
            gv = gpu[name]
            for (b, g, c, j), (m, l, o) in rv.items():
                s = gv[slot_index(w, b, g, c), j]
                tag = f"{name}[b{b} g{g} c{c} h{j}]"
                if m == -np.inf:
                    assert s[w.head_dim] == -np.inf and s[w.head_dim + 1] == 0, tag
                    continue
                note("partials.m", check_close(s[w.head_dim], m, tag + ".m", atol=atol, rtol=rtol))
                note("partials.l", check_close(s[w.head_dim + 1], l, tag + ".l", atol=atol * max(1.0, l), rtol=rtol))
                note("partials.o", check_close(s[:w.head_dim], o, tag + ".o", atol=atol * max(1.0, l), rtol=rtol))
            continue
        note(kind, check_close(gpu[name][rows], rv, name, atol=atol, rtol=rtol))
    print("[activations] max|d| " + " ".join(f"{k}={v:.2e}" for k, v in sorted(worst.items())), flush=True)
    return worst
