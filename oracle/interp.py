"""CPU descriptor interpreter -- TEST INFRASTRUCTURE ONLY.

Runs a lowered task array (from either lowering) on the CPU in any order that the
edge array allows, the way the on-GPU interpreter of "Megakernels" (runhoid.com,
section "Hoid's approach to megakernels") runs one unit of work as soon as its direct
producers have finished.  Each task reads only its descriptor (OpId, flags, buffer
indices, m/n/k, reserved fields, as laid out in "Mega kernel initial", descriptor
section).  Activation buffers start as NaN, so a read that no edge orders after its
write shows up as NaN or as a difference between two random orders.  Arithmetic is
float64 and identical for every order, so any two valid orders agree bit for bit.

A task left with unmet dependencies (for instance a corrupted remaining_deps) stops
the run with ``Stalled`` instead of hanging.
"""
from __future__ import annotations

import numpy as np

from . import decode as od
from .graph import APPEND, BufferIndex, COMBINE, FUSED_RESIDUAL, GEMV, MEMCPY, NOP, PARTIAL, RMSNORM, \
    RMS_NORM_INPUT, SAMPLE, SILU_MUL, ADD_RESIDUAL


class Stalled(RuntimeError):
    pass


def _act_shapes(w):
    bi = BufferIndex(w)
    B, H, hd = w.batch, w.hidden, w.head_dim
    slots = sum(w.chunks(b) for b in range(B)) * w.n_kv_heads
    L_ = w.n_layers
    shapes = {bi.x0: (B, H), bi.logits: (B, w.vocab)}
    for l in range(w.n_layers):
        shapes[bi.act(l, 0)] = (B, w.qkv_cols)
        shapes[bi.act(l, 1)] = (B, w.q_cols)
        shapes[bi.act(l, 2)] = (slots, w.grp, hd + 2)
        shapes[bi.act(l, 3)] = (B, w.q_cols)
        shapes[bi.act(l, 4)] = (B, H)
        shapes[bi.act(l, 5)] = (B, w.intermediate)
        shapes[bi.act(l, 6)] = (B, H)
        if bi.unfused:
            for j in range(4):
                shapes[bi.extra(l, j)] = (B, H)
    if bi.unfused:
        shapes[bi.extra(L_, 0)] = (B, H)
    return shapes


class Interpreter:
    def __init__(self, w, params, tokens, positions):
        self.w, self.p = w, params
        self.tokens = np.array(tokens, dtype=np.int64)
        self.positions = np.array(positions, dtype=np.int64)
        self.buf = {k: np.full(s, np.nan) for k, s in _act_shapes(w).items()}
        self.cache = {}  # (layer, which, b, g) -> float64[pos+1, hd], pre-filled slots
        for l in range(w.n_layers):
            for b in range(w.batch):
                for g in range(w.n_kv_heads):
                    for which in (0, 1):
                        self.cache[(l, which, b, g)] = params.cache(l, which, b, g, int(self.positions[b]) + 1)
        self.bi = BufferIndex(w)

    def _layer_of_cache(self, buf):
        return (buf - 3) // 8, (buf - 3) % 8 - 6

    def run_task(self, d):
        w, bi = self.w, self.bi
        op = int(d["op_id"])
        r = [int(v) for v in d["reserved"]]
        inb = [int(v) for v in d["in_buf"]]
        out = int(d["out_buf"])
        m, n, k = int(d["m"]), int(d["n"]), int(d["k"])
        hd = w.head_dim
        if op == NOP:
            return
        if op == MEMCPY:
            for b in range(m):
                self.buf[out][b] = self.p.embedding_row(int(self.tokens[b]))
            return
        if op == GEMV:
            c0, cnt, I = r[0], r[1], r[2]
            flags = int(d["flags"])
            x = self.buf[inb[0]][:, :k]
            if flags & RMS_NORM_INPUT:
                gamma = self.p.vector(inb[2])
                x = np.stack([od.rmsnorm(x[b], gamma, w.rms_eps) for b in range(m)])
            W = self.p.matrix(inb[1])
            if flags & SILU_MUL:
                gt = x @ W[c0:c0 + cnt].T
                up = x @ W[I + c0:I + c0 + cnt].T
                y = od.silu(gt) * up
            else:
                y = x @ W[c0:c0 + cnt].T
            if flags & ADD_RESIDUAL:
                y = y + self.buf[inb[2]][:, c0:c0 + cnt]
            self.buf[out][:, c0:c0 + cnt] = y
            return
        if op == APPEND:
            b, h0, hc, kc, vc = r
            g = k
            pos = int(self.positions[b])
            row = self.buf[inb[0]][b]
            Hq, Hkv = w.n_q_heads, w.n_kv_heads
            q = row[h0 * hd:(h0 + hc) * hd].reshape(hc, hd)
            kk = row[Hq * hd + g * hd: Hq * hd + (g + 1) * hd]
            vv = row[(Hq + Hkv) * hd + g * hd: (Hq + Hkv) * hd + (g + 1) * hd]
            self.buf[out][b, h0 * hd:(h0 + hc) * hd] = od.rope(q, pos, w.rope_theta).reshape(-1)
            lk, _ = self._layer_of_cache(kc)
            self.cache[(lk, 0, b, g)][pos] = od.round_storage(od.rope(kk, pos, w.rope_theta), w.kv_dtype)
            self.cache[(lk, 1, b, g)][pos] = od.round_storage(vv, w.kv_dtype)
            return
        if op == PARTIAL:
            b, h0, hc, c, bs = r
            g = k
            chunk = int(d["kv_len"])
            pos = int(self.positions[b])
            lk, _ = self._layer_of_cache(inb[1])
            K = self.cache[(lk, 0, b, g)]
            V = self.cache[(lk, 1, b, g)]
            hi = min((c + 1) * chunk, pos + 1)
            lo = min(c * chunk, hi)
            qr = self.buf[inb[0]][b]
            for j in range(hc):
                mm, ll, oo = od.chunk_partial(qr[(h0 + j) * hd:(h0 + j + 1) * hd], K[lo:hi], V[lo:hi])
                slot = self.buf[out][bs + c, j]
                slot[:hd] = oo
                slot[hd] = mm
                slot[hd + 1] = ll
            return
        if op == COMBINE:
            b, h0, hc, _, bs = r
            P = self.buf[inb[0]]
            for j in range(hc):
                parts = [(P[bs + c, j, hd], P[bs + c, j, hd + 1], P[bs + c, j, :hd]) for c in range(m)]
                self.buf[out][b, (h0 + j) * hd:(h0 + j + 1) * hd] = od.combine(parts)
            return
        if op == RMSNORM:
            b = r[0]
            v = self.buf[inb[0]][b].copy()
            if int(d["flags"]) & FUSED_RESIDUAL:
                v = v + self.buf[inb[2]][b]
                self.buf[r[1]][b] = v
            self.buf[out][b] = od.rmsnorm(v, self.p.vector(inb[1]), w.rms_eps)
            return
        if op == SAMPLE:
            # tokens and positions are the step's inputs, updated in place: every task
            # that reads them must have run already (the edges guarantee it)
            b = r[0]
            self.tokens[b] = od.greedy_token(self.buf[inb[0]][b])
            self.positions[b] += 1
            return
        raise ValueError(f"op {op} not run by this interpreter")

    def run(self, tasks, edges, order_seed=None):
        """Execute all tasks; order_seed None = emission order, "lifo" = the task that
        became ready last (runs consumers as early as the edges allow), an integer = a
        random ready task at each step.  Returns the logits buffer."""
        n = len(tasks)
        remaining = tasks["remaining_deps"].astype(np.int64).copy()
        offs = tasks["dependents_offset"].astype(np.int64)
        deg = tasks["num_dependents"].astype(np.int64)
        lifo = order_seed == "lifo"
        rng = None if order_seed is None or lifo else np.random.default_rng(order_seed)
        ready = [t for t in range(n) if remaining[t] == 0]
        done = 0
        while ready:
            if lifo:
                t = ready.pop()
            elif rng is None:
                ready.sort()
                t = ready.pop(0)
            else:
                t = ready.pop(int(rng.integers(len(ready))))
            self.run_task(tasks[t])
            done += 1
            for c in edges[offs[t]:offs[t] + deg[t]]:
                c = int(c)
                remaining[c] -= 1
                if remaining[c] == 0:
                    ready.append(c)
        if done != n:
            raise Stalled(f"no ready task: {done} of {n} tasks ran")
        return self.buf[self.bi.logits]
