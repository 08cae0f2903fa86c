"""Oracle lowering: decode step -> 64-byte task descriptors + CSR edges -- TEST
INFRASTRUCTURE ONLY.

An independent Python statement of the lowering in "Mega kernel initial"
(1y33.com): the lowering section (one GEMV task per output-column tile, one
ATTENTION_PARTIAL per (sequence, KV-head group, KV chunk) and a combine, RMSNorm /
residual / SiLU*mul as GEMV flags, the final norm fused into the lm_head GEMV), the
descriptor section (the 64-byte struct, uint16 buffer-table indices, per-op use of
``reserved``, flag bits), the edge section (each task records the tasks that wrote
the column ranges it reads; parents are inverted into one flat dependents array in
topological emission order) and the OpId table.  Its bytes must equal the C++
lowering's bytes.

Rules (the pages leave the exact field map open; this is the convention both
builders follow):
  R1 emission: MEMCPY; per layer qkv tiles, APPEND (b, g), PARTIAL (b, g, c),
     COMBINE (b, g), o tiles, gate_up tiles, down tiles; lm_head tiles.  A join NOP
     is emitted just before the op whose shared parents it joins.
  R2 tile i of T over N columns is [floor(iN/T), floor((i+1)N/T)); with the MFMA GEMV
     variant the bounds are 16 * floor(i (N/16) / T).
  R3 sequence b has ceil(kv_len[b] / kv_chunk) chunks; chunk c covers keys
     [c*chunk, (c+1)*chunk) clipped to the runtime length positions[b] + 1.
  R4 reads and writes are (row range) x (column range) rectangles of a buffer.
  R5 parents = every earlier task whose write overlaps one of the task's reads,
     ascending, without duplicates; remaining_deps = number of parents.
  R6 dependents of a task = its children ascending; dependents_offset = exclusive
     prefix sum of num_dependents; edges are uint32 child indices.
  R9 joins: for an op with >= 2 tasks whose tasks share >= 2 parents S, a NOP with
     parents S is emitted and each task's parents become (own - S) + {NOP}.
Parity: pinned by the page's worked tiling example (3072 columns in 8 tiles of 384),
the descriptor layout and OpId/flag values printed on the page, and by the invariants
in ``check_graph`` (topological order, read-after-write coverage, in-degrees, SSA).
"""
from __future__ import annotations

import numpy as np

TASK_DTYPE = np.dtype({
    "names": ["op_id", "config_id", "step", "flags", "remaining_deps", "num_dependents",
              "dependents_offset", "in_buf", "out_buf", "m", "n", "k", "kv_len", "reserved"],
    "formats": ["<u2", "<u2", "<u2", "<u2", "<i4", "<i4", "<u4", ("<u2", (3,)), "<u2", "<i4", "<i4",
                "<i4", "<i4", ("<u4", (5,))],
    "offsets": [0, 2, 4, 6, 8, 12, 16, 20, 26, 28, 32, 36, 40, 44],
    "itemsize": 64,
})
assert TASK_DTYPE.itemsize == 64

# OpId table of the page.
NOP, MEMCPY, GEMV, RMSNORM, ATTENTION, MLP, SAMPLE, APPEND, PARTIAL, COMBINE = range(10)
# Flag bits of the page.
SILU_MUL, ADD_RESIDUAL, RMS_NORM_INPUT = 1, 2, 4
NONE = 0xFFFF


class BufferIndex:
    """Canonical buffer-table indices (append-only order)."""

    def __init__(self, w):
        L = w.n_layers
        self.tokens, self.positions, self.embedding = 0, 1, 2
        self.final_norm = 3 + 8 * L
        self.w_lm = 4 + 8 * L
        self.scratch0 = 5 + 8 * L
        self.x0 = self.scratch0
        self.logits = self.scratch0 + 1 + 7 * L
        self.count = self.logits + 1

    @staticmethod
    def layer(l, which):
        return 3 + 8 * l + which

    def act(self, l, which):
        """which: 0 qkv_out, 1 q_rot, 2 partials, 3 att, 4 h, 5 gu, 6 x_out."""
        return self.scratch0 + 1 + 7 * l + which


def tile_bounds(N: int, T: int, mfma: bool):
    if mfma:
        n16 = N // 16
        return [(16 * (i * n16 // T), 16 * ((i + 1) * n16 // T)) for i in range(T)]
    return [(i * N // T, (i + 1) * N // T) for i in range(T)]


def _dtype_code(d: str) -> int:
    return 0 if d == "f32" else 1


class _Writers:
    """Per-buffer record of write rectangles: arrays (r0, r1, c0, c1, task)."""

    def __init__(self):
        self.parts = {}
        self.cache = {}

    def add(self, buf, r0, r1, c0, c1, task):
        self.parts.setdefault(buf, []).append((r0, r1, c0, c1, task))
        self.cache.pop(buf, None)

    def overlapping(self, buf, r0, r1, c0, c1):
        lst = self.parts.get(buf)
        if not lst:
            return np.empty(0, dtype=np.int64)
        a = self.cache.get(buf)
        if a is None:
            a = self.cache[buf] = np.asarray(lst, dtype=np.int64)
        m = (a[:, 0] < r1) & (r0 < a[:, 1]) & (a[:, 2] < c1) & (c0 < a[:, 3])
        return a[m, 4]


def validate(w) -> None:
    if w.n_q_heads % w.n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if w.head_dim % 2:
        raise ValueError("head_dim must be even")
    for N in (w.qkv_cols, w.hidden, w.intermediate, w.vocab):
        if w.gemv_tiles < 1 or w.gemv_tiles > (N // 16 if w.gemv_config == 2 else N):
            raise ValueError("gemv_tiles out of range")
        if w.gemv_config == 2 and N % 16:
            raise ValueError("MFMA GEMV needs N % 16 == 0")
    if any(L < 1 or L > w.kv_capacity for L in w.kv_len) or len(w.kv_len) != w.batch:
        raise ValueError("kv_len out of range")
    if BufferIndex(w).count > 0xFFFF:
        raise ValueError("more than 65535 buffers")


def build_graph(w):
    """Lower one decode step of workload ``w``; returns (tasks[TASK_DTYPE], edges[uint32])."""
    validate(w)
    bi = BufferIndex(w)
    B, H, hd, Hq, Hkv, I, V = w.batch, w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.intermediate, w.vocab
    grp, T, mfma = Hq // Hkv, w.gemv_tiles, w.gemv_config == 2
    C = [w.chunks(b) for b in range(B)]
    base = {}
    s = 0
    for b in range(B):
        for g in range(Hkv):
            base[(b, g)] = s
            s += C[b]

    rows = []        # descriptor field dicts, final order
    parents = []     # parent index arrays, final order
    writers = _Writers()

    def emit_op(specs):
        """specs: list of (fields, reads, writes) for one op's tasks, in order.
        reads/writes: lists of (buf, r0, r1, c0, c1)."""
        plist = []
        for fields, reads, _ in specs:
            ps = set()
            for rd in reads:
                ps.update(int(x) for x in writers.overlapping(*rd))
            plist.append(ps)
        shared = set.intersection(*plist) if plist else set()
        if w.join_nodes and len(specs) >= 2 and len(shared) >= 2:
            nop = len(rows)
            rows.append(dict(op_id=NOP, in_buf=(NONE, NONE, NONE), out_buf=NONE))
            parents.append(np.array(sorted(shared), dtype=np.int64))
            plist = [(ps - shared) | {nop} for ps in plist]
        for (fields, _, wr), ps in zip(specs, plist):
            idx = len(rows)
            rows.append(fields)
            parents.append(np.array(sorted(ps), dtype=np.int64))
            for rect in wr:
                writers.add(*rect, idx)

    def gemv_op(x, K, W, N, flags, aux, y):
        specs = []
        for (c0, c1) in tile_bounds(N, T, mfma):
            f = dict(op_id=GEMV, config_id=w.gemv_config, flags=flags, m=B, n=N, k=K,
                     in_buf=(x, W, aux), out_buf=y,
                     reserved=(c0, c1 - c0, I if flags & SILU_MUL else 0, 0, 0))
            reads = [(x, 0, B, 0, K)]
            if flags & ADD_RESIDUAL:
                reads.append((aux, 0, B, c0, c1))
            specs.append((f, reads, [(y, 0, B, c0, c1)]))
        emit_op(specs)

    emit_op([(dict(op_id=MEMCPY, config_id=_dtype_code(w.weight_dtype), m=B, n=H, k=0,
                   in_buf=(bi.tokens, bi.embedding, NONE), out_buf=bi.x0), [], [(bi.x0, 0, B, 0, H)])])
    x = bi.x0
    for l in range(w.n_layers):
        qkv, qrot, part, att, hbuf, gu, xo = (bi.act(l, j) for j in range(7))
        kc, vc = bi.layer(l, 6), bi.layer(l, 7)
        gemv_op(x, H, bi.layer(l, 1), w.qkv_cols, RMS_NORM_INPUT, bi.layer(l, 0), qkv)
        kvc = _dtype_code(w.kv_dtype)
        specs = []
        for b in range(B):
            for g in range(Hkv):
                q0, q1 = g * grp * hd, (g + 1) * grp * hd
                k0 = Hq * hd + g * hd
                v0 = (Hq + Hkv) * hd + g * hd
                f = dict(op_id=APPEND, config_id=kvc, m=B, n=hd, k=g, kv_len=w.kv_capacity,
                         in_buf=(qkv, NONE, NONE), out_buf=qrot, reserved=(b, g * grp, grp, kc, vc))
                reads = [(qkv, b, b + 1, q0, q1), (qkv, b, b + 1, k0, k0 + hd), (qkv, b, b + 1, v0, v0 + hd)]
                specs.append((f, reads, [(qrot, b, b + 1, q0, q1)]))
        emit_op(specs)
        specs = []
        for b in range(B):
            for g in range(Hkv):
                q0, q1 = g * grp * hd, (g + 1) * grp * hd
                for c in range(C[b]):
                    sl = base[(b, g)] + c
                    f = dict(op_id=PARTIAL, config_id=kvc, m=C[b], n=hd, k=g, kv_len=w.kv_chunk,
                             in_buf=(qrot, kc, vc), out_buf=part, reserved=(b, g * grp, grp, c, base[(b, g)]))
                    specs.append((f, [(qrot, b, b + 1, q0, q1)], [(part, 0, 1, sl, sl + 1)]))
        emit_op(specs)
        specs = []
        for b in range(B):
            for g in range(Hkv):
                q0, q1 = g * grp * hd, (g + 1) * grp * hd
                bs = base[(b, g)]
                f = dict(op_id=COMBINE, config_id=0, m=C[b], n=hd, k=g, kv_len=w.kv_chunk,
                         in_buf=(part, NONE, NONE), out_buf=att, reserved=(b, g * grp, grp, 0, bs))
                specs.append((f, [(part, 0, 1, bs, bs + C[b])], [(att, b, b + 1, q0, q1)]))
        emit_op(specs)
        gemv_op(att, Hq * hd, bi.layer(l, 2), H, ADD_RESIDUAL, x, hbuf)
        gemv_op(hbuf, H, bi.layer(l, 4), I, RMS_NORM_INPUT | SILU_MUL, bi.layer(l, 3), gu)
        gemv_op(gu, I, bi.layer(l, 5), H, ADD_RESIDUAL, hbuf, xo)
        x = xo
    gemv_op(x, H, bi.w_lm, V, RMS_NORM_INPUT, bi.final_norm, bi.logits)

    n = len(rows)
    tasks = np.zeros(n, dtype=TASK_DTYPE)
    for i, f in enumerate(rows):
        for key, val in f.items():
            tasks[i][key] = val
    indeg = np.array([len(p) for p in parents], dtype=np.int64)
    child = np.repeat(np.arange(n, dtype=np.int64), indeg)
    par = np.concatenate(parents) if n else np.empty(0, dtype=np.int64)
    order = np.lexsort((child, par))
    edges = child[order].astype(np.uint32)
    outdeg = np.bincount(par, minlength=n)
    offs = np.concatenate([[0], np.cumsum(outdeg)[:-1]]) if n else np.empty(0, dtype=np.int64)
    tasks["remaining_deps"] = indeg
    tasks["num_dependents"] = outdeg
    tasks["dependents_offset"] = offs
    return tasks, edges


# --------------------------------------------------------------------------------------
# Invariants and derived quantities
# --------------------------------------------------------------------------------------

def parents_from_csr(tasks, edges):
    """Parent lists recovered from the CSR dependents array."""
    n = len(tasks)
    deg = tasks["num_dependents"].astype(np.int64)
    src = np.repeat(np.arange(n, dtype=np.int64), deg)
    dst = edges.astype(np.int64)
    order = np.lexsort((src, dst))
    src, dst = src[order], dst[order]
    cuts = np.searchsorted(dst, np.arange(n + 1))
    return [src[cuts[i]:cuts[i + 1]] for i in range(n)]


def levels(tasks, edges):
    """Level of each task: 0 without parents, else 1 + max level of its parents (the
    page's level definition); one forward pass over the topological order."""
    par = parents_from_csr(tasks, edges)
    lv = np.zeros(len(tasks), dtype=np.int64)
    for t, ps in enumerate(par):
        if len(ps):
            lv[t] = 1 + lv[ps].max()
    return lv


def waves(n_tasks: int, n_units: int) -> int:
    """Waves needed to run n independent equal tasks on n_units units."""
    return -(-n_tasks // n_units)


def rects_from_descriptor(d, w):
    """(reads, writes) rectangles of one descriptor, derived from its fields alone."""
    bi = BufferIndex(w)
    op = int(d["op_id"])
    hd, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    r = [int(v) for v in d["reserved"]]
    inb = [int(v) for v in d["in_buf"]]
    out = int(d["out_buf"])
    m, n, k = int(d["m"]), int(d["n"]), int(d["k"])
    if op == NOP:
        return [], []
    if op == MEMCPY:
        return [], [(out, 0, m, 0, n)]
    if op == GEMV:
        c0, cnt = r[0], r[1]
        reads = [(inb[0], 0, m, 0, k)]
        if int(d["flags"]) & ADD_RESIDUAL:
            reads.append((inb[2], 0, m, c0, c0 + cnt))
        return reads, [(out, 0, m, c0, c0 + cnt)]
    if op == APPEND:
        b, h0, hc = r[0], r[1], r[2]
        g = k
        q0, q1 = h0 * hd, (h0 + hc) * hd
        k0, v0 = Hq * hd + g * hd, (Hq + Hkv) * hd + g * hd
        reads = [(inb[0], b, b + 1, q0, q1), (inb[0], b, b + 1, k0, k0 + hd), (inb[0], b, b + 1, v0, v0 + hd)]
        return reads, [(out, b, b + 1, q0, q1)]
    if op == PARTIAL:
        b, h0, hc, c, bs = r
        return [(inb[0], b, b + 1, h0 * hd, (h0 + hc) * hd)], [(out, 0, 1, bs + c, bs + c + 1)]
    if op == COMBINE:
        b, h0, hc, _, bs = r
        return [(inb[0], 0, 1, bs, bs + m)], [(out, b, b + 1, h0 * hd, (h0 + hc) * hd)]
    raise ValueError(f"unexpected op {op}")


def check_graph(tasks, edges, w, brute_ancestors: bool = False):
    """Invariants I1-I5 (raises AssertionError); returns the parent lists.

    I1 every edge goes from a lower to a higher index; I2 every earlier writer of an
    overlapping rectangle is an ancestor of the reader; I3 remaining_deps is the
    in-degree and the dependents counts sum to the edge count; I4 no two tasks write
    overlapping rectangles (single assignment); offsets are the exclusive prefix sum.
    """
    n = len(tasks)
    deg = tasks["num_dependents"].astype(np.int64)
    assert int(deg.sum()) == len(edges), "I3: sum(num_dependents) != n_edges"
    offs = np.concatenate([[0], np.cumsum(deg)[:-1]]) if n else deg
    assert np.array_equal(tasks["dependents_offset"].astype(np.int64), offs), "CSR offsets"
    src = np.repeat(np.arange(n, dtype=np.int64), deg)
    assert np.all(src < edges.astype(np.int64)), "I1: edge not forward in emission order"
    par = parents_from_csr(tasks, edges)
    indeg = np.array([len(p) for p in par], dtype=np.int64)
    assert np.array_equal(indeg, tasks["remaining_deps"].astype(np.int64)), "I3: remaining_deps != in-degree"
    for t in range(n):
        ps = par[t]
        assert len(np.unique(ps)) == len(ps), "duplicate edge"
    is_nop = tasks["op_id"] == NOP
    writes = {}
    anc = None
    if brute_ancestors:
        anc = [set() for _ in range(n)]
        for t in range(n):
            for p in par[t]:
                anc[t].add(int(p))
                anc[t] |= anc[int(p)]
    for t in range(n):
        reads, wr = rects_from_descriptor(tasks[t], w)
        near = set(int(p) for p in par[t])
        for p in par[t]:
            if is_nop[p]:
                near.update(int(q) for q in par[int(p)])
        for rd in reads:
            lst = writes.get(rd[0])
            if not lst:
                continue
            a = np.asarray(lst, dtype=np.int64)
            msk = (a[:, 0] < rd[2]) & (rd[1] < a[:, 1]) & (a[:, 2] < rd[4]) & (rd[3] < a[:, 3])
            for wt in a[msk, 4]:
                ok = int(wt) in near or (anc is not None and int(wt) in anc[t])
                assert ok, f"I2: task {t} reads buffer {rd[0]} written by {int(wt)}, not an ancestor"
        for wrr in wr:
            lst = writes.setdefault(wrr[0], [])
            if lst:
                a = np.asarray(lst, dtype=np.int64)
                msk = (a[:, 0] < wrr[2]) & (wrr[1] < a[:, 1]) & (a[:, 2] < wrr[4]) & (wrr[3] < a[:, 3])
                assert not msk.any(), f"I4: task {t} overwrites buffer {wrr[0]}"
            lst.append((wrr[1], wrr[2], wrr[3], wrr[4], t))
    return par


def closed_form_counts(w):
    """(n_tasks, n_edges) of direct lowering (joins off) from the shapes alone."""
    B, G, T = w.batch, w.n_kv_heads, w.gemv_tiles
    grp, hd, Hq = w.n_q_heads // G, w.head_dim, w.n_q_heads
    C = [w.chunks(b) for b in range(B)]
    sumC = sum(C)
    tasks_per_layer = T + B * G + G * sumC + B * G + 3 * T
    n_tasks = 1 + w.n_layers * tasks_per_layer + T
    return n_tasks, tasks_per_layer
