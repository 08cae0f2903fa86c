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
  R10 the step is first written as a list of ops, the way the page's graph API builds
     it (embed, rmsnorm, matmul, attention, and sample for a greedy step).  Written
     without fusion, every RMSNorm is its own op and each residual add rides on the
     next RMSNorm (the FUSED_RESIDUAL flag of the descriptor section: the norm also
     writes the sum).  The epilogue-fusion pass the page names as future work (graph
     API section) then folds each residual add into the matmul that produced the
     summand (ADD_RESIDUAL) and each RMSNorm read only by matmuls into those matmuls
     (RMS_NORM_INPUT); the result is the hand-fused decoder of the graph-API section.
  R11 RMSNORM (OpId 3) is one task per batch row (the norm needs the whole row); SAMPLE
     (OpId 6) is one task per batch row after the lm_head, writing the row's greedy
     token and advancing its position.
Parity: pinned by the page's worked tiling example (3072 columns in 8 tiles of 384),
the descriptor layout and OpId/flag values printed on the page, and by the invariants
in ``check_graph`` (topological order, read-after-write coverage, in-degrees, SSA).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

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
FUSED_RESIDUAL = 2  # the same bit on an RMSNORM descriptor
NONE = 0xFFFF


class BufferIndex:
    """Canonical buffer-table indices (append-only order).  A graph lowered without
    epilogue fusion has five more activation buffers per layer group, appended after
    the logits: per layer the normed attention input, the o-projection output, the
    normed MLP input and the down-projection output, then the normed final input."""

    def __init__(self, w):
        L = w.n_layers
        self.L = L
        self.tokens, self.positions, self.embedding = 0, 1, 2
        self.final_norm = 3 + 8 * L
        self.w_lm = 4 + 8 * L
        self.scratch0 = 5 + 8 * L
        self.x0 = self.scratch0
        self.logits = self.scratch0 + 1 + 7 * L
        self.unfused = bool(getattr(w, "unfused", 0))
        self.count = self.logits + 1 + ((4 * L + 1) if self.unfused else 0)

    @staticmethod
    def layer(l, which):
        return 3 + 8 * l + which

    def act(self, l, which):
        """which: 0 qkv_out, 1 q_rot, 2 partials, 3 att, 4 h, 5 gu, 6 x_out."""
        return self.scratch0 + 1 + 7 * l + which

    def extra(self, l, which):
        """Unfused graphs only.  which: 0 xn (normed attention input), 1 o (o-projection
        output), 2 hn (normed MLP input), 3 d (down-projection output); l = n_layers,
        which 0: the normed final input."""
        return self.logits + 1 + 4 * l + which


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


EMBED, NORM, MATMUL, ATTN, SAMPLE_OP = "embed", "rmsnorm", "matmul", "attention", "sample"


@dataclass(frozen=True)
class Op:
    """One op of the step as the graph API builds it, before the fan-out into tasks.
    matmul: out = x W^T, with gamma (RMS_NORM_INPUT: x is normed first), residual
    (ADD_RESIDUAL) and silu (SILU_MUL) as its epilogue flags.  rmsnorm: out =
    rmsnorm(x [+ residual]) * gamma, writing the sum x + residual to out2 when there
    is a residual (FUSED_RESIDUAL).  attention: layer ``layer`` from its qkv input x.
    embed: x0 from the tokens.  sample: greedy token of each row of x."""
    kind: str
    out: int
    x: int = NONE
    w: int = NONE
    gamma: int = NONE
    residual: int = NONE
    out2: int = NONE
    silu: bool = False
    K: int = 0
    N: int = 0
    layer: int = -1


def decoder_program(w):
    """The decode step written with the graph API and no fusion: every RMSNorm its
    own op, each residual add carried by the next RMSNorm (FUSED_RESIDUAL)."""
    bi = BufferIndex(w.replace(unfused=1))
    H, I, V, L = w.hidden, w.intermediate, w.vocab, w.n_layers
    ops = [Op(EMBED, bi.x0, x=bi.tokens, w=bi.embedding)]
    x_in = bi.x0
    for l in range(L):
        qkv, _, _, att, h, gu, xo = (bi.act(l, j) for j in range(7))
        xn, o, hn, d = (bi.extra(l, j) for j in range(4))
        if l == 0:
            ops.append(Op(NORM, xn, x=bi.x0, gamma=bi.layer(0, 0), N=H))
        else:  # the previous layer's residual add rides on this norm
            ops.append(Op(NORM, xn, x=bi.extra(l - 1, 3), gamma=bi.layer(l, 0), residual=bi.act(l - 1, 4),
                          out2=x_in, N=H))
        ops.append(Op(MATMUL, qkv, x=xn, w=bi.layer(l, 1), K=H, N=w.qkv_cols))
        ops.append(Op(ATTN, att, x=qkv, layer=l))
        ops.append(Op(MATMUL, o, x=att, w=bi.layer(l, 2), K=w.q_cols, N=H))
        ops.append(Op(NORM, hn, x=o, gamma=bi.layer(l, 3), residual=x_in, out2=h, N=H))
        ops.append(Op(MATMUL, gu, x=hn, w=bi.layer(l, 4), silu=True, K=H, N=I))
        ops.append(Op(MATMUL, d, x=gu, w=bi.layer(l, 5), K=I, N=H))
        x_in = xo
    xf = bi.extra(L, 0)
    ops.append(Op(NORM, xf, x=bi.extra(L - 1, 3), gamma=bi.final_norm, residual=bi.act(L - 1, 4), out2=x_in, N=H))
    ops.append(Op(MATMUL, bi.logits, x=xf, w=bi.w_lm, K=H, N=V))
    return ops


def hand_fused_program(w):
    """The decoder as the graph-API section writes it, fusions given by hand: norm and
    residual as kwargs of the matmuls, the final norm inside the lm_head matmul."""
    bi = BufferIndex(w)
    H, I, V = w.hidden, w.intermediate, w.vocab
    ops = [Op(EMBED, bi.x0, x=bi.tokens, w=bi.embedding)]
    x = bi.x0
    for l in range(w.n_layers):
        qkv, _, _, att, h, gu, xo = (bi.act(l, j) for j in range(7))
        ops.append(Op(MATMUL, qkv, x=x, w=bi.layer(l, 1), gamma=bi.layer(l, 0), K=H, N=w.qkv_cols))
        ops.append(Op(ATTN, att, x=qkv, layer=l))
        ops.append(Op(MATMUL, h, x=att, w=bi.layer(l, 2), residual=x, K=w.q_cols, N=H))
        ops.append(Op(MATMUL, gu, x=h, w=bi.layer(l, 4), gamma=bi.layer(l, 3), silu=True, K=H, N=I))
        ops.append(Op(MATMUL, xo, x=gu, w=bi.layer(l, 5), residual=h, K=I, N=H))
        x = xo
    ops.append(Op(MATMUL, bi.logits, x=x, w=bi.w_lm, gamma=bi.final_norm, K=H, N=V))
    return ops


def fuse_epilogues(ops):
    """The automatic epilogue-fusion pass over an op list.
      1. rmsnorm(m, gamma, residual r) -> (y, sum s), where m is written by a matmul
         with no epilogue and read by nothing else: the matmul adds r itself
         (ADD_RESIDUAL) and writes s; the norm then reads s with no residual.
      2. rmsnorm(x, gamma) -> y with no residual, where every reader of y is a matmul
         with neither an input norm nor a residual (one gamma/residual slot per
         descriptor): each reader reads x with RMS_NORM_INPUT gamma, and the norm op
         is dropped.
    Anything else stays as it is."""
    ops = list(ops)

    def readers(buf):
        return [i for i, o in enumerate(ops) if o is not None and buf in (o.x, o.residual)]

    def writer(buf):
        return [i for i, o in enumerate(ops) if o is not None and buf in (o.out, o.out2)]

    for i, o in enumerate(ops):
        if o.kind != NORM or o.residual == NONE:
            continue
        wr = writer(o.x)
        if len(wr) != 1 or readers(o.x) != [i]:
            continue
        m = ops[wr[0]]
        if m.kind != MATMUL or m.gamma != NONE or m.residual != NONE or m.silu:
            continue
        ops[wr[0]] = dataclasses.replace(m, residual=o.residual, out=o.out2)
        ops[i] = dataclasses.replace(o, x=o.out2, residual=NONE, out2=NONE)
    for i, o in enumerate(ops):
        if o is None or o.kind != NORM or o.residual != NONE:
            continue
        rs = readers(o.out)
        if not rs or any(ops[r].kind != MATMUL or ops[r].x != o.out or ops[r].gamma != NONE
                         or ops[r].residual != NONE for r in rs):
            continue
        for r in rs:
            ops[r] = dataclasses.replace(ops[r], x=o.x, gamma=o.gamma)
        ops[i] = None
    return [o for o in ops if o is not None]


def step_program(w):
    """The op list build_graph lowers: the decoder program, through the fusion pass
    unless the workload asks for the unfused graph, plus the sample op for a greedy
    step."""
    ops = decoder_program(w)
    if not getattr(w, "unfused", 0):
        ops = fuse_epilogues(ops)
    if getattr(w, "sample", 0):
        bi = BufferIndex(w)
        ops.append(Op(SAMPLE_OP, bi.tokens, x=bi.logits, out2=bi.positions, N=w.vocab))
    return ops


def build_graph(w, program=None):
    """Lower one decode step of workload ``w`` (the op list of step_program, or
    ``program``); returns (tasks[TASK_DTYPE], edges[uint32])."""
    validate(w)
    ops = step_program(w) if program is None else program
    bi = BufferIndex(w)
    B, H, hd, Hq, Hkv, I = w.batch, w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.intermediate
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

    def gemv_op(o):
        flags = (RMS_NORM_INPUT if o.gamma != NONE else 0) | (ADD_RESIDUAL if o.residual != NONE else 0) | \
                (SILU_MUL if o.silu else 0)
        aux = o.gamma if o.gamma != NONE else o.residual
        specs = []
        for (c0, c1) in tile_bounds(o.N, T, mfma):
            f = dict(op_id=GEMV, config_id=w.gemv_config, flags=flags, m=B, n=o.N, k=o.K,
                     in_buf=(o.x, o.w, aux), out_buf=o.out,
                     reserved=(c0, c1 - c0, I if o.silu else 0, 0, 0))
            reads = [(o.x, 0, B, 0, o.K)]
            if o.residual != NONE:
                reads.append((o.residual, 0, B, c0, c1))
            specs.append((f, reads, [(o.out, 0, B, c0, c1)]))
        emit_op(specs)

    def norm_op(o):
        specs = []
        for b in range(B):
            f = dict(op_id=RMSNORM, config_id=_dtype_code(w.weight_dtype),
                     flags=FUSED_RESIDUAL if o.residual != NONE else 0, m=B, n=o.N, k=0,
                     in_buf=(o.x, o.gamma, o.residual), out_buf=o.out, reserved=(b, o.out2, 0, 0, 0))
            reads = [(o.x, b, b + 1, 0, o.N)]
            writes = [(o.out, b, b + 1, 0, o.N)]
            if o.residual != NONE:
                reads.append((o.residual, b, b + 1, 0, o.N))
                writes.append((o.out2, b, b + 1, 0, o.N))
            specs.append((f, reads, writes))
        emit_op(specs)

    def attention_ops(o):
        l, qkv, att = o.layer, o.x, o.out
        qrot, part = bi.act(l, 1), bi.act(l, 2)
        kc, vc = bi.layer(l, 6), bi.layer(l, 7)
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

    def sample_op(o):
        specs = []
        for b in range(B):
            f = dict(op_id=SAMPLE, config_id=0, m=B, n=o.N, k=0, in_buf=(o.x, NONE, NONE), out_buf=o.out,
                     reserved=(b, o.out2, 0, 0, 0))
            specs.append((f, [(o.x, b, b + 1, 0, o.N)], [(o.out, b, b + 1, 0, 1), (o.out2, b, b + 1, 0, 1)]))
        emit_op(specs)

    for o in ops:
        if o.kind == EMBED:
            emit_op([(dict(op_id=MEMCPY, config_id=_dtype_code(w.weight_dtype), m=B, n=H, k=0,
                           in_buf=(o.x, o.w, NONE), out_buf=o.out), [], [(o.out, 0, B, 0, H)])])
        elif o.kind == MATMUL:
            gemv_op(o)
        elif o.kind == NORM:
            norm_op(o)
        elif o.kind == ATTN:
            attention_ops(o)
        elif o.kind == SAMPLE_OP:
            sample_op(o)
        else:
            raise ValueError(f"unknown op kind {o.kind}")

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
    if op == RMSNORM:
        b = r[0]
        reads, writes = [(inb[0], b, b + 1, 0, n)], [(out, b, b + 1, 0, n)]
        if int(d["flags"]) & FUSED_RESIDUAL:
            reads.append((inb[2], b, b + 1, 0, n))
            writes.append((r[1], b, b + 1, 0, n))
        return reads, writes
    if op == SAMPLE:
        b = r[0]
        return [(inb[0], b, b + 1, 0, n)], [(out, b, b + 1, 0, 1), (r[1], b, b + 1, 0, 1)]
    raise ValueError(f"unexpected op {op}")


def external_reads(d, w):
    """Rows of the per-step inputs tokens and positions a descriptor reads, as (buf,
    row) pairs: the embedding gather reads every row's token, RoPE-append and the
    attention partials read their row's position."""
    op = int(d["op_id"])
    bi = BufferIndex(w)
    if op == MEMCPY:
        return [(bi.tokens, b) for b in range(int(d["m"]))]
    if op in (APPEND, PARTIAL):
        return [(bi.positions, int(d["reserved"][0]))]
    return []


def check_graph(tasks, edges, w, brute_ancestors: bool = False):
    """Invariants I1-I5 and I7 (raises AssertionError); returns the parent lists.

    I1 every edge goes from a lower to a higher index; I2 every earlier writer of an
    overlapping rectangle is an ancestor of the reader; I3 remaining_deps is the
    in-degree and the dependents counts sum to the edge count; I4 no two tasks write
    overlapping rectangles (single assignment); offsets are the exclusive prefix sum;
    I7 a task that writes a row of tokens or positions (SAMPLE) has every task that
    reads that row as an ancestor (write after read; needs brute_ancestors).
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
    bi = BufferIndex(w)
    ext_readers, ext_writers = {}, {}
    for t in range(n):
        for key in external_reads(tasks[t], w):
            for wt in ext_writers.get(key, []):
                assert anc is not None, "I7 needs brute_ancestors"
                assert wt in anc[t], f"I7: task {t} reads {key} after task {wt} wrote it, without an edge"
            ext_readers.setdefault(key, []).append(t)
        _, wr = rects_from_descriptor(tasks[t], w)
        for (buf, r0, r1, _, _) in wr:
            if buf not in (bi.tokens, bi.positions):
                continue
            assert anc is not None, "I7 needs brute_ancestors"
            for row in range(r0, r1):
                for rd in ext_readers.get((buf, row), []):
                    assert rd in anc[t], f"I7: task {t} writes row {row} of buffer {buf} before reader {rd} is done"
                ext_writers.setdefault((buf, row), []).append(t)
    return par


def closed_form_counts(w):
    """(n_tasks, n_edges) of direct lowering (joins off) from the shapes alone."""
    B, G, T = w.batch, w.n_kv_heads, w.gemv_tiles
    grp, hd, Hq = w.n_q_heads // G, w.head_dim, w.n_q_heads
    C = [w.chunks(b) for b in range(B)]
    sumC = sum(C)
    tasks_per_layer = T + B * G + G * sumC + B * G + 3 * T
    if getattr(w, "unfused", 0):
        tasks_per_layer += 2 * B       # the attention and MLP norms, one task per row
    n_tasks = 1 + w.n_layers * tasks_per_layer + T
    if getattr(w, "unfused", 0):
        n_tasks += B                   # the final norm
    if getattr(w, "sample", 0):
        n_tasks += B                   # one SAMPLE per row
    return n_tasks, tasks_per_layer
