"""Summaries of a trace-mode step (``Graph.mk_set_trace``): where a workgroup's time goes.

A trace holds eight 64-bit words per task, written by the workgroup that ran it:
0 its XCD (high word) and hardware id (low word), 1 start (the task was taken), 2 ready
(the dependency wait ended), 3 end of the body, 4 end of the release (its dependents
counted), 5..7 optional points inside the body (0 = unused).  Times are ticks of the
100 MHz device clock.  NOP joins never run and keep zero words.

``summarize`` groups the tasks by kind (op and, for GEMV tiles, matrix shape and flags)
and reports, in microseconds, the mean wait (start -> ready), busy (ready -> end) and
release (end -> release) per kind, and per workgroup the share of the step spent busy,
waiting, releasing and idle between tasks.  Pure host-side arithmetic on the trace.
"""
from __future__ import annotations

import numpy as np

from .binding import MK_FLAG_ADD_RESIDUAL, MK_FLAG_RMS_NORM_INPUT, MK_FLAG_SILU_MUL, MK_OP_ATTENTION_APPEND, \
    MK_OP_ATTENTION_COMBINE, MK_OP_ATTENTION_PARTIAL, MK_OP_GEMV, MK_OP_MEMCPY, MK_OP_NOP, MK_TASK_DTYPE

TICKS_PER_US = 100.0
_OP_NAMES = {MK_OP_MEMCPY: "memcpy", MK_OP_ATTENTION_APPEND: "append", MK_OP_ATTENTION_PARTIAL: "partial",
             MK_OP_ATTENTION_COMBINE: "combine"}


def task_kind(d) -> str:
    """A readable kind for one descriptor: the op, and for a GEMV tile its matrix
    shape (n x k) and fused flags."""
    op = int(d["op_id"])
    if op != MK_OP_GEMV:
        return _OP_NAMES.get(op, f"op{op}")
    f = int(d["flags"])
    tags = [t for bit, t in ((MK_FLAG_RMS_NORM_INPUT, "norm"), (MK_FLAG_SILU_MUL, "silu"),
                             (MK_FLAG_ADD_RESIDUAL, "resid")) if f & bit]
    return f"gemv {int(d['n'])}x{int(d['k'])}" + (f" [{'+'.join(tags)}]" if tags else "")


def summarize(trace: np.ndarray, tasks: np.ndarray) -> dict:
    """trace: int64 [n_tasks, 8]; tasks: the descriptor array of the same graph (records
    or its raw bytes)."""
    tr = np.asarray(trace, dtype=np.int64).reshape(-1, 8)
    if tasks.dtype.names is None:
        tasks = np.ascontiguousarray(tasks).view(np.uint8).view(MK_TASK_DTYPE).reshape(-1)
    ran = (tasks["op_id"] != MK_OP_NOP) & (tr[:, 1] > 0)
    if not ran.any():
        raise ValueError("the trace holds no task (was trace mode on for the step?)")
    t0 = tr[ran, 1].min()
    start, ready, end, rel = [(tr[:, i] - t0) / TICKS_PER_US for i in (1, 2, 3, 4)]
    span = float(rel[ran].max())
    kinds = np.array([task_kind(tasks[i]) if ran[i] else "" for i in range(len(tasks))])
    per_kind = {}
    for k in dict.fromkeys(kinds[ran]):
        m = kinds == k
        busy = end[m] - ready[m]
        per_kind[k] = {"count": int(m.sum()), "wait_us": float((ready[m] - start[m]).mean()),
                       "busy_us": float(busy.mean()), "busy_min_us": float(busy.min()),
                       "busy_max_us": float(busy.max()), "release_us": float((rel[m] - end[m]).mean())}
    wg = tr[:, 0]
    per_wg = []
    for u in np.unique(wg[ran]):
        m = ran & (wg == u)
        b = float((end[m] - ready[m]).sum())
        wt = float((ready[m] - start[m]).sum())
        r = float((rel[m] - end[m]).sum())
        per_wg.append((b, wt, r, span - b - wt - r))
    a = np.array(per_wg)
    tot = a.sum(axis=0) / (len(per_wg) * span)
    return {"span_us": span, "workgroups": len(per_wg), "tasks": int(ran.sum()),
            "share": {"busy": float(tot[0]), "wait": float(tot[1]), "release": float(tot[2]),
                      "idle": float(tot[3])},
            "kinds": per_kind}


def format_summary(s: dict) -> str:
    lines = [f"step span {s['span_us']:.1f} us over {s['workgroups']} workgroups, {s['tasks']} tasks; "
             f"share of workgroup time: busy {s['share']['busy']:.2f}, wait {s['share']['wait']:.2f}, "
             f"release {s['share']['release']:.2f}, idle {s['share']['idle']:.2f}",
             f"{'kind':34s} {'count':>7s} {'wait':>8s} {'busy':>8s} {'min':>8s} {'max':>8s} {'release':>8s}"]
    for k, v in s["kinds"].items():
        lines.append(f"{k:34s} {v['count']:7d} {v['wait_us']:8.2f} {v['busy_us']:8.2f} {v['busy_min_us']:8.2f} "
                     f"{v['busy_max_us']:8.2f} {v['release_us']:8.2f}")
    return "\n".join(lines)
