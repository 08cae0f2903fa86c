"""Trace-mode summary arithmetic on a hand-made trace (host only)."""
import numpy as np
import pytest

from oracle import graph as og
from synth import workloads
from task_graph_interpreter_amd import trace as mktrace


def _fake_trace(tasks):
    # Task i (not a NOP) runs on workgroup i % 2: start 1000 i, ready +10, end +30,
    # release +35 ticks (100 ticks = 1 us).
    tr = np.zeros((len(tasks), 8), dtype=np.int64)
    for i in range(len(tasks)):
        if tasks["op_id"][i] == og.NOP:
            continue
        s = 1000 * i + 5000
        tr[i, :5] = (i % 2, s, s + 10, s + 30, s + 35)
    return tr


def test_summary_means_and_shares():
    w = workloads.tiny()
    tasks, _ = og.build_graph(w)
    s = mktrace.summarize(_fake_trace(tasks), tasks)
    ran = int((tasks["op_id"] != og.NOP).sum())
    assert s["tasks"] == ran and s["workgroups"] == 2
    for k, v in s["kinds"].items():
        assert v["wait_us"] == pytest.approx(0.10) and v["busy_us"] == pytest.approx(0.20)
        assert v["release_us"] == pytest.approx(0.05), k
    assert sum(v["count"] for v in s["kinds"].values()) == ran
    # Kinds: one per op, the GEMV tiles split by matrix shape and flags.
    assert s["kinds"]["partial"]["count"] == w.n_layers * w.n_kv_heads * w.chunks(0)
    assert s["kinds"][f"gemv {w.vocab}x{w.hidden} [norm]"]["count"] == w.gemv_tiles
    # Shares of workgroup time add up to 1.
    assert sum(s["share"].values()) == pytest.approx(1.0)
    last = max(i for i in range(len(tasks)) if tasks["op_id"][i] != og.NOP)
    assert s["span_us"] == pytest.approx((1000 * last + 35) / 100)


def test_empty_trace_is_an_error():
    tasks, _ = og.build_graph(workloads.tiny())
    with pytest.raises(ValueError):
        mktrace.summarize(np.zeros((len(tasks), 8), dtype=np.int64), tasks)


def test_raw_descriptor_bytes_and_dtype_mirror():
    from task_graph_interpreter_amd import binding
    assert binding.MK_TASK_DTYPE.itemsize == og.TASK_DTYPE.itemsize == 64
    for name in og.TASK_DTYPE.names:
        assert binding.MK_TASK_DTYPE.fields[name][1] == og.TASK_DTYPE.fields[name][1], name
    tasks, _ = og.build_graph(workloads.tiny())
    tr = _fake_trace(tasks)
    raw = tasks.view(np.uint8).reshape(len(tasks), 64)
    assert mktrace.summarize(tr, raw) == mktrace.summarize(tr, tasks)
