"""Static per-workgroup schedule (host side, no GPU): it partitions the non-NOP tasks,
keeps each list in increasing task order, gives wide matmuls one tile per workgroup,
and every list drains under adversarial timing when NOP joins are fired inline by
their last parent -- the property the persistent kernel's progress rests on."""
import os

import numpy as np
import pytest

import task_graph_interpreter_amd as mk
from task_graph_interpreter_amd import binding
from oracle import graph as og
from synth import workloads

OP_NOP, OP_GEMV = 0, 2


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(binding.LIB_PATH):
        from task_graph_interpreter_amd import build
        build.build()


def _lowered(w):
    f = w.mk_fields()
    cfg, keep = mk.make_cfg(**f)
    return mk.mk_lower(cfg), keep


def _graph(w):
    tasks, edges = og.build_graph(w)
    return tasks, edges


def _drains(tasks, edges, order, offsets, rng):
    """Runs the lists with random interleaving: at every step a random workgroup whose
    head task is ready runs it.  NOP joins complete when their last parent does.
    Returns the number of tasks run; all of them iff no workgroup is stuck."""
    n = len(tasks)
    indeg = tasks["remaining_deps"].astype(np.int64)
    arrived = np.zeros(n, np.int64)
    done = np.zeros(n, bool)
    nop = tasks["op_id"] == OP_NOP
    heads = [int(offsets[w]) for w in range(len(offsets) - 1)]
    ends = [int(offsets[w + 1]) for w in range(len(offsets) - 1)]

    def complete(t):
        done[t] = True
        off, nd = int(tasks["dependents_offset"][t]), int(tasks["num_dependents"][t])
        for c in edges[off:off + nd]:
            arrived[c] += 1
            if nop[c] and arrived[c] == indeg[c]:
                complete(int(c))

    ran = 0
    live = [w for w in range(len(heads)) if heads[w] < ends[w]]
    while live:
        ready = [w for w in live if arrived[order[heads[w]]] == indeg[order[heads[w]]]]
        if not ready:
            break
        w = ready[rng.integers(len(ready))]
        complete(int(order[heads[w]]))
        heads[w] += 1
        ran += 1
        if heads[w] == ends[w]:
            live.remove(w)
    return ran, done


@pytest.mark.parametrize("name", ["tiny", "1b_b1", "8b_b1", "8b_b8_ragged"])
@pytest.mark.parametrize("workers", [256, 37, 1])
def test_schedule_partitions_non_nop_tasks(name, workers):
    w = workloads.get(name)
    lo, keep = _lowered(w)
    (order, offsets), est = lo.schedule(workers)
    tasks, _ = _graph(w)
    assert offsets.shape == (workers + 1,) and offsets[0] == 0 and offsets[-1] == len(order)
    assert np.all(np.diff(offsets.astype(np.int64)) >= 0)
    non_nop = np.flatnonzero(tasks["op_id"] != OP_NOP)
    assert np.array_equal(np.sort(order), non_nop)
    for i in range(workers):
        lst = order[offsets[i]:offsets[i + 1]]
        assert np.all(np.diff(lst.astype(np.int64)) > 0), "each list must be in increasing task order"
    assert est > 0


@pytest.mark.parametrize("name", ["1b_b1", "8b_b1"])
def test_wide_matmuls_get_one_tile_per_workgroup(name):
    """With one tile per CU, no workgroup runs two tiles of one GEMV op (the
    wave-quantisation tail the static lists remove)."""
    w = workloads.get(name)
    lo, keep = _lowered(w)
    workers = 256
    (order, offsets), _ = lo.schedule(workers)
    tasks, _ = _graph(w)
    owner = np.empty(len(tasks), np.int64)
    owner[:] = -1
    for i in range(workers):
        owner[order[offsets[i]:offsets[i + 1]]] = i
    gemv = np.flatnonzero(tasks["op_id"] == OP_GEMV)
    # group GEMV tasks into ops: runs of consecutive indices with the same out_buf
    groups = {}
    for t in gemv:
        groups.setdefault(int(tasks["out_buf"][t]), []).append(t)
    for buf, ts in groups.items():
        assert len(ts) <= workers
        own = owner[ts]
        assert len(np.unique(own)) == len(ts), f"buffer {buf}: a workgroup got two tiles"


@pytest.mark.parametrize("name,joins", [("tiny", 1), ("tiny", 0), ("8b_b8_ragged", 1), ("1b_b1", 1)])
@pytest.mark.parametrize("workers", [256, 5])
def test_lists_drain_under_random_timing(name, joins, workers):
    w = workloads.get(name).replace(join_nodes=joins)
    if name != "tiny":
        w = w.replace(n_layers=2)
    lo, keep = _lowered(w)
    (order, offsets), _ = lo.schedule(workers)
    tasks, edges = _graph(w)
    rng = np.random.default_rng(7)
    for _ in range(3):
        ran, done = _drains(tasks, edges, order, offsets, rng)
        assert ran == len(order)
        assert done.all(), "every NOP join fired and every task ran"


def test_a_list_out_of_order_can_stall():
    """The check above has teeth: reversing one workgroup's list that holds a parent
    and its child makes that workgroup wait on itself."""
    w = workloads.tiny()
    lo, keep = _lowered(w)
    tasks, edges = _graph(w)
    # a single worker whose list is reversed cannot start (its head is the last task)
    order = np.flatnonzero(tasks["op_id"] != OP_NOP)[::-1].astype(np.uint32)
    offsets = np.array([0, len(order)], np.uint32)
    ran, _ = _drains(tasks, edges, order, offsets, np.random.default_rng(0))
    assert ran < len(order)


def test_schedule_rejects_zero_workers():
    lo, keep = _lowered(workloads.tiny())
    with pytest.raises(mk.MkError):
        lo.schedule(0)
