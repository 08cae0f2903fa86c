"""Level-synchronous lists (MK_SCHED_LEVELS): the library's grouping against the
oracle's independently lowered graph and its level function, and the property the
level kernel relies on (every producer of a task runs in an earlier level)."""
import numpy as np
import pytest

import task_graph_interpreter_amd as mk
from oracle import graph as og
from synth import workloads

CASES = {
    "tiny": lambda: workloads.tiny(),
    "tiny_nojoins": lambda: workloads.tiny().replace(join_nodes=0),
    "tiny_bf16_b3": lambda: workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                                     kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24,
                                                     name="tiny_bf16_b3"),
    "1b_b1": lambda: workloads.get("1b_b1"),
    "8b_b1": lambda: workloads.get("8b_b1"),
}


def _library_levels(w):
    cfg, keep = mk.make_cfg(**w.mk_fields())
    low = mk.mk_lower(cfg)
    try:
        return low.levels()
    finally:
        low.close()
        del keep


@pytest.mark.parametrize("name", list(CASES))
def test_levels_match_oracle_grouping(name):
    w = CASES[name]()
    tasks, edges = og.build_graph(w)
    lv = np.asarray(og.levels(tasks, edges))
    work = np.nonzero(tasks["op_id"] != 0)[0]  # op_id 0 = NOP join
    expect = [work[lv[work] == l] for l in range(int(lv.max()) + 1)]
    expect = [e for e in expect if e.size]
    got = _library_levels(w)
    assert len(got) == len(expect)
    for g, e in zip(got, expect):
        assert np.array_equal(g, e)


@pytest.mark.parametrize("name", ["tiny", "tiny_nojoins", "tiny_bf16_b3", "1b_b1"])
def test_every_producer_runs_in_an_earlier_level(name):
    w = CASES[name]()
    tasks, edges = og.build_graph(w)
    got = _library_levels(w)
    where = np.full(len(tasks), -1)
    for i, g in enumerate(got):
        assert g.size > 0 and np.all(np.diff(g.astype(np.int64)) > 0)  # non-empty, ascending
        where[g] = i
    nop = tasks["op_id"] == 0
    assert np.all((where >= 0) == ~nop)  # every non-NOP task exactly once, no NOP
    parents = [[] for _ in range(len(tasks))]
    for p in range(len(tasks)):
        o, n = int(tasks["dependents_offset"][p]), int(tasks["num_dependents"][p])
        for c in edges[o:o + n]:
            parents[int(c)].append(p)
    for c in np.nonzero(~nop)[0]:
        for p in parents[c]:
            producers = parents[p] if nop[p] else [p]  # a join stands for its own parents
            for q in producers:
                assert where[q] < where[c], (int(q), int(c))
