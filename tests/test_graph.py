"""Lowering: page facts, invariants, closed-form counts, and C++ == Python bytes."""
import json
import os

import numpy as np
import pytest

from oracle import graph as og
from synth import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_descriptor_layout_matches_page():
    g = GOLDEN["task_descriptor"]
    assert og.TASK_DTYPE.itemsize == g["size"]
    for name, off, size in g["fields"]:
        f = og.TASK_DTYPE.fields[name]
        assert f[1] == off and f[0].itemsize == size, name
    assert og.TASK_DTYPE.fields["remaining_deps"][1] % g["remaining_deps_alignment"] == 0


def test_opids_and_flags_match_page():
    for name, val in GOLDEN["op_ids"].items():
        if not name.startswith("_"):
            key = {"ATTENTION_APPEND": "APPEND", "ATTENTION_PARTIAL": "PARTIAL",
                   "ATTENTION_COMBINE": "COMBINE"}.get(name, name)
            assert getattr(og, key) == val
    for name, val in GOLDEN["flags"].items():
        if not name.startswith("_"):
            assert getattr(og, name) == val


def test_gemv_fanout_worked_example():
    ex = GOLDEN["gemv_fanout_example"]
    tiles = og.tile_bounds(ex["columns"], ex["tiles"], False)
    assert len(tiles) == ex["task_count"]
    assert all(c1 - c0 == ex["columns_per_task"] for c0, c1 in tiles)
    # The same fan-out inside a lowered graph: a 1B-class qkv (3072 columns) with 8 tiles.
    w = workloads.llama1b().replace(gemv_tiles=8, n_layers=1, vocab=4096)
    tasks, _ = og.build_graph(w)
    qkv = tasks[(tasks["op_id"] == og.GEMV) & (tasks["n"] == 3072)]
    assert len(qkv) == 8 and (qkv["reserved"][:, 1] == 384).all()
    assert list(qkv["reserved"][:, 0]) == [384 * i for i in range(8)]


def test_wave_quantization_example():
    wq = GOLDEN["wave_quantization"]
    for n, waves in wq["cases"]:
        assert og.waves(n, wq["units"]) == waves


def test_level_definition_on_small_dag():
    # Hand-checked DAG: 0,1 roots; 2<-0; 3<-0,1; 4<-2,3; 5<-1  => levels 0,0,1,1,2,1.
    parents = [[], [], [0], [0, 1], [2, 3], [1]]
    n = len(parents)
    tasks = np.zeros(n, dtype=og.TASK_DTYPE)
    children = [[c for c in range(n) if p in parents[c]] for p in range(n)]
    edges = np.array([c for p in range(n) for c in children[p]], dtype=np.uint32)
    tasks["num_dependents"] = [len(c) for c in children]
    tasks["dependents_offset"] = np.concatenate([[0], np.cumsum([len(c) for c in children])[:-1]])
    tasks["remaining_deps"] = [len(p) for p in parents]
    assert list(og.levels(tasks, edges)) == [0, 0, 1, 1, 2, 1]


@pytest.mark.parametrize("joins", [0, 1])
def test_tiny_invariants_brute_force(joins):
    w = workloads.tiny().replace(join_nodes=joins)
    tasks, edges = og.build_graph(w)
    og.check_graph(tasks, edges, w, brute_ancestors=True)


@pytest.mark.parametrize("name", ["1b_b1", "8b_b8_ragged"])
def test_invariants_large(name):
    w = workloads.get(name)
    tasks, edges = og.build_graph(w)
    og.check_graph(tasks, edges, w)


def _direct_edges_closed_form(w):
    """Direct-lowering edge count from the shapes alone (own derivation)."""
    B, G, T, L = w.batch, w.n_kv_heads, w.gemv_tiles, w.n_layers
    hd, Hq, grp = w.head_dim, w.n_q_heads, w.grp
    C = [w.chunks(b) for b in range(B)]
    qkv_tiles = og.tile_bounds(w.qkv_cols, T, w.gemv_config == 2)

    def covering(lo, hi):
        return {i for i, (c0, c1) in enumerate(qkv_tiles) if c0 < hi and lo < c1}

    app = 0
    for g in range(G):
        s = covering(g * grp * hd, (g + 1) * grp * hd)
        s |= covering(Hq * hd + g * hd, Hq * hd + (g + 1) * hd)
        s |= covering((Hq + G) * hd + g * hd, (Hq + G) * hd + (g + 1) * hd)
        app += len(s)
    per_layer_attn = B * app + G * sum(C) + G * sum(C)
    o = T * (B * G + 1)
    gate_up = T * T
    down = T * (T + 1)
    qkv = T + (L - 1) * T * T
    return qkv + L * (per_layer_attn + o + gate_up + down) + T * T


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_closed_form_counts(name):
    w = workloads.get(name).replace(join_nodes=0)
    n_tasks, _ = og.closed_form_counts(w)
    tasks, edges = og.build_graph(w)
    assert len(tasks) == n_tasks
    assert len(edges) == _direct_edges_closed_form(w)


def test_joins_cut_edges_and_keep_coverage():
    w = workloads.llama8b()
    tj, ej = og.build_graph(w)
    td, ed = og.build_graph(w.replace(join_nodes=0))
    assert len(ej) < len(ed) / 50
    # one NOP per shared-parent op: qkv (layers > 0), o, gate_up, down per layer, lm_head
    assert (tj["op_id"] == og.NOP).sum() == 4 * w.n_layers - 1 + 1


def test_check_graph_catches_planted_mistakes():
    w = workloads.tiny()
    tasks, edges = og.build_graph(w)
    # 1) drop one edge (a qkv tile -> APPEND edge) and keep the counters consistent
    t = int(np.flatnonzero(tasks["op_id"] == og.APPEND)[0])
    par = og.parents_from_csr(tasks, edges)
    victim = int(par[t][0])
    bad_t, bad_e = tasks.copy(), edges.copy()
    off, deg = int(bad_t[victim]["dependents_offset"]), int(bad_t[victim]["num_dependents"])
    kids = list(bad_e[off:off + deg])
    kids.remove(t)
    bad_e = np.concatenate([bad_e[:off], np.array(kids, dtype=np.uint32), bad_e[off + deg:]])
    bad_t["num_dependents"][victim] -= 1
    bad_t["dependents_offset"][victim + 1:] -= 1
    bad_t["remaining_deps"][t] -= 1
    with pytest.raises(AssertionError, match="I2"):
        og.check_graph(bad_t, bad_e, w)
    # 2) an in-degree that does not match the edges
    bad_t = tasks.copy()
    bad_t["remaining_deps"][t] += 1
    with pytest.raises(AssertionError, match="I3"):
        og.check_graph(bad_t, edges, w)
    # 3) a GEMV tile claiming a wrong column range overlaps its neighbour's write
    bad_t = tasks.copy()
    g = int(np.flatnonzero(tasks["op_id"] == og.GEMV)[1])
    bad_t["reserved"][g, 1] += 1
    with pytest.raises(AssertionError):
        og.check_graph(bad_t, edges, w)
