"""CPU descriptor interpreter: random dependency-respecting orders agree bit for bit,
agree with the oracle step, and expose missing edges and corrupted counters."""
import numpy as np
import pytest

from oracle import decode as od
from oracle import graph as og
from oracle import interp as oi
from oracle.params import GeneratedParams
from synth import workloads


def _run(w, tasks, edges, seed):
    p = GeneratedParams(w)
    return oi.Interpreter(w, p, w.tokens(), w.positions()).run(tasks, edges, order_seed=seed).copy()


@pytest.mark.parametrize("joins", [0, 1])
def test_random_orders_bit_identical_and_match_oracle(joins):
    w = workloads.tiny().replace(join_nodes=joins)
    tasks, edges = og.build_graph(w)
    ref = _run(w, tasks, edges, None)
    for seed in (1, 2, 3):
        np.testing.assert_array_equal(_run(w, tasks, edges, seed), ref)
    p = GeneratedParams(w)
    logits, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), split=True)
    np.testing.assert_allclose(ref, logits, rtol=1e-12, atol=1e-12)


def test_batch_ragged_gqa_graph_runs_like_oracle():
    w = workloads.tiny().replace(batch=3, kv_len=(128, 40, 97), n_q_heads=8, kv_dtype="bf16", kv_capacity=128)
    tasks, edges = og.build_graph(w)
    got = _run(w, tasks, edges, 7)
    p = GeneratedParams(w)
    logits, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p))
    np.testing.assert_allclose(got, logits, rtol=1e-11, atol=1e-11)


def test_missing_edge_is_detected():
    w = workloads.tiny()
    tasks, edges = og.build_graph(w)
    ref = _run(w, tasks, edges, None)
    # Drop the edge from the first qkv tile feeding the first APPEND; a consumers-first
    # order runs that tile last among its siblings.
    t = int(np.flatnonzero(tasks["op_id"] == og.APPEND)[0])
    par = og.parents_from_csr(tasks, edges)
    victim = int(par[t][0])
    off, deg = int(tasks[victim]["dependents_offset"]), int(tasks[victim]["num_dependents"])
    kids = [int(k) for k in edges[off:off + deg] if int(k) != t]
    bad_e = np.concatenate([edges[:off], np.array(kids, dtype=np.uint32), edges[off + deg:]])
    bad_t = tasks.copy()
    bad_t["num_dependents"][victim] -= 1
    bad_t["dependents_offset"][victim + 1:] -= 1
    bad_t["remaining_deps"][t] -= 1
    # Consumers-first order runs the APPEND before its unordered producer: NaN reaches the logits.
    assert np.isnan(_run(w, bad_t, bad_e, "lifo")).any()
    # With the edge in place the same order is exact.
    np.testing.assert_array_equal(_run(w, tasks, edges, "lifo"), ref)


def test_corrupted_counter_stalls_instead_of_hanging():
    w = workloads.tiny()
    tasks, edges = og.build_graph(w)
    bad = tasks.copy()
    bad["remaining_deps"][len(bad) // 2] += 1
    with pytest.raises(oi.Stalled):
        _run(w, bad, edges, 5)
