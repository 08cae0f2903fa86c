"""The op-list form of the step, the automatic epilogue-fusion pass, standalone RMSNORM
tasks and SAMPLE tasks, in the oracle's lowering (CPU).

"Mega kernel initial" (1y33.com) writes the decoder with the fusions given by hand
as matmul kwargs (graph-API section), names a pass that finds them automatically as
future work, and lists RMSNORM (OpId 3, FUSED_RESIDUAL flag) and SAMPLE (OpId 6) in
its OpId table and flags paragraph."""
import numpy as np
import pytest

from oracle import decode as od
from oracle import graph as og
from oracle import interp as oi
from oracle.params import GeneratedParams
from synth import workloads

SHAPES = {
    "tiny": workloads.tiny(),
    "tiny_bf16_b3": workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                             kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24),
    "1b": workloads.get("1b_b1").replace(n_layers=3),
    "8b_b8": workloads.get("8b_b8_ragged").replace(n_layers=2),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_fusion_pass_gives_the_hand_fused_program(name):
    w = SHAPES[name]
    assert og.fuse_epilogues(og.decoder_program(w)) == og.hand_fused_program(w)


@pytest.mark.parametrize("joins", [1, 0])
@pytest.mark.parametrize("name", ["tiny", "tiny_bf16_b3", "8b_b8"])
def test_pass_graph_equals_hand_fused_graph_byte_for_byte(name, joins):
    w = SHAPES[name].replace(join_nodes=joins)
    t1, e1 = og.build_graph(w)
    t2, e2 = og.build_graph(w, program=og.hand_fused_program(w))
    assert t1.tobytes() == t2.tobytes() and e1.tobytes() == e2.tobytes()


def test_unfused_program_shape():
    w = SHAPES["tiny"]
    ops = og.decoder_program(w)
    norms = [o for o in ops if o.kind == og.NORM]
    assert len(norms) == 2 * w.n_layers + 1
    assert [o.residual != og.NONE for o in norms] == [False] + [True] * (2 * w.n_layers)
    # no matmul carries an epilogue except SiLU*mul, which has no standalone op
    for o in ops:
        if o.kind == og.MATMUL:
            assert o.gamma == og.NONE and o.residual == og.NONE


def test_pass_leaves_a_norm_with_a_non_matmul_reader():
    # A norm whose output is also read by an op that cannot take it as an input
    # epilogue stays a standalone op.
    w = SHAPES["tiny"]
    ops = og.decoder_program(w)
    first_norm = next(i for i, o in enumerate(ops) if o.kind == og.NORM)
    spy = og.Op(og.NORM, 9999, x=ops[first_norm].out, gamma=ops[first_norm].gamma, N=w.hidden)
    fused = og.fuse_epilogues(ops[:first_norm + 1] + [spy] + ops[first_norm + 1:])
    assert ops[first_norm] in fused


@pytest.mark.parametrize("joins", [1, 0])
def test_unfused_graph_invariants_and_counts(joins):
    w = SHAPES["tiny_bf16_b3"].replace(unfused=1, join_nodes=joins)
    tasks, edges = og.build_graph(w)
    og.check_graph(tasks, edges, w, brute_ancestors=True)
    rms = tasks[tasks["op_id"] == og.RMSNORM]
    assert len(rms) == (2 * w.n_layers + 1) * w.batch
    assert ((rms["flags"] == og.FUSED_RESIDUAL).sum()) == 2 * w.n_layers * w.batch
    n_nop = int((tasks["op_id"] == og.NOP).sum())
    assert len(tasks) - n_nop == og.closed_form_counts(w.replace(join_nodes=0))[0]
    assert not (tasks["flags"][tasks["op_id"] == og.GEMV] & (og.RMS_NORM_INPUT | og.ADD_RESIDUAL)).any()


@pytest.mark.parametrize("name", ["tiny", "tiny_bf16_b3"])
def test_unfused_graph_runs_like_the_oracle_in_any_order(name):
    w = SHAPES[name].replace(unfused=1)
    tasks, edges = og.build_graph(w)
    p = GeneratedParams(w)
    runs = []
    for seed in (None, 3, "lifo"):
        it = oi.Interpreter(w, p, w.tokens(), w.positions())
        runs.append(it.run(tasks, edges, order_seed=seed).copy())
    for r in runs[1:]:
        np.testing.assert_array_equal(r, runs[0])
    ref, inter = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), keep=True)
    np.testing.assert_allclose(runs[0], ref, rtol=1e-11, atol=1e-11)
    # the unfused graph's own buffers hold the oracle's intermediate values
    bi = og.BufferIndex(w)
    for l in range(w.n_layers):
        for j, nm in enumerate(["xn", "o", "hn", "d"]):
            np.testing.assert_allclose(it.buf[bi.extra(l, j)], inter[f"l{l}.{nm}"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(it.buf[bi.extra(w.n_layers, 0)], inter["xn_final"], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("unfused", [0, 1])
def test_sample_graph_gives_greedy_tokens_and_next_positions(unfused):
    w = SHAPES["tiny_bf16_b3"].replace(sample=1, unfused=unfused)
    tasks, edges = og.build_graph(w)
    og.check_graph(tasks, edges, w, brute_ancestors=True)
    smp = np.flatnonzero(tasks["op_id"] == og.SAMPLE)
    assert len(smp) == w.batch and smp[-1] == len(tasks) - 1
    assert [int(tasks[t]["reserved"][0]) for t in smp] == list(range(w.batch))
    p = GeneratedParams(w)
    ref, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p))
    for seed in (None, 11, "lifo"):
        it = oi.Interpreter(w, p, w.tokens(), w.positions())
        it.run(tasks, edges, order_seed=seed)
        assert it.tokens.tolist() == [od.greedy_token(r) for r in ref]
        assert it.positions.tolist() == (w.positions() + 1).tolist()


def test_sample_before_the_last_readers_breaks_i7():
    # A sample op placed before the last layer's attention writes positions that later
    # tasks read, and runs before earlier readers are done: the write-after-read check
    # must reject it.
    w = SHAPES["tiny"].replace(sample=1)
    ops = og.step_program(w)
    smp = ops.pop()
    at = max(i for i, o in enumerate(ops) if o.kind == og.ATTN)
    bad = ops[:at] + [smp] + ops[at:]
    tasks, edges = og.build_graph(w, program=bad)
    with pytest.raises(AssertionError, match="I7"):
        og.check_graph(tasks, edges, w, brute_ancestors=True)


def test_sample_counts_closed_form():
    w = SHAPES["tiny_bf16_b3"].replace(sample=1, join_nodes=0)
    tasks, _ = og.build_graph(w)
    assert len(tasks) == og.closed_form_counts(w)[0]
