"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every test builds a graph with mk_build_graph, runs mk_decode_step (the persistent
interpreter) and/or mk_decode_step_per_op (one launch per op, same task bodies) and
compares logits within |gpu - ref| <= 2e-2 + 1e-2 |ref| and within the tighter bound of
the arithmetic path (gpu_common.TIERS), greedy tokens exactly (a row is exempt only
when the oracle's own top-2 margin is below what that bound lets two logits move),
and (on the small workloads) every activation buffer of the step.
"""
import numpy as np
import pytest
import torch

import task_graph_interpreter_amd as mk
from oracle import decode as od
from oracle import graph as og
from oracle.params import GeneratedParams
from synth import gen, native, workloads
from synth.device import DeviceInputs

import gpu_common
from gpu_common import TIERS, MkRun, check_close, check_logits, check_tokens, compare_activations, tier_of

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


def _oracle(w, keep=False, rows=None, split=False):
    p = GeneratedParams(w)
    return od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), rows=rows, keep=keep, split=split)


def _check_step(w, logits, ref, what="logits"):
    """Logits at the contract and the path's tier, then exact greedy tokens; returns
    (max |dlogit|, GPU tokens, oracle tokens)."""
    err = check_logits(logits, ref, w, what)
    toks, exempt = check_tokens(logits, ref, TIERS[tier_of(w)], what)
    ref_toks = [od.greedy_token(r) for r in ref]
    _say(f"{what}: max|dlogit|={err:.2e} tokens={toks} oracle={ref_toks} exempt rows={exempt} "
         f"min oracle top-2 margin={min(od.top2_margin(r) for r in ref):.2e}")
    return err, toks, ref_toks


def test_fill_kernel_matches_generator():
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1)
    _say("fill kernel vs numpy generator")
    inp = DeviceInputs(w)
    torch.cuda.synchronize()
    for (tid, name, shape, mean, std, dtype), t in zip(w.weight_specs(), inp.weights):
        got = t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        assert np.array_equal(got, gen.fill(w.seed, tid, got.size, mean, std, dtype)), name
    kc = inp.kcache[1].view(torch.int16).cpu().numpy().view(np.uint16)
    ref = native.cpu_fill_cache(0, w.batch * w.n_kv_heads, 0, w.kv_capacity, w.head_dim, w.seed,
                                w.tid_layer(1, workloads.KCACHE), 0.0, 1.0, "bf16")
    assert np.array_equal(kc.reshape(ref.shape), ref)


@pytest.mark.parametrize("path", ["persistent", "per_op"])
def test_tiny_step_all_activations(path):
    w = workloads.tiny()
    _say(f"tiny one step, {path}")
    run = MkRun(w)
    logits = run.step(path)
    ref, inter = _oracle(w, keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    run.close()


SCHED = {"static": mk.MK_SCHED_STATIC, "dynamic": mk.MK_SCHED_DYNAMIC, "levels": mk.MK_SCHED_LEVELS}


def test_persistent_equals_per_op_bitwise_and_is_repeatable():
    w = workloads.tiny()
    _say("tiny persistent (static and dynamic lists, level-synchronous) vs per-op bitwise, 5 repeats each")
    run = MkRun(w)
    a = run.step("per_op")
    for mode in ["static", "dynamic", "levels", "static", "levels"]:
        run.graph.mk_set_schedule(SCHED[mode])
        for _ in range(5):
            b = run.step("persistent")
            assert np.array_equal(a, b), mode
    run.close()


def test_per_op_graph_replays_equal_eager_per_op():
    w = workloads.tiny()
    _say("tiny per-op launches captured in a HIP graph: 4 replays vs eager per-op, bitwise")
    run = MkRun(w)
    ref = run.step("per_op")
    run.graph.mk_capture_per_op_graph(*run.inp.step_ptrs())
    for i in range(4):
        run.inp.logits.zero_()  # eager work on the same buffers between replays
        run.graph.mk_launch_per_op_graph(run.stream)
        assert run.graph.mk_status() == 0
        torch.cuda.synchronize()
        got = run.inp.logits.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), f"replay {i}"
        assert np.array_equal(run.step("per_op"), ref), f"eager step after replay {i}"
    run.close()


def test_device_schedule_equals_host_schedule():
    w = workloads.tiny()
    _say("tiny schedule uploaded == host schedule")
    run = MkRun(w)
    (order, offsets), est = run.graph.mk_graph_schedule()
    (horder, hoffsets), hest = run.lowered.schedule(run.graph.mk_graph_grid())
    assert np.array_equal(order, horder) and np.array_equal(offsets, hoffsets) and est == hest
    assert run.graph.mk_graph_kernel_name() == "tiny_f32"
    run.close()


@pytest.mark.parametrize("mode", ["static", "dynamic", "levels"])
@pytest.mark.parametrize("joins", [1, 0])
def test_tiny_variants_bf16_batch_ragged(joins, mode):
    # bf16 weights and cache, 3 sequences of different lengths, GQA 8/2, tiles and
    # chunks that do not divide the sizes evenly.
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                 kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24,
                                 join_nodes=joins, name="tiny_bf16_b3")
    _say(f"tiny bf16 batch 3 ragged, joins={joins}, {mode} lists")
    run = MkRun(w)
    run.graph.mk_set_schedule(SCHED[mode])
    logits = run.step("persistent")
    ref, inter = _oracle(w, keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    run.close()


MFMA_CASES = {
    # batch 32 (two 16-row halves of one block), 8 even tiles: groups of 8, 4 and 2 blocks
    "b32": dict(batch=32, kv_len=(128,) * 32, gemv_tiles=8, kv_chunk=32),
    # ragged batch 3 (masked batch rows), GQA 8/2, 5 uneven 16-aligned tiles (groups of
    # 8, 4, 2 and 1 blocks), chunks that do not divide the lengths
    "b3_ragged": dict(batch=3, kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24),
    # batch 40: a full block of 32 rows, then a block of 8
    "b40": dict(batch=40, kv_len=tuple(40 + 2 * i for i in range(40)), gemv_tiles=8, kv_chunk=32),
    # 5 tiles per matmul: 6-7 blocks per qkv tile and 12-13 per lm_head tile, so groups
    # of 8 slots run with 5-7 real blocks (the empty slots read nothing)
    "b32_odd": dict(batch=32, kv_len=(128,) * 32, gemv_tiles=5, kv_chunk=32),
    # wider layers: 4 and 8 chunks of K, so the input staging and the weight ring run
    # in steady state (several chunks per group)
    "b32_wide": dict(batch=32, kv_len=(128,) * 32, hidden=1024, n_q_heads=16, n_kv_heads=4, intermediate=2048,
                     gemv_tiles=24, kv_chunk=64),
    # batch <= 8 runs the small-batch matrix-core tile: a full batch of 8, ragged;
    # wider layers with groups of 8, 4, 2 and 1 blocks and several k-steps per wave
    "b8": dict(batch=8, kv_len=tuple(40 + 11 * i for i in range(8)), gemv_tiles=8, kv_chunk=32),
    "b8_wide": dict(batch=8, kv_len=(128,) * 8, hidden=2048, n_q_heads=16, n_kv_heads=4, intermediate=4096,
                    gemv_tiles=12, kv_chunk=64),
    "b1": dict(batch=1, kv_len=(128,), gemv_tiles=7, kv_chunk=32),
}


@pytest.mark.parametrize("case", list(MFMA_CASES))
def test_tiny_mfma_gemv_all_activations(case):
    # bf16 weights and cache with gemv_config 2: every GEMV runs on the matrix cores
    # (input split into bf16 hi + lo parts, fp32 accumulate).
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=2, kv_capacity=128,
                                 name=f"tiny_mfma_{case}", **MFMA_CASES[case])
    _say(f"tiny MFMA GEMV {case}")
    run = MkRun(w)
    assert run.graph.mk_graph_kernel_name().startswith("mfma8_" if w.batch <= 8 else "mfma_")
    logits = run.step("persistent")
    ref, inter = _oracle(w, keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    again = run.step("per_op")
    assert np.array_equal(logits, again), "per-op and persistent MFMA paths differ"
    run.close()


@pytest.mark.parametrize("rows,cols", [(16, 32), (48, 96), (208, 4096), (4096, 1024)])
def test_pack_matrix_layout(rows, cols):
    # mk_pack_matrix against the layout its declaration defines, written here with
    # numpy: tile (r, j) at (r * cols / 32 + j) KiB, lane l's 8 values
    # src[16 r + l % 16, 32 j + 8 (l / 16) + e] at byte 16 l + 2 e.  Bit-exact.
    _say(f"mk_pack_matrix {rows} x {cols}")
    g = torch.Generator().manual_seed(rows * 7919 + cols)
    src = torch.randint(-32768, 32767, (rows, cols), dtype=torch.int16, generator=g)
    d_src = src.view(torch.bfloat16).cuda()
    d_dst = torch.empty_like(d_src)
    mk.mk_pack_matrix(d_src.data_ptr(), d_dst.data_ptr(), rows, cols, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = d_dst.cpu().view(torch.int16).numpy().reshape(-1)
    s = src.numpy()
    want = np.empty((rows // 16, cols // 32, 64, 8), dtype=np.int16)
    for l in range(64):
        for e in range(8):
            want[:, :, l, e] = s[(l % 16)::16, :][:, (8 * (l // 16) + e)::32]
    assert np.array_equal(got, want.reshape(-1))


@pytest.mark.parametrize("case", ["b8", "b8_wide", "b1", "b3_ragged", "b32", "b40", "b32_wide", "b32_odd"])
def test_tiny_mfma_packed_weights_bitwise_row_major(case):
    # The matrix-core tiles reading the tile layout (MK_LOWER_PACKED_WEIGHTS) do the
    # same products in the same order as with row-major weights: every activation and
    # the logits are bitwise equal; the packed run also against the oracle.
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=2, kv_capacity=128,
                                 name=f"tiny_mfma_{case}", **MFMA_CASES[case])
    _say(f"tiny MFMA GEMV {case}, packed weights vs row-major")
    run = MkRun(w)
    logits = run.step("persistent")
    acts = run.activations()
    runp = MkRun(w.replace(packed=1, name=f"tiny_mfma_{case}_packed"), inputs=run.inp)
    assert runp.graph.mk_graph_kernel_name().startswith("mfma8_" if w.batch <= 8 else "mfma_")
    logits_p = runp.step("persistent")
    acts_p = runp.activations()
    assert np.array_equal(logits_p, logits), "packed and row-major logits differ"
    for k in acts:
        assert np.array_equal(acts_p[k], acts[k]), k
    assert np.array_equal(runp.step("per_op"), logits_p), "per-op and persistent packed paths differ"
    ref, inter = _oracle(w, keep=True)
    compare_activations(w, acts_p, inter, range(w.batch))
    _check_step(w, logits_p, ref)
    runp.close()
    run.close()


def test_8b_shapes_2_layers_b32_mfma_all_activations():
    # 8B-class layer shapes (K = 4096 and 14336: 16 and 56 chunks per group; o and down
    # tiles of one 16-row block, gate_up pairs, lm_head groups of 8) with 2 layers,
    # batch 32 and a short cache, every activation against the oracle.
    w = workloads.get("8b_b32_32k").replace(n_layers=2, kv_len=(256,) * 32, kv_capacity=256, kv_chunk=128,
                                             name="8b_shapes_l2_b32")
    _say("8B shapes, 2 layers, batch 32, MFMA GEMV, all activations")
    run = MkRun(w)
    logits = run.step("persistent")
    p = GeneratedParams(w, backend="c")
    ref, inter = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    run.close()
    del run
    torch.cuda.empty_cache()


UNFUSED_CASES = {
    "tiny_f32": workloads.tiny().replace(unfused=1, name="tiny_unfused"),
    "tiny_bf16_b3": workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                             kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24,
                                             unfused=1, name="tiny_bf16_b3_unfused"),
    "mfma_b32": workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=2, batch=32,
                                         kv_len=(128,) * 32, kv_capacity=128, gemv_tiles=8, unfused=1,
                                         name="tiny_mfma_b32_unfused"),
}


@pytest.mark.parametrize("mode", ["static", "dynamic", "levels", "per_op"])
@pytest.mark.parametrize("case", list(UNFUSED_CASES))
def test_unfused_graph_all_activations(case, mode):
    # The graph lowered without the epilogue-fusion pass: standalone RMSNORM tasks
    # (one per row, FUSED_RESIDUAL carrying the residual adds), GEMVs with no norm or
    # residual flag.  Every activation, including the unfused graph's own buffers
    # (normed inputs, o and down projections before their residual), against the oracle.
    w = UNFUSED_CASES[case]
    _say(f"unfused graph {case}, {mode}")
    run = MkRun(w)
    if mode != "per_op":
        run.graph.mk_set_schedule(SCHED[mode])
    logits = run.step("per_op" if mode == "per_op" else "persistent")
    ref, inter = _oracle(w, keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    run.close()


def test_unfused_8b_shapes_2_layers():
    # RMSNORM tasks at hidden 4096 with the 8B-class batch-1 GEMV specialisation.
    w = workloads.get("8b_b1").replace(n_layers=2, kv_len=(256,), kv_capacity=256, unfused=1,
                                       name="8b_shapes_l2_unfused")
    _say("8B shapes, 2 layers, batch 1, unfused graph, all activations")
    run = MkRun(w)
    assert run.graph.mk_graph_kernel_name() == "h4096_i14336_b1"
    logits = run.step("persistent")
    p = GeneratedParams(w, backend="c")
    ref, inter = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    run.close()
    del run
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["static", "dynamic", "levels", "per_op"])
def test_sample_tasks_one_step(mode):
    # SAMPLE tasks at the end of the graph: one launch gives the logits, each row's
    # greedy token in tokens and the next positions.
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                 kv_len=(128, 41, 97), kv_capacity=160, n_q_heads=8, gemv_tiles=5, kv_chunk=24,
                                 sample=1, name="tiny_bf16_b3_sample")
    _say(f"tiny bf16 batch 3 with SAMPLE tasks, {mode}")
    run = MkRun(w)
    if mode != "per_op":
        run.graph.mk_set_schedule(SCHED[mode])
    logits = run.step("per_op" if mode == "per_op" else "persistent")
    ref, _ = _oracle(w)
    _, toks, ref_toks = _check_step(w, logits, ref)
    assert run.inp.tokens.cpu().tolist() == toks == ref_toks
    assert run.inp.positions.cpu().tolist() == (w.positions() + 1).tolist()
    run.close()


@pytest.mark.parametrize("name,steps", [("tiny", 8), ("1b_b1", 4)])
def test_sample_graph_greedy_loop_one_launch_per_token(name, steps):
    # mk_decode_greedy on a graph with SAMPLE tasks: one launch per token, tokens and
    # positions updated on the device; every token against the oracle's greedy loop.
    w = workloads.get(name).replace(sample=1).with_steps(steps)
    _say(f"{name}: {steps} greedy steps, SAMPLE in the graph (one launch per token)")
    run = MkRun(w)
    p = GeneratedParams(w, backend="c" if name != "tiny" else "auto")
    kv = od.KVState(p)
    tok, pos = w.tokens(), workloads.get(name).positions()
    run.inp.set_step(tok, pos)
    out = torch.full((steps * w.batch,), -1, dtype=torch.int32, device="cuda")
    run.graph.mk_decode_greedy(run.stream, steps, *run.inp.step_ptrs(), out.data_ptr())
    assert run.graph.mk_status() == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(steps, w.batch)
    tol = TIERS[tier_of(w)]
    diverged = False
    for s in range(steps):
        ref, _ = od.decode_step(w, p, tok, pos, kv)
        ref_t = [od.greedy_token(r) for r in ref]
        margin = min(od.top2_margin(r) for r in ref)
        _say(f"{name} step {s}: device tokens {got[s].tolist()} oracle {ref_t} (top-2 margin {margin:.2e})")
        if got[s].tolist() != ref_t:
            # only a near-tie of the oracle may differ; the two sequences part there
            for b in range(w.batch):
                if got[s][b] != ref_t[b]:
                    assert od.top2_margin(ref[b]) < gpu_common.tie_bound(ref[b], tol), (s, b)
                    assert ref[b][ref_t[b]] - ref[b][got[s][b]] <= gpu_common.tie_bound(ref[b], tol), (s, b)
            diverged = True
            break
        tok = np.array(ref_t, dtype=np.int32)
        pos = pos + 1
    if not diverged:
        check_logits(run.inp.logits.cpu().numpy().astype(np.float64), ref, w, "logits of the last step")
        assert run.inp.positions.cpu().tolist() == pos.tolist()
    assert run.inp.tokens.cpu().tolist() == got[-1].tolist()
    run.close()
    del run
    torch.cuda.empty_cache()


def test_8b_shapes_2_layers_b8_mfma_all_activations():
    # The small-batch matrix-core tile at the 8B-class layer shapes (K = 4096 and
    # 14336 split over 8 waves: 16 and 56 k-steps each; o and down tiles of one block,
    # gate_up tiles of 6 and 8 interleaved blocks, lm_head groups of 8, 4, 2 and 1),
    # 2 layers, batch 8 with ragged lengths, every activation against the oracle.
    w = workloads.get("8b_b8_ragged").replace(n_layers=2, name="8b_shapes_l2_b8")
    assert w.packed  # the benchmarked layout: matrices in 16-row tiles
    _say("8B shapes, 2 layers, batch 8 ragged, small-batch MFMA GEMV (packed weights), all activations")
    run = MkRun(w)
    assert run.graph.mk_graph_kernel_name() == "mfma8_bf16_bf16"
    logits = run.step("persistent")
    p = GeneratedParams(w, backend="c")
    ref, inter = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), keep=True)
    compare_activations(w, run.activations(), inter, range(w.batch))
    _check_step(w, logits, ref)
    assert np.array_equal(run.step("per_op"), logits), "per-op and persistent paths differ"
    run.close()
    del run
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["persistent", "per_op"])
def test_tiny_greedy_8_steps(path):
    w = workloads.tiny().with_steps(8)
    _say(f"tiny 8 greedy steps, {path}")
    run = MkRun(w)
    p = GeneratedParams(w)
    kv = od.KVState(p)
    tok = w.tokens()
    pos = workloads.tiny().positions()
    for s in range(8):
        run.inp.set_step(tok, pos)
        logits = run.step(path)
        ref, _ = od.decode_step(w, p, tok, pos, kv)
        _, _, t_ref = _check_step(w, logits, ref, f"logits step {s}")
        tok = np.array(t_ref, dtype=np.int32)
        pos = pos + 1
    run.close()


def test_sample_greedy_lowest_index_on_ties():
    w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                                 kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24, name="tiny_bf16_b3")
    _say("greedy SAMPLE kernel on crafted logits: ties, an all-equal row, a NaN")
    run = MkRun(w)
    rng = np.random.default_rng(7)
    rows = rng.standard_normal((w.batch, w.vocab)).astype(np.float32)
    rows[0, [900, 7, 513]] = 9.0            # tie: the lowest index wins
    rows[1, :] = -2.5                        # every entry equal: index 0
    rows[2, 11] = np.nan                     # NaN never wins
    rows[2, 700] = 8.0
    logits = torch.from_numpy(rows).cuda()
    tokens = torch.full((w.batch,), -1, dtype=torch.int32, device="cuda")
    positions = torch.tensor([5, 40, 96], dtype=torch.int32, device="cuda")
    run.graph.mk_sample_greedy(run.stream, logits.data_ptr(), tokens.data_ptr(), positions.data_ptr())
    torch.cuda.synchronize()
    assert tokens.cpu().tolist() == [7, 0, 700]
    assert tokens.cpu().tolist()[2] == int(np.nanargmax(rows[2]))
    assert positions.cpu().tolist() == [6, 41, 97]
    run.close()


def test_device_greedy_loop_8_steps():
    w = workloads.tiny().with_steps(8)
    _say("tiny 8 greedy steps on the device (decode step + SAMPLE kernel, no host round trip)")
    run = MkRun(w)
    p = GeneratedParams(w)
    kv = od.KVState(p)
    tok = w.tokens()
    pos = workloads.tiny().positions()
    run.inp.set_step(tok, pos)
    out = torch.full((8 * w.batch,), -1, dtype=torch.int32, device="cuda")
    run.graph.mk_decode_greedy(run.stream, 8, *run.inp.step_ptrs(), out.data_ptr())
    assert run.graph.mk_status() == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(8, w.batch)
    for s in range(8):
        ref, _ = od.decode_step(w, p, tok, pos, kv)
        t_ref = od.greedy_token(ref[0])
        assert got[s, 0] == t_ref, (s, int(got[s, 0]), t_ref, od.top2_margin(ref[0]))
        tok = np.array([t_ref], dtype=np.int32)
        pos = pos + 1
    check_logits(run.inp.logits.cpu().numpy().astype(np.float64), ref, w, "logits of the last step")
    assert run.inp.tokens.cpu().tolist() == [int(got[7, 0])]
    assert run.inp.positions.cpu().tolist() == pos.tolist()
    run.close()


def test_bad_position_reports_status_then_recovers():
    w = workloads.tiny()
    _say("tiny bad position status")
    run = MkRun(w)
    good = run.step("persistent")
    run.inp.set_step(w.tokens(), np.array([w.kv_capacity], dtype=np.int32))
    run.graph.mk_decode_step(run.stream, *run.inp.step_ptrs())
    st = run.graph.mk_status()
    assert st & 0xF0000000 == 0x20000000
    run.inp.set_step(w.tokens(), w.positions())
    run.inp.refill_caches()
    again = run.step("persistent")
    assert np.array_equal(good, again)
    run.close()


@pytest.mark.parametrize("mode", ["static", "levels"])
def test_step_after_a_failed_step_runs_nothing(mode):
    # A step enqueued while the status word still holds an earlier failure (no
    # mk_status in between) runs no task: its logits stay as they were.
    w = workloads.tiny()
    _say(f"tiny step after a failed step, {mode} lists")
    run = MkRun(w)
    run.graph.mk_set_schedule(SCHED[mode])
    good = run.step("persistent")
    run.inp.set_step(w.tokens(), np.array([w.kv_capacity], dtype=np.int32))
    run.graph.mk_decode_step(run.stream, *run.inp.step_ptrs())
    run.inp.set_step(w.tokens(), w.positions())
    run.inp.refill_caches()
    run.inp.logits.fill_(7.0)
    run.graph.mk_decode_step(run.stream, *run.inp.step_ptrs())
    torch.cuda.synchronize()
    assert (run.inp.logits == 7.0).all()
    assert run.graph.mk_status() & 0xF0000000 == 0x20000000
    assert np.array_equal(run.step("persistent"), good)
    run.close()


def test_greedy_loop_after_a_failed_step_writes_no_token():
    # mk_decode_greedy from an out-of-range position: the first step fails, its SAMPLE
    # and every later step and SAMPLE leave tokens, positions and tokens_out alone.
    w = workloads.tiny().with_steps(4)
    _say("tiny greedy loop from a bad position")
    run = MkRun(w)
    bad = np.array([w.kv_capacity], dtype=np.int32)
    run.inp.set_step(w.tokens(), bad)
    out = torch.full((3 * w.batch,), -1, dtype=torch.int32, device="cuda")
    run.graph.mk_decode_greedy(run.stream, 3, *run.inp.step_ptrs(), out.data_ptr())
    st = run.graph.mk_status()
    assert st & 0xF0000000 == 0x20000000
    assert out.cpu().tolist() == [-1, -1, -1]
    assert run.inp.positions.cpu().tolist() == bad.tolist()
    assert run.inp.tokens.cpu().tolist() == w.tokens().tolist()
    run.close()


@pytest.mark.parametrize("bad", [-1, 1024])
def test_bad_token_reports_status_then_recovers(bad):
    # An out-of-range token id is clamped to row 0 for the gather (no out-of-bounds
    # read) and reported through the status word; the next good step is bitwise equal.
    w = workloads.tiny()
    _say(f"tiny bad token {bad}")
    run = MkRun(w)
    good = run.step("persistent")
    run.inp.set_step(np.array([bad], dtype=np.int32), w.positions())
    run.graph.mk_decode_step(run.stream, *run.inp.step_ptrs())
    st = run.graph.mk_status()
    assert st & 0xF0000000 == 0x30000000 and st & 0x0FFFFFFF == 0  # the MEMCPY is task 0
    run.inp.set_step(w.tokens(), w.positions())
    run.inp.refill_caches()
    assert np.array_equal(run.step("persistent"), good)
    run.close()


@pytest.mark.parametrize("mode", ["static", "dynamic", "levels"])
def test_wait_timeout_drains_and_recovers(mode):
    # A 1-tick bound on every dependency wait: tasks whose producers are not done at
    # the first look give up, the step drains, mk_status reports a timeout, and the
    # next step with the normal bound is correct again.
    w = workloads.tiny()
    _say(f"tiny forced wait timeout, {mode} lists")
    run = MkRun(w)
    run.graph.mk_set_schedule(SCHED[mode])
    good = run.step("persistent")
    run.graph.mk_set_wait_limit(1)
    run.graph.mk_decode_step(run.stream, *run.inp.step_ptrs())
    st = run.graph.mk_status()
    assert st == 0 or st & 0xF0000000 == 0x10000000
    run.graph.mk_set_wait_limit(200_000_000)
    run.inp.refill_caches()
    assert np.array_equal(run.step("persistent"), good)
    run.close()


@pytest.mark.parametrize("mode", ["static", "dynamic"])
def test_trace_mode_records_every_task(mode):
    w = workloads.tiny()
    _say(f"tiny trace mode, {mode} lists")
    run = MkRun(w)
    run.graph.mk_set_schedule(SCHED[mode])
    n = run.plan["n_tasks"]
    trace = torch.zeros(n * 8, dtype=torch.int64, device="cuda")
    run.graph.mk_set_trace(trace.data_ptr())
    run.step("persistent")
    run.graph.mk_set_trace(None)
    tr = trace.cpu().numpy().reshape(n, 8)
    tasks, edges = og.build_graph(w)
    nop = tasks["op_id"] == 0
    assert nop.any(), "the tiny graph has NOP joins"
    assert (tr[nop] == 0).all(), "NOP joins never run as tasks"
    run_ = ~nop
    assert (tr[run_, 1] > 0).all()
    t1, t2, t3, t4 = (tr[run_, i] for i in (1, 2, 3, 4))
    assert (t1 <= t2).all() and (t2 <= t3).all() and (t3 <= t4).all()
    if mode == "static":  # each workgroup runs its list in order, on one CU
        (order, offsets), _ = run.graph.mk_graph_schedule()
        for i in range(len(offsets) - 1):
            lst = order[offsets[i]:offsets[i + 1]]
            assert len(set(tr[lst, 0].tolist())) <= 1
            assert (np.diff(tr[lst, 1]) >= 0).all()
    par = og.parents_from_csr(tasks, edges)

    def ends(p):  # when a parent's data was complete: a NOP's parents' ends
        return [tr[p, 3]] if not nop[p] else [e for q in par[p] for e in ends(q)]

    for t in np.flatnonzero(run_):  # a task becomes ready only after every parent ended
        for p in par[t]:
            for e in ends(p):
                assert e <= tr[t, 2] + 1, (p, t)
    run.close()


def _big_parity(name, rows=None, steps=1):
    """``steps`` greedy steps of a full-size workload on the persistent kernel against
    the oracle (all batch rows, or the sampled ``rows``: rows are independent, so the
    oracle computes exactly those).  Both sides take the oracle's tokens as the next
    step's input, after the GPU's tokens were asserted equal to them."""
    w = workloads.get(name)
    if steps > 1:
        w = w.with_steps(steps)
    _say(f"{name} parity, rows={rows}, steps={steps}")
    run = MkRun(w)
    p = GeneratedParams(w, backend="c")
    kv = od.KVState(p)
    tok = w.tokens()
    pos = workloads.get(name).positions()
    rows = list(range(w.batch)) if rows is None else rows
    for s in range(steps):
        run.inp.set_step(tok, pos)
        logits = run.step("persistent")
        ref, _ = od.decode_step(w, p, tok, pos, kv, rows=rows)
        _, _, t_ref = _check_step(w, logits[rows], ref, f"{name} step {s}")
        if steps > 1:
            assert rows == list(range(w.batch))
            tok = np.array(t_ref, dtype=np.int32)
        pos = pos + 1
    run.close()
    del run
    torch.cuda.empty_cache()


def test_1b_greedy_4_steps():
    _big_parity("1b_b1", steps=4)


def test_1b_schedulers_and_graph_replay_equal_persistent_bitwise():
    w = workloads.get("1b_b1")
    _say("1b_b1: level-synchronous, per-op and HIP-graph replay vs persistent, bitwise")
    run = MkRun(w)
    ref = run.step("persistent")
    run.graph.mk_set_schedule(mk.MK_SCHED_LEVELS)
    assert np.array_equal(run.step("persistent"), ref), "levels"
    run.graph.mk_set_schedule(mk.MK_SCHED_STATIC)
    assert np.array_equal(run.step("per_op"), ref), "per-op"
    run.graph.mk_capture_per_op_graph(*run.inp.step_ptrs())
    run.inp.logits.zero_()
    run.graph.mk_launch_per_op_graph(run.stream)
    assert run.graph.mk_status() == 0
    torch.cuda.synchronize()
    assert np.array_equal(run.inp.logits.cpu().numpy().astype(np.float64), ref), "graph replay"
    assert np.array_equal(run.step("persistent"), ref), "persistent again"
    run.close()
    del run
    torch.cuda.empty_cache()


def test_1b_device_greedy_loop_equals_host_loop():
    # The host loop (decode step, argmax of the copied logits, next position) is the
    # path the 4-step oracle test above checks; the device loop must give its tokens.
    n = 4
    w = workloads.get("1b_b1").with_steps(n)
    _say("1b_b1: 4 greedy steps, device loop (mk_decode_greedy) vs host loop")
    run = MkRun(w)
    tok0, pos0 = w.tokens(), workloads.get("1b_b1").positions()
    tok, pos, host = tok0, pos0, []
    for _ in range(n):
        run.inp.set_step(tok, pos)
        logits = run.step("persistent")
        tok = np.array([od.greedy_token(logits[0])], dtype=np.int32)
        host.append(int(tok[0]))
        pos = pos + 1
    last = logits
    run.inp.refill_caches()
    run.inp.set_step(tok0, pos0)
    out = torch.full((n * w.batch,), -1, dtype=torch.int32, device="cuda")
    run.graph.mk_decode_greedy(run.stream, n, *run.inp.step_ptrs(), out.data_ptr())
    assert run.graph.mk_status() == 0
    torch.cuda.synchronize()
    assert out.cpu().tolist() == host
    assert np.array_equal(run.inp.logits.cpu().numpy().astype(np.float64), last)
    assert run.inp.positions.cpu().tolist() == pos.tolist()
    run.close()
    del run
    torch.cuda.empty_cache()


def test_8b_b1_step():
    _big_parity("8b_b1")


def test_8b_b8_ragged_step():
    _big_parity("8b_b8_ragged")


def test_8b_b32_32k_step_sampled_rows():
    _big_parity("8b_b32_32k", rows=[0, 1, 17, 31])
