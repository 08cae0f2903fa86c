"""The C-ABI library: loads without a GPU, exports every declared symbol, validates
configurations, and its host lowering equals the oracle lowering byte for byte."""
import ctypes
import os
import re

import numpy as np
import pytest

import task_graph_interpreter_amd as mk
from task_graph_interpreter_amd import binding
from oracle import graph as og
from synth import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mk.h")


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(binding.LIB_PATH):
        from task_graph_interpreter_amd import build
        build.build()


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|void|const char\*|uint32_t)\s+(mk_\w+)\s*\(", text, re.M))
    assert declared == set(binding.EXPORTS)
    L = mk.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert mk.mk_abi_version() == binding.MK_ABI_VERSION


def test_struct_layouts():
    assert ctypes.sizeof(binding.MkTask) == 64
    for name, off, size in [("op_id", 0, 2), ("remaining_deps", 8, 4), ("in_buf", 20, 6), ("out_buf", 26, 2),
                            ("kv_len", 40, 4), ("reserved", 44, 20)]:
        f = getattr(binding.MkTask, name)
        assert f.offset == off and f.size == size
    assert ctypes.sizeof(binding.MkModelCfg) == 88


def _cfg(w, **over):
    f = w.mk_fields()
    f.update(over)
    return mk.make_cfg(**f)


def test_abi_mismatch_fails_loudly():
    cfg, keep = _cfg(workloads.tiny())
    cfg.struct_size = 80
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan(cfg)
    assert e.value.code == binding.MK_ERR_ABI


@pytest.mark.parametrize("over,msg", [
    (dict(n_kv_heads=3), "n_q_heads"),
    (dict(gemv_tiles=10_000), "gemv_tiles"),
    (dict(kv_len=(129,)), "kv_len"),
    (dict(gemv_config=1), "gemv_config"),
    (dict(head_dim=63), "head_dim"),
    (dict(kv_chunk=0), "kv_chunk"),
    (dict(vocab=20_000_000), "4 GiB"),
    (dict(kv_capacity=1 << 24), "KV head"),
    (dict(batch=65536, kv_len=(128,) * 65536, weight_dtype="bf16", kv_dtype="bf16", gemv_config=2,
          hidden=16384, n_q_heads=64, n_kv_heads=16), "batch x K x 4"),
])
def test_invalid_configs_rejected(over, msg):
    cfg, keep = _cfg(workloads.tiny(), **over)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan(cfg)
    assert e.value.code == binding.MK_ERR_INVALID and msg in str(e.value)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
@pytest.mark.parametrize("joins", [1, 0])
def test_cpp_lowering_equals_oracle_lowering(name, joins):
    w = workloads.get(name).replace(join_nodes=joins)
    cfg, keep = _cfg(w)
    lo = mk.mk_lower(cfg)
    tasks, edges = og.build_graph(w)
    assert np.array_equal(lo.tasks_bytes(), tasks.view(np.uint8).reshape(-1, 64))
    assert np.array_equal(lo.edges(), edges)
    plan = mk.mk_plan(cfg)
    assert plan["n_tasks"] == len(tasks) and plan["n_edges"] == len(edges)
    assert plan["n_levels"] == int(og.levels(tasks, edges).max()) + 1


@pytest.mark.parametrize("opts", [dict(unfused=1), dict(sample=1), dict(unfused=1, sample=1)])
@pytest.mark.parametrize("name", ["tiny", "1b_b1", "8b_b8_ragged"])
@pytest.mark.parametrize("joins", [1, 0])
def test_cpp_lowering_options_equal_oracle_lowering(name, joins, opts):
    # The unfused graph (standalone RMSNORM tasks) and the SAMPLE tasks, lowered by
    # both builders.
    w = workloads.get(name).replace(join_nodes=joins, **opts)
    cfg, keep = _cfg(w)
    lo = mk.mk_lower(cfg)
    tasks, edges = og.build_graph(w)
    assert np.array_equal(lo.tasks_bytes(), tasks.view(np.uint8).reshape(-1, 64))
    assert np.array_equal(lo.edges(), edges)
    plan = mk.mk_plan(cfg)
    assert plan["n_buffers"] == og.BufferIndex(w).count


def test_unfused_scratch_holds_the_extra_buffers():
    w = workloads.tiny().replace(batch=3, kv_len=(128, 41, 97), unfused=1)
    cfg, keep = _cfg(w)
    lo = mk.mk_lower(cfg)
    bi = og.BufferIndex(w)
    fused = mk.mk_plan(_cfg(w.replace(unfused=0))[0])["scratch_bytes"]
    extras = [bi.extra(l, j) for l in range(w.n_layers) for j in range(4)] + [bi.extra(w.n_layers, 0)]
    spans = [lo.scratch_span(b) for b in extras]
    assert all(nb == 4 * w.batch * w.hidden for _, nb in spans)
    assert min(o for o, _ in spans) >= fused  # appended after the fused graph's buffers
    assert mk.mk_plan(cfg)["scratch_bytes"] >= spans[-1][0] + spans[-1][1]


def test_unknown_option_rejected():
    cfg, keep = _cfg(workloads.tiny(), options=8)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan(cfg)
    assert e.value.code == binding.MK_ERR_INVALID and "options" in str(e.value)


@pytest.mark.parametrize("name", ["8b_b8_ragged", "tiny_b8"])
def test_packed_weight_option_lowers_the_same_graph(name):
    # MK_LOWER_PACKED_WEIGHTS changes the layout the GEMV reads its matrices in, not
    # the graph: descriptors and edges are byte-equal to the row-major graph's.
    if name == "tiny_b8":
        w = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=2, batch=8,
                                     kv_len=(128,) * 8, packed=1)
    else:
        w = workloads.get(name)
    assert w.packed
    a = mk.mk_lower(_cfg(w)[0])
    b = mk.mk_lower(_cfg(w.replace(packed=0))[0])
    assert np.array_equal(a.tasks_bytes(), b.tasks_bytes())
    assert np.array_equal(a.edges(), b.edges())


@pytest.mark.parametrize("over", [dict(), dict(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1)])
def test_packed_weight_option_needs_the_mfma_gemv(over):
    cfg, keep = _cfg(workloads.tiny().replace(packed=1), **over)
    with pytest.raises(mk.MkError) as e:
        mk.mk_plan(cfg)
    assert e.value.code == binding.MK_ERR_INVALID and "MK_LOWER_PACKED_WEIGHTS" in str(e.value)


def test_pack_matrix_rejects_bad_arguments_without_a_gpu():
    # Every argument check runs before the kernel is enqueued.
    L = binding.lib()
    p = lambda a: ctypes.c_void_p(a)
    big = 1 << 40
    cases = [
        (L.mk_pack_matrix(None, p(big), 16, 32, None), binding.MK_ERR_INVALID, "NULL"),
        (L.mk_pack_matrix(p(big), p(2 * big), 15, 32, None), binding.MK_ERR_INVALID, "multiple of 16"),
        (L.mk_pack_matrix(p(big), p(2 * big), 16, 48, None), binding.MK_ERR_INVALID, "multiple of 16"),
        (L.mk_pack_matrix(p(big), p(2 * big), 0, 32, None), binding.MK_ERR_INVALID, "multiple of 16"),
        (L.mk_pack_matrix(p(big + 8), p(2 * big), 16, 32, None), binding.MK_ERR_ALIGN, "aligned"),
        (L.mk_pack_matrix(p(big), p(big + 1008), 16, 32, None), binding.MK_ERR_INVALID, "overlap"),
    ]
    for rc, code, msg in cases:
        assert rc == code
    assert "overlap" in mk.mk_last_error()


def test_scratch_layout():
    w = workloads.llama8b_ragged()
    cfg, keep = _cfg(w)
    lo = mk.mk_lower(cfg)
    bi = og.BufferIndex(w)
    spans = []
    slots = sum(w.chunks(b) for b in range(w.batch)) * w.n_kv_heads
    expect = {0: w.batch * w.qkv_cols, 1: w.batch * w.q_cols, 2: slots * w.grp * (w.head_dim + 2),
              3: w.batch * w.q_cols, 4: w.batch * w.hidden, 5: w.batch * w.intermediate, 6: w.batch * w.hidden}
    spans.append(lo.scratch_span(bi.x0))
    for l in range(w.n_layers):
        for j in range(7):
            off, nb = lo.scratch_span(bi.act(l, j))
            assert nb == 4 * expect[j]
            spans.append((off, nb))
    offs = [o for o, _ in spans]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert all(a[0] + a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert spans[-1][0] + spans[-1][1] <= mk.mk_plan(cfg)["scratch_bytes"]
    with pytest.raises(mk.MkError):
        lo.scratch_span(bi.w_lm)


def test_step_entry_points_reject_bad_arguments_without_a_gpu():
    # Argument checks run before any HIP call, so they answer on a machine with no GPU.
    L = binding.lib()
    tok = ctypes.c_void_p(16)
    err = [
        L.mk_sample_greedy(None, None, tok, tok, tok),
        L.mk_decode_greedy(None, None, 1, tok, tok, tok, tok, tok, None),
        L.mk_capture_per_op_graph(None, tok, tok, tok, tok, tok),
        L.mk_launch_per_op_graph(None, None),
        L.mk_decode_step(None, None, tok, tok, tok, tok, tok),
        L.mk_set_schedule(None, binding.MK_SCHED_LEVELS),
    ]
    assert err == [binding.MK_ERR_INVALID] * len(err)
    assert "NULL" in mk.mk_last_error()
