"""mk_decode_step_noalloc -- the decode step with its activations in the library's
static device array, for callers that cannot allocate -- against mk_decode_step on
the same graphs, through the C ABI: two calls in a row, the second on a smaller
graph, then the size limit and a graph built without a scratch block."""
import numpy as np
import pytest
import torch

import task_graph_interpreter_amd as mk
from task_graph_interpreter_amd import binding
from oracle import decode as od
from oracle.params import GeneratedParams
from synth import workloads

from gpu_common import TIERS, MkRun, check_logits, check_tokens, tier_of

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.init()


BIG = workloads.tiny().replace(weight_dtype="bf16", kv_dtype="bf16", gemv_config=1, batch=3,
                               kv_len=(128, 41, 97), n_q_heads=8, gemv_tiles=5, kv_chunk=24, name="tiny_bf16_b3")
SMALL = workloads.tiny()


def _logits(run):
    torch.cuda.synchronize()
    return run.inp.logits.cpu().numpy().astype(np.float64)


def test_noalloc_equals_step_two_calls_second_smaller():
    _say("mk_decode_step_noalloc: tiny bf16 batch 3, then tiny fp32 batch 1, against mk_decode_step")
    runs = [MkRun(BIG), MkRun(SMALL)]
    assert runs[0].plan["scratch_bytes"] > runs[1].plan["scratch_bytes"]
    refs = [r.step("persistent") for r in runs]
    for r in runs:
        r.inp.logits.fill_(float("nan"))
    for r in runs:  # back to back on one stream: the second call reuses the array
        r.graph.mk_decode_step_noalloc(r.stream, *r.inp.step_ptrs())
    for r, ref in zip(runs, refs):
        assert r.graph.mk_status() == 0
        got = _logits(r)
        assert np.array_equal(got, ref), "noalloc step differs from mk_decode_step"
        p = GeneratedParams(r.w)
        oracle, _ = od.decode_step(r.w, p, r.w.tokens(), r.w.positions(), od.KVState(p))
        err = check_logits(got, oracle, r.w, f"{r.w.name} noalloc logits")
        toks, _ = check_tokens(got, oracle, TIERS[tier_of(r.w)], f"{r.w.name} noalloc tokens")
        _say(f"{r.w.name}: noalloc == mk_decode_step bitwise; max|dlogit| vs oracle {err:.2e}; tokens {toks}")
    # and again, the smaller graph first this time
    for r in reversed(runs):
        r.inp.logits.fill_(float("nan"))
        r.graph.mk_decode_step_noalloc(r.stream, *r.inp.step_ptrs())
    for r, ref in zip(runs, refs):
        assert r.graph.mk_status() == 0
        assert np.array_equal(_logits(r), ref)
    for r in runs:
        r.close()


def test_graph_without_scratch_block_runs_only_noalloc():
    w = SMALL
    _say("graph built with scratch_dev = NULL")
    ref_run = MkRun(w)
    ref = ref_run.step("persistent")
    cfg, keep = mk.make_cfg(**w.mk_fields())
    g = mk.mk_build_graph(cfg, ref_run.inp.weight_ptrs(), 0, ref_run.stream)
    with pytest.raises(mk.MkError) as e:
        g.mk_decode_step(ref_run.stream, *ref_run.inp.step_ptrs())
    assert e.value.code == binding.MK_ERR_INVALID and "scratch" in str(e.value)
    ref_run.inp.logits.fill_(float("nan"))
    g.mk_decode_step_noalloc(ref_run.stream, *ref_run.inp.step_ptrs())
    assert g.mk_status() == 0
    assert np.array_equal(_logits(ref_run), ref)
    g.close()
    ref_run.close()
    del keep


def test_noalloc_rejects_a_graph_beyond_the_limit():
    w = workloads.tiny().replace(batch=4000, kv_len=(8,) * 4000, kv_capacity=8, name="tiny_b4000")
    cfg, keep = mk.make_cfg(**w.mk_fields())
    need = mk.mk_plan(cfg)["scratch_bytes"]
    assert need > binding.MK_STATIC_SCRATCH_BYTES
    _say(f"tiny batch 4000: {need / 2**20:.1f} MiB of activations, beyond the 64 MiB array")
    run = MkRun(w)
    with pytest.raises(mk.MkError) as e:
        run.graph.mk_decode_step_noalloc(run.stream, *run.inp.step_ptrs())
    assert e.value.code == binding.MK_ERR_INVALID and "64 MiB" in str(e.value)
    run.close()
    del keep
