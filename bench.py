"""Decode-step benchmark of the persistent megakernel on one GPU.

One step = one mk_decode_step: the whole decode step of the workload (embedding
gather, every layer's GEMV tiles, RoPE-append, split-KV attention partials and
combines, and the lm_head with the fused final norm) in ONE persistent-kernel launch.
Inputs (seeded synthetic weights and KV caches) are resident in HBM before timing.

Prints ONE JSON line: decode tokens/s over the timed steps, step latency, the HBM
roofline fraction of the step (algorithmic bytes = every weight byte read once + the
KV bytes attended, divided by the step time and by 8 TB/s), the same step run as one
launch per op (same task bodies), and the CPU oracle timed on a bounded sample.

Usage: python bench.py [--steps K] [--warmup W] [--workload 8b_b1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/sec and step latency at 1 GPU; % of HBM roofline per step"
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def blas_threads() -> tuple[int, int]:
    """(threads for the oracle's BLAS, cores this process may run on): every core of
    the affinity mask, capped by OMP_NUM_THREADS when the environment sets it (the
    host's share of CPUs for one GPU)."""
    affinity = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    cap = int(env) if env.isdigit() and int(env) > 0 else affinity
    return min(affinity, cap), affinity


def cpu_baseline(w, layer_counts=(1, 2, 3), min_seconds=12.0):
    """The oracle (float64 numpy) timed on this host on a bounded sample: the full step
    of the same shapes with 1, 2 and 3 layers.  Weights and the cache slices the step
    reads are generated beforehand, so only the oracle's arithmetic is timed.  The
    three variants run round robin until about min_seconds of oracle work is timed
    (slow drifts of the host then hit all three alike); a least-squares line through
    the three medians is extrapolated to the workload's layer count, and the spread of
    the per-layer slope between pairs of samples is reported with it."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import decode as od
    from oracle.params import GeneratedParams

    class Pregenerated:
        def __init__(self, p, tids):
            self.p = p
            self.m = {t: p.matrix(t) for t in tids}
            self.c = {}

        def embedding_row(self, tok):
            return self.p.embedding_row(tok)

        def vector(self, tid):
            return self.p.vector(tid)

        def matrix(self, tid):
            return self.m[tid]

        def cache(self, *a):
            if a not in self.c:
                self.c[a] = self.p.cache(*a)
            return self.c[a]

    threads, affinity = blas_threads()
    runs = {n: [] for n in layer_counts}
    with threadpool_limits(limits=threads):
        used = max([1] + [i.get("num_threads", 1) for i in threadpool_info()])
        variants = {}
        for nl in layer_counts:
            ws = w.replace(n_layers=nl)
            p = GeneratedParams(ws, backend="c")
            mats = [s[0] for s in ws.weight_specs() if len(s[2]) == 2 and s[1] != "embedding"]
            pre = Pregenerated(p, mats)
            od.decode_step(ws, pre, ws.tokens(), ws.positions(), od.KVState(pre))  # fills the cache slices
            variants[nl] = (ws, pre)
        while sum(sum(r) for r in runs.values()) < min_seconds or min(len(r) for r in runs.values()) < 3:
            for nl in layer_counts:
                ws, pre = variants[nl]
                kv = od.KVState(pre)
                t0 = time.perf_counter()
                od.decode_step(ws, pre, ws.tokens(), ws.positions(), kv)
                runs[nl].append(time.perf_counter() - t0)
        del variants
    times = {n: float(np.median(r)) for n, r in runs.items()}
    xs = np.array(layer_counts, dtype=np.float64)
    ys = np.array([times[n] for n in layer_counts])
    per_layer, fixed = np.polyfit(xs, ys, 1)
    slopes = [(times[b] - times[a]) / (b - a) for i, a in enumerate(layer_counts) for b in layer_counts[i + 1:]]
    est = float(fixed + w.n_layers * per_layer)
    samples = ", ".join(f"{n} layer{'s' if n > 1 else ''} median {times[n]:.3f} s of {len(runs[n])} runs"
                        for n in layer_counts)
    return {"value": w.batch / est, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": (f"float64 numpy oracle, full step of the same shapes with {samples}, run round robin; "
                       f"least-squares line extrapolated to {w.n_layers} layers = {est:.2f} s/step (per-layer "
                       f"slope {per_layer:.4f} s, pairwise slopes {min(slopes):.4f}-{max(slopes):.4f} s)"),
            "affinity_cores": affinity, "seconds_per_step_estimate": est}


KERNEL_SRC = os.path.join(ROOT, "task_graph_interpreter_amd", "csrc")


# The sources the persistent kernel is compiled from (kern_spec.hip and what it
# includes, the specialisation list, and the ABI header that fixes the descriptor
# layout); host-only files (lowering, scheduling, runtime) do not change it.
KERNEL_FILES = ["kern_spec.hip", "kernels.h", "tasks.h", "task_gemv.h", "task_gemv_mfma.h", "task_gemv_mfma_small.h",
                "task_attn.h",
                "device_common.h", "specs.def", os.path.join("..", "..", "include", "mk.h")]


def kernel_source_hash() -> str:
    """Hash of the persistent kernel's sources: a traffic figure taken from hardware
    counters is only reported while the kernel is the one it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_FILES:
        h.update(os.path.basename(name).encode())
        with open(os.path.join(KERNEL_SRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_interpreter_{workload}.json")


def measured_traffic(workload: str):
    """HBM bytes per persistent-kernel launch from the committed counter summary, or
    None if there is none or the kernels changed since it was taken."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def summarize_pmc(fetch_dir: str, write_dir: str, copy_bytes: int, workload: str, command: str) -> dict:
    """Per-launch HBM traffic of the persistent kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same
    counter reads for a plain copy of copy_bytes (read once, written once)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row["Kernel_Name"]
                    key = "interpreter" if "interpreter_kernel" in name else "copy" if "copy16_kernel" in name else None
                    if key:
                        vals.setdefault(key, []).append(float(row["Counter_Value"]))
        return vals

    fv, wv = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    f_int, w_int = float(np.median(fv["interpreter"])), float(np.median(wv["interpreter"]))
    f_cp, w_cp = float(np.median(fv["copy"])), float(np.median(wv["copy"]))
    kf, kw = copy_bytes / (f_cp * 1024.0), copy_bytes / (w_cp * 1024.0)
    return {"workload": workload, "kernel": "interpreter_kernel", "kernel_source_hash": kernel_source_hash(),
            "fetch_kib_per_launch": f_int, "write_kib_per_launch": w_int,
            "copy_bytes": copy_bytes, "copy_fetch_kib": f_cp, "copy_write_kib": w_cp,
            "fetch_scale": kf, "write_scale": kw,
            "traffic_bytes_per_launch": f_int * 1024.0 * kf + w_int * 1024.0 * kw,
            "launches": [len(fv["interpreter"]), len(wv["interpreter"])], "command": command}


def greedy_run(w, inp, n_tokens, stream):
    """Greedy decode of n_tokens tokens from the timed step's position onward, with a
    graph lowered for n_tokens more cache slots on the same weights, with SAMPLE tasks
    at its end.  The loop never touches the host: mk_decode_greedy enqueues one launch
    per token, whose SAMPLE tasks pick the tokens (argmax, lowest index on ties) and
    advance the positions.  Returns time between tokens."""
    import torch

    import task_graph_interpreter_amd as mk
    from synth.device import DeviceInputs

    w2 = w.replace(kv_len=tuple(int(l) + n_tokens for l in w.kv_len), kv_capacity=w.kv_capacity + n_tokens,
                   sample=1)
    inp2 = DeviceInputs(w2, weights=inp.weights)
    cfg2, keep2 = mk.make_cfg(**w2.mk_fields())
    plan2 = mk.mk_plan(cfg2)
    scratch2 = torch.zeros(plan2["scratch_bytes"], dtype=torch.uint8, device="cuda")
    g2 = mk.mk_build_graph(cfg2, inp2.weight_ptrs(), scratch2.data_ptr(), stream)
    inp2.set_step(w.tokens(), w.positions())
    ptrs2 = inp2.step_ptrs()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = torch.empty(n_tokens * w.batch, dtype=torch.int32, device="cuda")
    ev0.record()
    g2.mk_decode_greedy(stream, n_tokens, *ptrs2, out.data_ptr())
    ev1.record()
    torch.cuda.synchronize()
    assert g2.mk_status() == 0
    assert int(inp2.positions[0]) == int(w.positions()[0]) + n_tokens
    total = ev0.elapsed_time(ev1)
    g2.close()
    del keep2
    log(f"greedy: {n_tokens} tokens, {total / n_tokens:.4f} ms between tokens")
    return {"tokens": n_tokens, "ms_per_token": total / n_tokens, "tokens_per_s": w.batch * n_tokens / (total / 1e3),
            "first_position": int(w.positions()[0]), "kv_slots": w2.kv_capacity,
            "note": "graph lowered for kv_len + tokens (empty chunks until reached) with SAMPLE tasks after the "
                    "lm_head; mk_decode_greedy: one launch per token, no host round trip"}


def timed(fn, steps, warmup, stream, ptrs):
    """Run fn(stream, *ptrs) warmup times, then time steps calls with HIP events on the
    stream the kernels run on.  Returns (total ms, per-call ms array)."""
    import torch

    for _ in range(warmup):
        fn(stream, *ptrs)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(stream, *ptrs)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return ev[0].elapsed_time(ev[steps]), per


def model_key(w):
    """Workloads with equal keys have bitwise-equal weights (same shapes and seed)."""
    return (w.n_layers, w.hidden, w.n_q_heads, w.n_kv_heads, w.head_dim, w.intermediate, w.vocab, w.weight_dtype,
            w.seed, w.packed)


def time_other_workload(name, steps, warmup, stream, shared):
    """Another workload timed in the same run: the persistent step and the per-op
    launches of the same graph, after checking that both give the same logits within
    the parity tolerance.  ``shared`` = (model_key, weight tensors) of a workload
    already on the device, reused when the model is the same."""
    import torch

    import task_graph_interpreter_amd as mk
    from synth import workloads
    from synth.device import DeviceInputs

    w = workloads.get(name)
    reuse = shared is not None and shared[0] == model_key(w)
    log(f"{name}: filling inputs" + (" (weights shared)" if reuse else ""))
    inp = DeviceInputs(w, weights=shared[1] if reuse else None)
    if w.packed and not reuse:
        inp.weights = inp.packed_weights()  # one-time load-time layout change, not timed
    cfg, keep = mk.make_cfg(**w.mk_fields())
    plan = mk.mk_plan(cfg)
    scratch = torch.zeros(plan["scratch_bytes"], dtype=torch.uint8, device="cuda")
    g = mk.mk_build_graph(cfg, inp.weight_ptrs(), scratch.data_ptr(), stream)
    ptrs = inp.step_ptrs()
    g.mk_decode_step(stream, *ptrs)
    assert g.mk_status() == 0
    mega = inp.logits.clone()
    g.mk_decode_step_per_op(stream, *ptrs)
    torch.cuda.synchronize()
    diff = (inp.logits - mega).abs().max().item()
    assert diff <= 2e-2, f"{name}: per-op and persistent logits differ by {diff}"
    total, per = timed(g.mk_decode_step, steps, warmup, stream, ptrs)
    assert g.mk_status() == 0
    t2, _ = timed(g.mk_decode_step_per_op, steps, warmup, stream, ptrs)
    ms, ms2 = total / steps, t2 / steps
    achieved = w.bytes_per_step() / (ms / 1e3) / 1e9
    out = {"workload": name, "batch": w.batch, "kv_len": list(w.kv_len), "kv_chunk": w.kv_chunk,
           "gemv_config": w.gemv_config, "kernel": g.mk_graph_kernel_name(),
           "weight_layout": "tile16" if w.packed else "row-major", "ms_per_step": ms,
           "latency_ms_median": float(np.median(per)), "tokens_per_s": w.batch * steps / (total / 1e3),
           "bytes_per_step": w.bytes_per_step(), "achieved_gbs": achieved, "frac": achieved / PEAK_HBM_GBS,
           "traffic": measured_traffic(name), "per_op_ms_per_step": ms2, "speedup_over_per_op": ms2 / ms}
    log(f"{name}: persistent {ms:.4f} ms/step ({achieved:.0f} GB/s, {achieved / PEAK_HBM_GBS:.3f} of peak), "
        f"per-op {ms2:.4f} ms/step")
    g.close()
    del inp, scratch, keep
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="8b_b1")
    ap.add_argument("--others", default="1b_b1,8b_b8_ragged,8b_b32_32k",
                    help="comma-separated workloads also timed in this run ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-op", action="store_true")
    ap.add_argument("--no-alt-schedule", action="store_true", help="skip timing the other schedule mode")
    ap.add_argument("--trace-out", default=None, help="write a per-task trace of one step (.npy)")
    ap.add_argument("--kv-chunk", type=int, default=0, help="override the workload's split-KV chunk (keys)")
    ap.add_argument("--gemv-tiles", type=int, default=0, help="override the workload's GEMV tiles per matmul")
    ap.add_argument("--gemv-config", type=int, default=-1, help="override the GEMV variant (1 vector, 2 MFMA)")
    ap.add_argument("--packed", type=int, default=-1, help="override the weight layout (0 row-major, 1 tile16)")
    ap.add_argument("--greedy-tokens", type=int, default=-1,
                    help="greedy decode of N tokens after the timed step (time between tokens); "
                         "default 256 at batch 1, else 0")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of MIB MiB (byte-counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs into the traffic summary and exit")
    ap.add_argument("--pmc-command", default="", help="the profiled command, recorded in the summary")
    ap.add_argument("--schedule", choices=["static", "dynamic", "levels"], default="static",
                    help="how persistent workgroups find tasks: host-built lists or a ticket counter")
    args = ap.parse_args()

    if args.summarize_pmc:
        t = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.copy_calibration << 20,
                          args.workload, args.pmc_command)
        with open(traffic_path(args.workload), "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py runs on one GPU only: the decode megakernel has no multi-GPU path "
                  f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", flush=True)
        sys.exit(2)

    import torch

    import task_graph_interpreter_amd as mk
    from oracle import graph as og
    from synth import workloads
    from synth.device import DeviceInputs

    w = workloads.get(args.workload)
    if args.kv_chunk:
        w = w.replace(kv_chunk=args.kv_chunk)
    if args.gemv_tiles:
        w = w.replace(gemv_tiles=args.gemv_tiles)
    if args.gemv_config >= 0:
        w = w.replace(gemv_config=args.gemv_config)
    if args.packed >= 0:
        w = w.replace(packed=args.packed)
    torch.cuda.set_device(0)
    log(f"workload {w.name}: filling {w.weight_bytes_per_step() / 1e9:.2f} GB weights + caches")
    inp = DeviceInputs(w)
    if w.packed:
        # Matrices into the tile layout of mk_pack_matrix (a one-time conversion when the
        # weights are loaded, not timed); the row-major copies are dropped.
        inp.weights = inp.packed_weights()
        torch.cuda.synchronize()
    cfg, keep = mk.make_cfg(**w.mk_fields())
    plan = mk.mk_plan(cfg)
    n_closed, _ = og.closed_form_counts(w.replace(join_nodes=0))
    scratch = torch.zeros(plan["scratch_bytes"], dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    g = mk.mk_build_graph(cfg, inp.weight_ptrs(), scratch.data_ptr(), stream)
    modes = {"static": mk.MK_SCHED_STATIC, "dynamic": mk.MK_SCHED_DYNAMIC, "levels": mk.MK_SCHED_LEVELS}
    g.mk_set_schedule(modes[args.schedule])
    tasks = g.tasks_bytes()
    n_nop = int((tasks[:, :2].copy().view(np.uint16)[:, 0] == 0).sum())  # op_id NOP = 0
    assert plan["n_tasks"] - n_nop == n_closed, "timed graph must hold every layer and the lm_head"
    ptrs = inp.step_ptrs()
    torch.cuda.synchronize()
    if args.copy_calibration:
        from synth import native
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            native.gpu_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: 3 x {args.copy_calibration} MiB")

    # Both paths must agree before anything is timed.
    g.mk_decode_step(stream, *ptrs)
    assert g.mk_status() == 0
    mega = inp.logits.clone()
    if not args.no_per_op:
        g.mk_decode_step_per_op(stream, *ptrs)
        torch.cuda.synchronize()
        per_op_logits = inp.logits.clone()
        diff = (per_op_logits - mega).abs().max().item()
        assert diff <= 2e-2, f"per-op and persistent logits differ by {diff}"
    log(f"graph: {plan['n_tasks']} tasks, {plan['n_edges']} edges, {plan['n_levels']} levels, grid {g.mk_graph_grid()}")

    total, per = timed(g.mk_decode_step, args.steps, args.warmup, stream, ptrs)
    assert g.mk_status() == 0
    ms = total / args.steps
    tok_s = w.batch * args.steps / (total / 1e3)
    bytes_step = w.bytes_per_step()
    achieved = bytes_step / (ms / 1e3) / 1e9
    log(f"persistent: {ms:.4f} ms/step, {tok_s:.1f} tok/s, {achieved:.0f} GB/s")

    # Secondary denominator: what a plain streaming read reaches on this part (2 GiB,
    # well past the 256 MB memory-side cache), timed the same way on the same stream.
    from synth import native
    n_read = 2 << 30
    src = torch.empty(n_read, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    for _ in range(2):
        native.gpu_read(src.data_ptr(), n_read, sink.data_ptr(), 2048, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        native.gpu_read(src.data_ptr(), n_read, sink.data_ptr(), 2048, stream)
    e1.record()
    torch.cuda.synchronize()
    stream_gbs = 5 * n_read / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, sink
    stream_ceiling = {"value": stream_gbs, "unit": "GB/s", "bytes": n_read, "kernel": "read16_kernel (plain read)",
                      "frac": achieved / stream_gbs}
    log(f"streaming-read ceiling: {stream_gbs:.0f} GB/s; the step reaches {achieved / stream_gbs:.3f} of it")

    alt = None
    if not args.no_alt_schedule:
        # The other schedule modes on the same graph: dynamic tickets, and the
        # level-synchronous kernel (grid barrier between levels, no counters), each
        # checked bitwise against the timed mode's logits first.
        alt = []
        ref_logits = inp.logits.clone()
        for other in [m for m in modes if m != args.schedule]:
            g.mk_set_schedule(modes[other])
            g.mk_decode_step(stream, *ptrs)
            assert g.mk_status() == 0
            assert torch.equal(inp.logits, ref_logits), f"{other} schedule differs from {args.schedule}"
            t_alt, _ = timed(g.mk_decode_step, args.steps, args.warmup, stream, ptrs)
            assert g.mk_status() == 0
            alt.append({"schedule": other, "ms_per_step": t_alt / args.steps})
            log(f"persistent, {other} schedule: {t_alt / args.steps:.4f} ms/step")
        g.mk_set_schedule(modes[args.schedule])

    per_op = None
    if not args.no_per_op:
        t2, per2 = timed(g.mk_decode_step_per_op, args.steps, args.warmup, stream, ptrs)
        ms2 = t2 / args.steps
        per_op = {"ms_per_step": ms2, "value": w.batch * args.steps / (t2 / 1e3), "unit": "tokens/s",
                  "launches_per_step": 2 + 7 * w.n_layers,
                  "latency_ms_median": float(np.median(per2)),
                  "speedup_of_persistent": ms2 / ms}
        log(f"per-op baseline: {ms2:.4f} ms/step")
        # The same launches captured once into a HIP graph and replayed: no host cost
        # per launch, one kernel boundary per op still.  Checked bitwise against the
        # eager per-op step before it is timed.
        g.mk_decode_step_per_op(stream, *ptrs)
        torch.cuda.synchronize()
        eager = inp.logits.clone()
        g.mk_capture_per_op_graph(*ptrs)
        inp.logits.zero_()
        g.mk_launch_per_op_graph(stream)
        assert g.mk_status() == 0
        torch.cuda.synchronize()
        assert torch.equal(inp.logits, eager), "graph replay of the per-op launches differs from the eager step"
        t3, per3 = timed(lambda s, *p: g.mk_launch_per_op_graph(s), args.steps, args.warmup, stream, ptrs)
        assert g.mk_status() == 0
        per_op["graph_replay"] = {"ms_per_step": t3 / args.steps, "latency_ms_median": float(np.median(per3)),
                                  "speedup_of_persistent": (t3 / args.steps) / ms}
        log(f"per-op baseline, HIP graph replay: {t3 / args.steps:.4f} ms/step")

    if args.trace_out:
        tr = torch.zeros(plan["n_tasks"] * 8, dtype=torch.int64, device="cuda")
        g.mk_set_trace(tr.data_ptr())
        g.mk_decode_step(stream, *ptrs)
        torch.cuda.synchronize()
        g.mk_set_trace(None)
        trace = tr.cpu().numpy().reshape(-1, 8)
        np.save(args.trace_out, trace)
        np.save(args.trace_out.replace(".npy", "_tasks.npy"), tasks)
        from task_graph_interpreter_amd import trace as mktrace
        summary = mktrace.summarize(trace, tasks)
        with open(args.trace_out.replace(".npy", "_summary.json"), "w") as f:
            json.dump(summary, f, indent=1)
        log("trace summary:\n" + mktrace.format_summary(summary))
        del tr

    n_greedy = args.greedy_tokens if args.greedy_tokens >= 0 else (256 if w.batch == 1 else 0)
    greedy = greedy_run(w, inp, n_greedy, stream) if n_greedy > 0 else None

    traffic = (measured_traffic(w.name)
               if not (args.kv_chunk or args.gemv_tiles or args.gemv_config >= 0 or args.packed >= 0) else None)
    name_timed = g.mk_graph_kernel_name()
    g.close()
    del scratch

    others = []
    shared = (model_key(w), inp.weights)
    for name in [n for n in args.others.split(",") if n and n != w.name]:
        others.append(time_other_workload(name, args.steps, args.warmup, stream, shared))
    del shared, inp, ptrs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w)
        cpu.pop("seconds_per_step_estimate", None)

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "hidden": w.hidden, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "intermediate": w.intermediate,
                   "vocab": w.vocab, "batch": w.batch, "kv_len": list(w.kv_len)[:4], "weight_dtype": w.weight_dtype,
                   "kv_dtype": w.kv_dtype, "gemv_tiles": w.gemv_tiles, "kv_chunk": w.kv_chunk,
                   "tasks": plan["n_tasks"], "edges": plan["n_edges"], "schedule": args.schedule,
                   "kernel": name_timed, "weight_layout": "tile16" if w.packed else "row-major"},
        "latency_ms": {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
                       "p90": float(np.percentile(per, 90))},
        "bytes_per_step": bytes_step,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "per_op_baseline": per_op,
        "other_schedule": alt,
        "stream_ceiling": stream_ceiling,
        "greedy": greedy,
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
