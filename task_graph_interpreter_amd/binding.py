"""Thin ctypes binding of libmk.so (declared in include/mk.h).

Argument marshalling only: every step of the decode path runs in the library's HIP
kernels.  Functions keep the C names; device memory and streams are passed as
integer addresses (for example ``tensor.data_ptr()`` and
``torch.cuda.current_stream().cuda_stream``).  Loading fails loudly if the library
has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmk.so")

MK_ABI_VERSION = 1
MK_OK, MK_ERR_ABI, MK_ERR_INVALID, MK_ERR_ALIGN, MK_ERR_HIP, MK_ERR_NOMEM, MK_ERR_DEVICE = 0, -1, -2, -3, -4, -5, -6
MK_STATUS_TIMEOUT, MK_STATUS_BAD_POSITION, MK_STATUS_BAD_TOKEN = 0x10000000, 0x20000000, 0x30000000
MK_STATUS_KIND_MASK = 0xF0000000
MK_SCHED_STATIC, MK_SCHED_DYNAMIC, MK_SCHED_LEVELS = 0, 1, 2
MK_STATIC_SCRATCH_BYTES = 64 << 20
# OpIds and flag bits of the descriptor (mk.h).
(MK_OP_NOP, MK_OP_MEMCPY, MK_OP_GEMV, MK_OP_RMSNORM, MK_OP_ATTENTION, MK_OP_MLP, MK_OP_SAMPLE,
 MK_OP_ATTENTION_APPEND, MK_OP_ATTENTION_PARTIAL, MK_OP_ATTENTION_COMBINE) = range(10)
MK_FLAG_SILU_MUL, MK_FLAG_ADD_RESIDUAL, MK_FLAG_RMS_NORM_INPUT = 1, 2, 4
MK_FLAG_FUSED_RESIDUAL = 2
MK_LOWER_UNFUSED, MK_LOWER_SAMPLE, MK_LOWER_PACKED_WEIGHTS = 1, 2, 4
# numpy mirror of mk_task_t (64 bytes), for reading the descriptor array on the host.
MK_TASK_DTYPE = np.dtype({
    "names": ["op_id", "config_id", "step", "flags", "remaining_deps", "num_dependents", "dependents_offset",
              "in_buf", "out_buf", "m", "n", "k", "kv_len", "reserved"],
    "formats": ["<u2", "<u2", "<u2", "<u2", "<i4", "<i4", "<u4", ("<u2", (3,)), "<u2", "<i4", "<i4", "<i4", "<i4",
                ("<u4", (5,))],
    "offsets": [0, 2, 4, 6, 8, 12, 16, 20, 26, 28, 32, 36, 40, 44],
    "itemsize": 64,
})
MK_DTYPE = {"f32": 0, "bf16": 1}

# Every symbol include/mk.h declares.
EXPORTS = ["mk_plan", "mk_lower", "mk_lowered_tasks", "mk_lowered_edges", "mk_lowered_scratch_span",
           "mk_lowered_levels", "mk_lowered_free", "mk_build_graph", "mk_graph_tasks", "mk_graph_edges", "mk_decode_step",
           "mk_decode_step_noalloc", "mk_decode_step_per_op", "mk_sample_greedy", "mk_pack_matrix", "mk_decode_greedy", "mk_capture_per_op_graph",
           "mk_launch_per_op_graph", "mk_status",
           "mk_set_wait_limit", "mk_set_trace", "mk_graph_grid", "mk_graph_kernel_name", "mk_set_schedule", "mk_graph_schedule", "mk_lowered_schedule", "mk_destroy", "mk_last_error", "mk_abi_version"]


class MkTask(ctypes.Structure):
    _fields_ = [("op_id", ctypes.c_uint16), ("config_id", ctypes.c_uint16), ("step", ctypes.c_uint16),
                ("flags", ctypes.c_uint16), ("remaining_deps", ctypes.c_int32), ("num_dependents", ctypes.c_int32),
                ("dependents_offset", ctypes.c_uint32), ("in_buf", ctypes.c_uint16 * 3),
                ("out_buf", ctypes.c_uint16), ("m", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("kv_len", ctypes.c_int32), ("reserved", ctypes.c_uint32 * 5)]


class MkModelCfg(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("struct_size", ctypes.c_uint32),
                ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("batch", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("weight_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("gemv_tiles", ctypes.c_int32), ("kv_chunk", ctypes.c_int32), ("join_nodes", ctypes.c_int32),
                ("gemv_config", ctypes.c_int32), ("kv_capacity", ctypes.c_int32), ("options", ctypes.c_int32),
                ("kv_len", ctypes.POINTER(ctypes.c_int32))]


class MkWeights(ctypes.Structure):
    _fields_ = [("count", ctypes.c_uint32), ("dev_ptrs", ctypes.POINTER(ctypes.c_void_p))]


class MkPlanInfo(ctypes.Structure):
    _fields_ = [("n_tasks", ctypes.c_uint32), ("n_edges", ctypes.c_uint32), ("n_buffers", ctypes.c_uint32),
                ("n_levels", ctypes.c_uint32), ("scratch_bytes", ctypes.c_uint64),
                ("kv_layer_bytes", ctypes.c_uint64)]


class MkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mk error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
    P = ctypes.POINTER
    sig = {
        "mk_plan": ([P(MkModelCfg), P(MkPlanInfo)], i32),
        "mk_lower": ([P(MkModelCfg), P(vp)], i32),
        "mk_lowered_tasks": ([vp, P(P(MkTask)), P(u32)], i32),
        "mk_lowered_edges": ([vp, P(P(u32)), P(u32)], i32),
        "mk_lowered_scratch_span": ([vp, u32, P(u64), P(u64)], i32),
        "mk_lowered_levels": ([vp, P(P(u32)), P(P(u32)), P(u32)], i32),
        "mk_lowered_free": ([vp], None),
        "mk_build_graph": ([P(MkModelCfg), P(MkWeights), vp, vp, P(vp)], i32),
        "mk_graph_tasks": ([vp, P(P(MkTask)), P(u32)], i32),
        "mk_graph_edges": ([vp, P(P(u32)), P(u32)], i32),
        "mk_decode_step": ([vp, vp, vp, vp, vp, vp, vp], i32),
        "mk_decode_step_noalloc": ([vp, vp, vp, vp, vp, vp, vp], i32),
        "mk_decode_step_per_op": ([vp, vp, vp, vp, vp, vp, vp], i32),
        "mk_sample_greedy": ([vp, vp, vp, vp, vp], i32),
        "mk_pack_matrix": ([vp, vp, i32, i32, vp], i32),
        "mk_decode_greedy": ([vp, vp, i32, vp, vp, vp, vp, vp, vp], i32),
        "mk_capture_per_op_graph": ([vp, vp, vp, vp, vp, vp], i32),
        "mk_launch_per_op_graph": ([vp, vp], i32),
        "mk_status": ([vp, P(u32)], i32),
        "mk_set_wait_limit": ([vp, u64], i32),
        "mk_set_trace": ([vp, vp], i32),
        "mk_graph_grid": ([vp, P(u32)], i32),
        "mk_graph_kernel_name": ([vp], ctypes.c_char_p),
        "mk_set_schedule": ([vp, i32], i32),
        "mk_graph_schedule": ([vp, P(P(u32)), P(P(u32)), P(u32), P(ctypes.c_double)], i32),
        "mk_lowered_schedule": ([vp, u32, P(P(u32)), P(P(u32)), P(ctypes.c_double)], i32),
        "mk_destroy": ([vp], None),
        "mk_last_error": ([], ctypes.c_char_p),
        "mk_abi_version": ([], u32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    if L.mk_abi_version() != MK_ABI_VERSION:
        raise RuntimeError("libmk.so ABI version differs from the binding's")
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != MK_OK:
        raise MkError(rc, lib().mk_last_error().decode())


def mk_last_error() -> str:
    return lib().mk_last_error().decode()


def mk_abi_version() -> int:
    return int(lib().mk_abi_version())


def make_cfg(*, n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab, batch, rms_eps,
             rope_theta, weight_dtype, kv_dtype, gemv_tiles, kv_chunk, join_nodes, gemv_config, kv_capacity,
             kv_len, options=0):
    """Build an mk_model_cfg; returns (cfg, keepalive) -- keep both alive during calls."""
    kv = (ctypes.c_int32 * batch)(*[int(v) for v in kv_len])
    c = MkModelCfg(MK_ABI_VERSION, ctypes.sizeof(MkModelCfg), n_layers, hidden, n_q_heads, n_kv_heads, head_dim,
                   intermediate, vocab, batch, rms_eps, rope_theta, MK_DTYPE[weight_dtype], MK_DTYPE[kv_dtype],
                   gemv_tiles, kv_chunk, join_nodes, gemv_config, kv_capacity, options,
                   ctypes.cast(kv, ctypes.POINTER(ctypes.c_int32)))
    return c, kv


def mk_pack_matrix(src_dev: int, dst_dev: int, rows: int, cols: int, stream: int) -> None:
    """16-row tile layout of a bf16 [rows, cols] matrix into dst (device addresses)."""
    _check(lib().mk_pack_matrix(src_dev, dst_dev, rows, cols, stream))


def packed_matrix_indices(n_layers: int) -> list:
    """Indices (canonical weight order) of the matrices MK_LOWER_PACKED_WEIGHTS covers:
    per layer W_qkv, W_o, W_gate_up, W_down, then W_lm."""
    out = []
    for l in range(n_layers):
        out += [1 + 6 * l + 1, 1 + 6 * l + 2, 1 + 6 * l + 4, 1 + 6 * l + 5]
    return out + [2 + 6 * n_layers]


def mk_plan(cfg: MkModelCfg) -> dict:
    info = MkPlanInfo()
    _check(lib().mk_plan(ctypes.byref(cfg), ctypes.byref(info)))
    return {k: getattr(info, k) for k, _ in MkPlanInfo._fields_}


def _tasks_to_numpy(ptr, n) -> np.ndarray:
    raw = ctypes.string_at(ptr, n * 64) if n else b""
    return np.frombuffer(raw, dtype=np.uint8).reshape(n, 64).copy()


def _schedule_to_numpy(order_ptr, off_ptr, workers):
    offsets = np.ctypeslib.as_array(off_ptr, shape=(workers + 1,)).copy()
    n = int(offsets[-1])
    order = np.ctypeslib.as_array(order_ptr, shape=(n,)).copy() if n else np.zeros(0, np.uint32)
    return order, offsets


def _edges_to_numpy(ptr, n) -> np.ndarray:
    if n == 0:
        return np.zeros(0, dtype=np.uint32)
    return np.ctypeslib.as_array(ptr, shape=(n,)).copy()


class Lowered:
    """Host-only lowering (mk_lower): raw descriptor bytes and edges, no GPU needed."""

    def __init__(self, cfg: MkModelCfg):
        h = ctypes.c_void_p()
        _check(lib().mk_lower(ctypes.byref(cfg), ctypes.byref(h)))
        self.h = h

    def tasks_bytes(self) -> np.ndarray:
        p, n = ctypes.POINTER(MkTask)(), ctypes.c_uint32()
        _check(lib().mk_lowered_tasks(self.h, ctypes.byref(p), ctypes.byref(n)))
        return _tasks_to_numpy(p, n.value)

    def edges(self) -> np.ndarray:
        p, n = ctypes.POINTER(ctypes.c_uint32)(), ctypes.c_uint32()
        _check(lib().mk_lowered_edges(self.h, ctypes.byref(p), ctypes.byref(n)))
        return _edges_to_numpy(p, n.value)

    def schedule(self, workers: int):
        """Static schedule for `workers` workgroups: ((order, offsets), est_us)."""
        o, f, est = ctypes.POINTER(ctypes.c_uint32)(), ctypes.POINTER(ctypes.c_uint32)(), ctypes.c_double()
        _check(lib().mk_lowered_schedule(self.h, workers, ctypes.byref(o), ctypes.byref(f), ctypes.byref(est)))
        return _schedule_to_numpy(o, f, workers), est.value

    def levels(self):
        """Level-synchronous lists: a list of int arrays, one per level, in run order."""
        t, f, n = ctypes.POINTER(ctypes.c_uint32)(), ctypes.POINTER(ctypes.c_uint32)(), ctypes.c_uint32()
        _check(lib().mk_lowered_levels(self.h, ctypes.byref(t), ctypes.byref(f), ctypes.byref(n)))
        offs = np.ctypeslib.as_array(f, shape=(n.value + 1,)).copy()
        tasks = np.ctypeslib.as_array(t, shape=(int(offs[-1]),)).copy() if offs[-1] else np.zeros(0, np.uint32)
        return [tasks[offs[i]:offs[i + 1]] for i in range(n.value)]

    def scratch_span(self, buf_index: int):
        off, nb = ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().mk_lowered_scratch_span(self.h, buf_index, ctypes.byref(off), ctypes.byref(nb)))
        return off.value, nb.value

    def close(self):
        if self.h:
            lib().mk_lowered_free(self.h)
            self.h = None

    __del__ = close


def mk_lower(cfg: MkModelCfg) -> Lowered:
    return Lowered(cfg)


class Graph:
    """An uploaded graph (mk_build_graph); methods wrap the per-graph entry points."""

    def __init__(self, cfg: MkModelCfg, weight_ptrs, scratch_ptr: int, stream: int):
        arr = (ctypes.c_void_p * len(weight_ptrs))(*[int(p) for p in weight_ptrs])
        w = MkWeights(len(weight_ptrs), ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
        h = ctypes.c_void_p()
        _check(lib().mk_build_graph(ctypes.byref(cfg), ctypes.byref(w), scratch_ptr, stream, ctypes.byref(h)))
        self.h = h

    def mk_decode_step(self, stream, tokens, positions, kcache, vcache, logits) -> None:
        _check(lib().mk_decode_step(self.h, stream, tokens, positions, kcache, vcache, logits))

    def mk_decode_step_noalloc(self, stream, tokens, positions, kcache, vcache, logits) -> None:
        _check(lib().mk_decode_step_noalloc(self.h, stream, tokens, positions, kcache, vcache, logits))

    def mk_decode_step_per_op(self, stream, tokens, positions, kcache, vcache, logits) -> None:
        _check(lib().mk_decode_step_per_op(self.h, stream, tokens, positions, kcache, vcache, logits))

    def mk_sample_greedy(self, stream, logits, tokens, positions) -> None:
        _check(lib().mk_sample_greedy(self.h, stream, logits, tokens, positions))

    def mk_decode_greedy(self, stream, n_steps, tokens, positions, kcache, vcache, logits, tokens_out=None) -> None:
        _check(lib().mk_decode_greedy(self.h, stream, n_steps, tokens, positions, kcache, vcache, logits, tokens_out))

    def mk_capture_per_op_graph(self, tokens, positions, kcache, vcache, logits) -> None:
        _check(lib().mk_capture_per_op_graph(self.h, tokens, positions, kcache, vcache, logits))

    def mk_launch_per_op_graph(self, stream) -> None:
        _check(lib().mk_launch_per_op_graph(self.h, stream))

    def mk_status(self) -> int:
        st = ctypes.c_uint32()
        rc = lib().mk_status(self.h, ctypes.byref(st))
        if rc not in (MK_OK, MK_ERR_DEVICE):
            _check(rc)
        return st.value

    def mk_set_wait_limit(self, ticks: int) -> None:
        _check(lib().mk_set_wait_limit(self.h, ticks))

    def mk_set_trace(self, trace_ptr: int | None) -> None:
        _check(lib().mk_set_trace(self.h, trace_ptr or None))

    def mk_graph_grid(self) -> int:
        n = ctypes.c_uint32()
        _check(lib().mk_graph_grid(self.h, ctypes.byref(n)))
        return n.value

    def mk_graph_kernel_name(self) -> str:
        return lib().mk_graph_kernel_name(self.h).decode()

    def mk_set_schedule(self, mode: int) -> None:
        _check(lib().mk_set_schedule(self.h, mode))

    def mk_graph_schedule(self):
        """(order, offsets, est_us) of the static schedule, as numpy copies."""
        o, f, w, est = (ctypes.POINTER(ctypes.c_uint32)(), ctypes.POINTER(ctypes.c_uint32)(), ctypes.c_uint32(),
                        ctypes.c_double())
        _check(lib().mk_graph_schedule(self.h, ctypes.byref(o), ctypes.byref(f), ctypes.byref(w),
                                       ctypes.byref(est)))
        return _schedule_to_numpy(o, f, w.value), est.value

    def tasks_bytes(self) -> np.ndarray:
        p, n = ctypes.POINTER(MkTask)(), ctypes.c_uint32()
        _check(lib().mk_graph_tasks(self.h, ctypes.byref(p), ctypes.byref(n)))
        return _tasks_to_numpy(p, n.value)

    def edges(self) -> np.ndarray:
        p, n = ctypes.POINTER(ctypes.c_uint32)(), ctypes.c_uint32()
        _check(lib().mk_graph_edges(self.h, ctypes.byref(p), ctypes.byref(n)))
        return _edges_to_numpy(p, n.value)

    def close(self) -> None:
        if getattr(self, "h", None):
            lib().mk_destroy(self.h)
            self.h = None

    __del__ = close


def mk_build_graph(cfg, weight_ptrs, scratch_ptr, stream) -> Graph:
    return Graph(cfg, weight_ptrs, scratch_ptr, stream)
