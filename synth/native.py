"""Build and load the C and HIP twins of the seeded generator (see gen.py)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import gen

HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB = os.path.join(HERE, "libsynth_cpu.so")
GPU_LIB = os.path.join(HERE, "libsynth_fill.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    cmds = [
        ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
         os.path.join(HERE, "gen_cpu.c"), "-o", CPU_LIB + ".tmp"],
        ["hipcc", *HIP_FLAGS, os.path.join(HERE, "fill.hip"), "-o", GPU_LIB + ".tmp"],
    ]
    for cmd, out in zip(cmds, (CPU_LIB, GPU_LIB)):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)
        os.replace(out + ".tmp", out)


_cpu = None
_gpu = None


def cpu_lib():
    global _cpu
    if _cpu is None:
        if not os.path.exists(CPU_LIB):
            raise RuntimeError(f"{CPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(CPU_LIB)
        u64, dbl = ctypes.c_uint64, ctypes.c_double
        lib.synth_fill_flat.argtypes = [ctypes.c_void_p, ctypes.c_int, u64, u64, u64, u64, dbl, dbl]
        lib.synth_fill_flat.restype = None
        lib.synth_fill_flat_f64.argtypes = [ctypes.c_void_p, ctypes.c_int, u64, u64, u64, u64, dbl, dbl]
        lib.synth_fill_flat_f64.restype = None
        lib.synth_fill_cache.argtypes = [ctypes.c_void_p, ctypes.c_int, u64, u64, u64, u64, u64, u64,
                                         u64, u64, dbl, dbl]
        lib.synth_fill_cache.restype = None
        lib.synth_stream_key.argtypes = [u64, u64]
        lib.synth_stream_key.restype = u64
        _cpu = lib
    return _cpu


def gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_LIB):
            raise RuntimeError(f"{GPU_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB)
        u64, dbl, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        lib.synth_gpu_fill_flat.argtypes = [vp, ctypes.c_int, u64, u64, u64, u64, dbl, dbl, vp]
        lib.synth_gpu_fill_flat.restype = ctypes.c_int
        lib.synth_gpu_fill_cache.argtypes = [vp, ctypes.c_int, u64, u64, u64, u64, u64, u64, dbl, dbl, vp]
        lib.synth_gpu_copy.argtypes = [vp, vp, u64, vp]
        lib.synth_gpu_copy.restype = ctypes.c_int
        lib.synth_gpu_read.argtypes = [vp, u64, vp, ctypes.c_uint32, vp]
        lib.synth_gpu_read.restype = ctypes.c_int
        lib.synth_gpu_fill_cache.restype = ctypes.c_int
        _gpu = lib
    return _gpu


def _dt(dtype: str) -> int:
    return {"f32": 0, "bf16": 1}[dtype]


def _np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def cpu_fill_flat(n: int, start: int, seed: int, tid: int, mean: float, std: float, dtype: str) -> np.ndarray:
    out = np.empty(n, dtype=_np_dtype(dtype))
    cpu_lib().synth_fill_flat(out.ctypes.data, _dt(dtype), n, start, seed, tid, mean, gen.scale_for(std))
    return out


def cpu_fill_flat_f64(n: int, start: int, seed: int, tid: int, mean: float, std: float, dtype: str) -> np.ndarray:
    """Stored values widened exactly to float64 (same as gen.to_f64 of cpu_fill_flat)."""
    out = np.empty(n, dtype=np.float64)
    cpu_lib().synth_fill_flat_f64(out.ctypes.data, _dt(dtype), n, start, seed, tid, mean, gen.scale_for(std))
    return out


def cpu_fill_cache(bg0: int, n_bg: int, slot0: int, n_slots: int, head_dim: int, seed: int, tid: int,
                   mean: float, std: float, dtype: str) -> np.ndarray:
    out = np.empty((n_bg, n_slots, head_dim), dtype=_np_dtype(dtype))
    cpu_lib().synth_fill_cache(out.ctypes.data, _dt(dtype), bg0, n_bg, slot0, n_slots, head_dim,
                               gen.CACHE_SLOT_PITCH, seed, tid, mean, gen.scale_for(std))
    return out


def gpu_fill_flat(ptr: int, n: int, start: int, seed: int, tid: int, mean: float, std: float,
                  dtype: str, stream: int) -> None:
    rc = gpu_lib().synth_gpu_fill_flat(ptr, _dt(dtype), n, start, seed, tid, mean, gen.scale_for(std), stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_flat failed: hip error {rc}")


def gpu_fill_cache(ptr: int, n_bg: int, n_slots: int, head_dim: int, seed: int, tid: int, mean: float,
                   std: float, dtype: str, stream: int) -> None:
    rc = gpu_lib().synth_gpu_fill_cache(ptr, _dt(dtype), n_bg, n_slots, head_dim, gen.CACHE_SLOT_PITCH,
                                        seed, tid, mean, gen.scale_for(std), stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_fill_cache failed: hip error {rc}")


def gpu_copy(dst_ptr: int, src_ptr: int, n_bytes: int, stream: int = 0) -> None:
    """Plain 16-byte device copy (byte-counter calibration)."""
    rc = gpu_lib().synth_gpu_copy(dst_ptr, src_ptr, n_bytes, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_copy failed ({rc})")


def gpu_read(src_ptr: int, n_bytes: int, out_ptr: int, blocks: int, stream: int = 0) -> None:
    """Plain streaming read of n_bytes (a multiple of 16); out_ptr: `blocks` uint32 words."""
    rc = gpu_lib().synth_gpu_read(src_ptr, n_bytes, out_ptr, blocks, stream)
    if rc != 0:
        raise RuntimeError(f"synth_gpu_read failed ({rc})")
