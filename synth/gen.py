"""Counter-based seeded generator for the synthetic weights, KV caches and tokens.

This module is shared by the CPU oracle side and by the GPU side of the tests and
the benchmark.  It holds no arithmetic of the decode method itself: only a
stateless random generator, written three times (numpy here, plain C in
``gen_cpu.c``, a HIP fill kernel in ``fill.hip``) so that any slice of any tensor
can be regenerated anywhere, bit for bit.

Definition (all integer arithmetic modulo 2**64):

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014; constants as in
  Vigna's public-domain ``splitmix64.c``)::

      z ^= z >> 30; z *= 0xBF58476D1CE4E5B9
      z ^= z >> 27; z *= 0x94D049BB133111EB
      z ^= z >> 31

* ``key(seed, tid) = mix64(mix64(seed + G) + (tid + 1) * G)`` with
  ``G = 0x9E3779B97F4A7C15``; ``tid`` is the tensor's buffer index.
* ``word(seed, tid, i) = mix64(key + (i + 1) * G)``: the i-th output of a
  SplitMix64 stream that starts at ``key``.
* The four 16-bit fields of the word are summed: ``S`` in [0, 262140].
  ``z = S - 131070`` is an Irwin-Hall(4) draw, centred, in units of 2**-16.
* ``v64 = mean + z * scale`` in IEEE binary64, with
  ``scale = std * sqrt(3) / 65536`` (so the variance is std**2 * (1 - 2**-32)),
  one multiply and one add, never fused.
* The stored value is ``v64`` rounded to binary32 (round to nearest even); for
  bfloat16 storage that binary32 value is rounded again to bfloat16 (nearest
  even on the top 16 bits).  bfloat16 tensors are handled as ``uint16`` bit
  patterns on the host.
"""
from __future__ import annotations

import numpy as np

G = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
HALF_RANGE = 131070  # 4 * 65535 / 2


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (scalar reference)."""
    z &= MASK64
    z ^= z >> 30
    z = (z * M1) & MASK64
    z ^= z >> 27
    z = (z * M2) & MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, tid: int) -> int:
    """Start state of the stream of tensor ``tid`` under ``seed``."""
    return mix64_int((mix64_int((seed + G) & MASK64) + (tid + 1) * G) & MASK64)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(M2)
    z = z ^ (z >> np.uint64(31))
    return z


def words(seed: int, tid: int, idx) -> np.ndarray:
    """64-bit words for element indices ``idx`` (any integer array-like)."""
    idx = np.asarray(idx, dtype=np.uint64)
    key = np.uint64(stream_key(seed, tid))
    with np.errstate(over="ignore"):
        state = key + (idx + np.uint64(1)) * np.uint64(G)
        return _mix64_np(state)


def irwin_hall(w: np.ndarray) -> np.ndarray:
    """Centred Irwin-Hall(4) integer in [-131070, 131070] from 64-bit words."""
    m = np.uint64(0xFFFF)
    s = (w & m) + ((w >> np.uint64(16)) & m) + ((w >> np.uint64(32)) & m) + (w >> np.uint64(48))
    return s.astype(np.int64) - HALF_RANGE


def scale_for(std: float) -> float:
    return float(np.float64(std) * np.sqrt(np.float64(3.0)) / np.float64(65536.0))


def values_f64(seed: int, tid: int, idx, mean: float, std: float) -> np.ndarray:
    z = irwin_hall(words(seed, tid, idx)).astype(np.float64)
    t = z * np.float64(scale_for(std))
    return np.float64(mean) + t


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 to bfloat16 (nearest even), returned as uint16 bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def values(seed: int, tid: int, idx, mean: float, std: float, dtype: str) -> np.ndarray:
    """Stored values: float32 array for 'f32', uint16 bfloat16 bits for 'bf16'."""
    v32 = values_f64(seed, tid, idx, mean, std).astype(np.float32)
    if dtype == "f32":
        return v32
    if dtype == "bf16":
        return f32_to_bf16_bits(v32)
    raise ValueError(f"unknown dtype {dtype!r}")


def fill(seed: int, tid: int, n: int, mean: float, std: float, dtype: str, start: int = 0) -> np.ndarray:
    return values(seed, tid, np.arange(start, start + n, dtype=np.uint64), mean, std, dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(stored).astype(np.float64)


# Cache tensors index their elements independently of the allocated capacity, so a
# cache of any capacity holds the same value at the same (sequence, head, slot, dim).
CACHE_SLOT_PITCH = 1 << 20


def cache_index(bg: np.ndarray, slot: np.ndarray, d: np.ndarray, head_dim: int) -> np.ndarray:
    """Generator index of cache element (sequence*kv_heads + head, slot, dim)."""
    bg = np.asarray(bg, dtype=np.uint64)
    slot = np.asarray(slot, dtype=np.uint64)
    d = np.asarray(d, dtype=np.uint64)
    return (bg * np.uint64(CACHE_SLOT_PITCH) + slot) * np.uint64(head_dim) + d


def uniform_int(seed: int, tid: int, idx, modulus: int) -> np.ndarray:
    """Integers ``word mod modulus`` (used for tokens and ragged lengths)."""
    return (words(seed, tid, idx) % np.uint64(modulus)).astype(np.int64)
