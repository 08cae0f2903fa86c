"""Workload shapes and the seeded recipe of every input tensor.

Five decoder workloads (the shapes of the decode configurations the method is
measured on) plus helpers that describe each input tensor: its canonical buffer
index (which doubles as the generator's tensor id), shape, storage dtype and the
(mean, std) of its seeded Irwin-Hall draw.  No arithmetic of the decode step
lives here.

Canonical buffer order (append-only, one index per tensor the graph touches):

    0 tokens, 1 positions, 2 embedding,
    per layer l (base 3 + 8 l): attn_norm, W_qkv, W_o, mlp_norm, W_gate_up,
                                W_down, kcache_l, vcache_l,
    3 + 8 L final_norm, 4 + 8 L W_lm,
    then the step's activations in emission order
    (x0, per layer qkv_out, q_rot, partials, att, h, gu, x_out), then logits.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

from . import gen

TOKENS_TID = 0
LENGTHS_TID = 1

LAYER_BASE = 3
PER_LAYER = 8
ATTN_NORM, W_QKV, W_O, MLP_NORM, W_GATE_UP, W_DOWN, KCACHE, VCACHE = range(8)

WEIGHT_STD = 0.02
NORM_MEAN, NORM_STD = 1.0, 0.01
KV_STD = 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    batch: int
    weight_dtype: str  # 'f32' | 'bf16'
    kv_dtype: str
    gemv_tiles: int
    kv_chunk: int
    kv_len: tuple  # attended length per sequence, new token included
    kv_capacity: int
    gemv_config: int  # 0 fp32, 1 bf16 vector, 2 bf16 MFMA
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    join_nodes: int = 1
    unfused: int = 0  # 1: lower without the epilogue-fusion pass (standalone RMSNORM tasks)
    sample: int = 0   # 1: SAMPLE tasks after the lm_head (a whole greedy step per launch)
    packed: int = 0   # 1: matrices in the library's 16-row tile layout (MFMA GEMV only)
    seed: int = 0
    meta: dict = field(default_factory=dict, compare=False)

    # ---- derived sizes -------------------------------------------------
    @property
    def grp(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def qkv_cols(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_cols(self) -> int:
        return self.n_q_heads * self.head_dim

    def chunks(self, b: int) -> int:
        return -(-self.kv_len[b] // self.kv_chunk)

    def n_buffers_weights(self) -> int:
        return LAYER_BASE + PER_LAYER * self.n_layers + 2

    def tid_layer(self, l: int, which: int) -> int:
        return LAYER_BASE + PER_LAYER * l + which

    @property
    def tid_final_norm(self) -> int:
        return LAYER_BASE + PER_LAYER * self.n_layers

    @property
    def tid_lm(self) -> int:
        return LAYER_BASE + PER_LAYER * self.n_layers + 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def with_steps(self, n_steps: int) -> "Workload":
        """The same workload with room for ``n_steps`` greedy tokens: positions run from
        kv_len-1 to kv_len-2+n_steps, so the graph plans kv_len+n_steps-1 keys."""
        extra = n_steps - 1
        kv = tuple(L + extra for L in self.kv_len)
        return self.replace(kv_len=kv, kv_capacity=max(self.kv_capacity, max(kv)),
                            name=f"{self.name}+{n_steps}steps")

    def mk_fields(self) -> dict:
        """Keyword arguments of the library's model configuration for this workload."""
        return dict(n_layers=self.n_layers, hidden=self.hidden, n_q_heads=self.n_q_heads,
                    n_kv_heads=self.n_kv_heads, head_dim=self.head_dim, intermediate=self.intermediate,
                    vocab=self.vocab, batch=self.batch, rms_eps=self.rms_eps, rope_theta=self.rope_theta,
                    weight_dtype=self.weight_dtype, kv_dtype=self.kv_dtype, gemv_tiles=self.gemv_tiles,
                    kv_chunk=self.kv_chunk, join_nodes=self.join_nodes, gemv_config=self.gemv_config,
                    kv_capacity=self.kv_capacity, kv_len=self.kv_len,
                    options=(1 if self.unfused else 0) | (2 if self.sample else 0) | (4 if self.packed else 0))

    # ---- per-step inputs ----------------------------------------------
    def tokens(self) -> np.ndarray:
        return gen.uniform_int(self.seed, TOKENS_TID, np.arange(self.batch), self.vocab).astype(np.int32)

    def positions(self) -> np.ndarray:
        return np.asarray(self.kv_len, dtype=np.int32) - 1

    # ---- tensor recipes -------------------------------------------------
    def weight_specs(self):
        """(tid, name, shape, mean, std, dtype) of every weight tensor, canonical order."""
        H, wd = self.hidden, self.weight_dtype
        specs = [(2, "embedding", (self.vocab, H), 0.0, WEIGHT_STD, wd)]
        for l in range(self.n_layers):
            t = lambda k: self.tid_layer(l, k)
            specs += [
                (t(ATTN_NORM), f"l{l}.attn_norm", (H,), NORM_MEAN, NORM_STD, wd),
                (t(W_QKV), f"l{l}.W_qkv", (self.qkv_cols, H), 0.0, WEIGHT_STD, wd),
                (t(W_O), f"l{l}.W_o", (H, self.q_cols), 0.0, WEIGHT_STD, wd),
                (t(MLP_NORM), f"l{l}.mlp_norm", (H,), NORM_MEAN, NORM_STD, wd),
                (t(W_GATE_UP), f"l{l}.W_gate_up", (2 * self.intermediate, H), 0.0, WEIGHT_STD, wd),
                (t(W_DOWN), f"l{l}.W_down", (H, self.intermediate), 0.0, WEIGHT_STD, wd),
            ]
        specs += [
            (self.tid_final_norm, "final_norm", (H,), NORM_MEAN, NORM_STD, wd),
            (self.tid_lm, "W_lm", (self.vocab, H), 0.0, WEIGHT_STD, wd),
        ]
        return specs

    def cache_shape(self):
        """Per-layer cache slab [batch, kv_heads, capacity, head_dim]."""
        return (self.batch, self.n_kv_heads, self.kv_capacity, self.head_dim)

    # ---- byte accounting (algorithmic bytes of one step) ---------------
    def weight_bytes_per_step(self) -> int:
        es = 4 if self.weight_dtype == "f32" else 2
        H, I, V = self.hidden, self.intermediate, self.vocab
        per_layer = (self.qkv_cols * H + H * self.q_cols + 2 * I * H + H * I + 2 * H)
        return es * (self.n_layers * per_layer + V * H + H + self.batch * H)

    def kv_bytes_per_step(self) -> int:
        es = 4 if self.kv_dtype == "f32" else 2
        return es * 2 * self.n_layers * self.n_kv_heads * self.head_dim * int(sum(self.kv_len))

    def bytes_per_step(self) -> int:
        return self.weight_bytes_per_step() + self.kv_bytes_per_step()


def _ragged_lengths(seed: int, batch: int, lo: int, hi: int):
    n = hi - lo + 1
    return tuple(int(lo + v) for v in gen.uniform_int(seed, LENGTHS_TID, np.arange(batch), n))


def tiny() -> Workload:
    return Workload(name="tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                    intermediate=512, vocab=1024, batch=1, weight_dtype="f32", kv_dtype="f32",
                    gemv_tiles=8, kv_chunk=32, kv_len=(128,), kv_capacity=128, gemv_config=0)


def llama1b() -> Workload:
    return Workload(name="1b_b1", n_layers=16, hidden=2048, n_q_heads=32, n_kv_heads=8, head_dim=64,
                    intermediate=8192, vocab=128256, batch=1, weight_dtype="bf16", kv_dtype="bf16",
                    gemv_tiles=256, kv_chunk=128, kv_len=(1024,), kv_capacity=1024, gemv_config=1)


def llama1b_kv512() -> Workload:
    # The first page's measured point: 1B-class decoder, 512 cached tokens, greedy decode.
    return llama1b().replace(name="1b_b1_kv512", kv_len=(512,), kv_capacity=512)


def llama8b() -> Workload:
    return Workload(name="8b_b1", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
                    intermediate=14336, vocab=128256, batch=1, weight_dtype="bf16", kv_dtype="bf16",
                    gemv_tiles=256, kv_chunk=128, kv_len=(2048,), kv_capacity=2048, gemv_config=1)


def llama8b_ragged(seed: int = 0) -> Workload:
    kv = _ragged_lengths(seed, 8, 512, 8192)
    return llama8b().replace(name="8b_b8_ragged", batch=8, kv_chunk=512, kv_len=kv,
                             kv_capacity=max(kv), seed=seed, gemv_config=2, packed=1)


def llama8b_long() -> Workload:
    return llama8b().replace(name="8b_b32_32k", batch=32, kv_chunk=8192, kv_len=(32768,) * 32,
                             kv_capacity=32768, gemv_config=2)


WORKLOADS = {
    "tiny": tiny,
    "1b_b1": llama1b,
    "1b_b1_kv512": llama1b_kv512,
    "8b_b1": llama8b,
    "8b_b8_ragged": llama8b_ragged,
    "8b_b32_32k": llama8b_long,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()
