"""Seeded input generator: the numpy definition, its C twin and bf16 rounding."""
import numpy as np
import pytest
import torch

from synth import gen, native, workloads


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not (__import__("os").path.exists(native.CPU_LIB)):
        native.build()


def test_mix64_matches_scalar_definition():
    # SplitMix64 reference values: state 0 -> first output of Vigna's splitmix64.c
    # with seed 0 is mix64(0x9E3779B97F4A7C15) = 0xE220A8397B1DCDAF.
    assert gen.mix64_int(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    w = gen.words(3, 7, np.arange(5))
    key = gen.stream_key(3, 7)
    for i in range(5):
        assert int(w[i]) == gen.mix64_int(key + (i + 1) * gen.G)


@pytest.mark.parametrize("dtype,mean,std", [("f32", 0.0, 0.02), ("bf16", 0.0, 0.02), ("bf16", 1.0, 0.01),
                                            ("f32", 0.0, 1.0)])
def test_c_twin_bit_exact(dtype, mean, std):
    a = gen.fill(0, 11, 50000, mean, std, dtype, start=987654321)
    b = native.cpu_fill_flat(50000, 987654321, 0, 11, mean, std, dtype)
    assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_c_twin_f64_widening():
    a = gen.to_f64(gen.fill(2, 4, 30000, 0.0, 0.02, "bf16", start=5), "bf16")
    b = native.cpu_fill_flat_f64(30000, 5, 2, 4, 0.0, 0.02, "bf16")
    assert np.array_equal(a, b)


def test_c_twin_cache_layout():
    hd = 64
    a = native.cpu_fill_cache(3, 2, 5, 7, hd, 0, 9, 0.0, 1.0, "bf16")
    bg, slot, d = np.meshgrid(np.arange(3, 5), np.arange(5, 12), np.arange(hd), indexing="ij")
    ref = gen.values(0, 9, gen.cache_index(bg, slot, d, hd), 0.0, 1.0, "bf16")
    assert np.array_equal(a, ref)


def test_moments_and_range():
    v = gen.to_f64(gen.fill(1, 2, 400000, 0.0, 0.02, "f32"), "f32")
    assert abs(v.mean()) < 2e-4 and abs(v.std() - 0.02) < 2e-4
    # Irwin-Hall(4) centred support is +-2*sqrt(3) standard deviations.
    assert np.abs(v).max() <= 0.02 * 2 * np.sqrt(3) * (1 + 1e-6)


def test_bf16_rounding_matches_torch():
    x = gen.values_f64(5, 5, np.arange(100000), 0.0, 3.0).astype(np.float32)
    ours = gen.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_tokens_and_lengths_in_range():
    w = workloads.llama8b_ragged()
    assert all(512 <= L <= 8192 for L in w.kv_len) and len(set(w.kv_len)) > 1
    for name in workloads.WORKLOADS:
        wl = workloads.get(name)
        t = wl.tokens()
        assert t.shape == (wl.batch,) and (t >= 0).all() and (t < wl.vocab).all()
        assert (wl.positions() == np.asarray(wl.kv_len) - 1).all()


def test_byte_accounting_closed_form():
    # 8B-class: per layer qkv 6144x4096, o 4096x4096, gate_up 28672x4096, down 4096x14336,
    # two gammas; plus lm_head 128256x4096, the final gamma and one embedding row; bf16.
    w = workloads.llama8b()
    per_layer = 6144 * 4096 + 4096 * 4096 + 28672 * 4096 + 4096 * 14336 + 2 * 4096
    assert w.weight_bytes_per_step() == 2 * (32 * per_layer + 128256 * 4096 + 4096 + 4096)
    assert w.kv_bytes_per_step() == 2 * 2 * 32 * 8 * 128 * 2048
