"""Pins of the oracle's building blocks against closed forms, textbook identities and
library routines (none of them re-types the oracle's own formula)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import decode as od

RNG = np.random.default_rng(1234)


def test_rms_inv_closed_forms():
    # constant vector c: mean(x^2) = c^2
    assert od.rms_inv(np.full(16, 3.0), 0.0) == pytest.approx(1 / 3.0, rel=1e-15)
    # [3, 4]: mean of squares 12.5
    assert od.rms_inv(np.array([3.0, 4.0]), 0.5) == pytest.approx(1 / np.sqrt(13.0), rel=1e-15)
    x = RNG.standard_normal(257)
    y = od.rmsnorm(x, np.ones(257), 0.0)
    assert np.sqrt(np.mean(y * y)) == pytest.approx(1.0, rel=1e-13)


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((3, 64))
    g = 1 + 0.1 * RNG.standard_normal(64)
    ours = np.stack([od.rmsnorm(r, g, 1e-6) for r in x])
    theirs = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(ours, theirs, rtol=1e-13, atol=1e-14)


def test_silu_identities_and_torch():
    t = np.linspace(-30, 30, 1001)
    s = od.silu(t)
    np.testing.assert_allclose(s, F.silu(torch.from_numpy(t)).numpy(), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(od.silu(t) - od.silu(-t), t, rtol=1e-12, atol=1e-12)  # t*sig(t) + t*sig(-t) = t
    assert od.silu(np.array([0.0]))[0] == 0.0


def test_rope_position_zero_is_identity():
    v = RNG.standard_normal((3, 64))
    np.testing.assert_array_equal(od.rope(v, 0, 10000.0), v)


def test_rope_matches_complex_rotation():
    # Rotate-half RoPE == multiply the complex number (v_i + j v_{i+hd/2}) by e^{j pos theta^(-2i/hd)}.
    hd, pos, theta = 128, 1234, 10000.0
    v = RNG.standard_normal(hd)
    z = v[: hd // 2] + 1j * v[hd // 2:]
    ang = pos * theta ** (-2.0 * np.arange(hd // 2) / hd)
    rz = z * np.exp(1j * ang)
    np.testing.assert_allclose(od.rope(v, pos, theta), np.concatenate([rz.real, rz.imag]), rtol=1e-12, atol=1e-12)


def test_rope_norm_and_relative_position():
    hd = 64
    q, k = RNG.standard_normal(hd), RNG.standard_normal(hd)
    for p in (1, 17, 4000):
        r = od.rope(q, p, 10000.0)
        pairs = lambda x: x[: hd // 2] ** 2 + x[hd // 2:] ** 2
        np.testing.assert_allclose(pairs(r), pairs(q), rtol=1e-12)
    d1 = od.rope(q, 100, 1e4) @ od.rope(k, 90, 1e4)
    d2 = od.rope(q, 1010, 1e4) @ od.rope(k, 1000, 1e4)
    assert d1 == pytest.approx(d2, rel=1e-9)


def test_softmax_attention_brute_force_and_torch():
    n, hd = 37, 16
    q, K, V = RNG.standard_normal(hd), RNG.standard_normal((n, hd)), RNG.standard_normal((n, hd))
    # brute force with explicit loops
    scores = [sum(q[d] * K[j, d] for d in range(hd)) / np.sqrt(hd) for j in range(n)]
    mx = max(scores)
    w = [np.exp(s - mx) for s in scores]
    ref = sum(wj * V[j] for j, wj in enumerate(w)) / sum(w)
    np.testing.assert_allclose(od.softmax_attention(q, K, V), ref, rtol=1e-12, atol=1e-13)
    t = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
                                       torch.from_numpy(V)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(od.softmax_attention(q, K, V), t, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    hd = 8
    q, K, V = RNG.standard_normal(hd), RNG.standard_normal((1, hd)), RNG.standard_normal((1, hd))
    np.testing.assert_allclose(od.softmax_attention(q, K, V), V[0], rtol=1e-15)   # one key -> its value
    K = np.tile(RNG.standard_normal(hd), (9, 1))
    V = RNG.standard_normal((9, hd))
    np.testing.assert_allclose(od.softmax_attention(q, K, V), V.mean(0), rtol=1e-12)  # equal keys -> mean


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 16, 40, 64])
def test_split_and_combine_equal_unsplit(chunk):
    n, hd = 40, 16
    q = RNG.standard_normal(hd) * 3
    K, V = RNG.standard_normal((n, hd)), RNG.standard_normal((n, hd))
    parts = [od.chunk_partial(q, K[i:i + chunk], V[i:i + chunk]) for i in range(0, n, chunk)]
    parts.append(od.chunk_partial(q, K[:0], V[:0]))   # an empty chunk merges as nothing
    np.testing.assert_allclose(od.combine(parts), od.softmax_attention(q, K, V), rtol=1e-12, atol=1e-13)


def test_chunk_partial_m_and_l_brute_force():
    # m is the largest score and l the sum of e^(s - m), each from explicit loops
    # over keys and dimensions; o against the same loop.  A wrong m with a matching
    # l would cancel in the merge, so they are pinned here on their own.
    n, hd = 23, 8
    q = RNG.standard_normal(hd) * 2
    K, V = RNG.standard_normal((n, hd)), RNG.standard_normal((n, hd))
    scores = []
    for j in range(n):
        acc = 0.0
        for d in range(hd):
            acc += q[d] * K[j, d]
        scores.append(acc / np.sqrt(hd))
    mx = scores[0]
    for s in scores[1:]:
        mx = s if s > mx else mx
    l_ref, o_ref = 0.0, np.zeros(hd)
    for j in range(n):
        e = np.exp(scores[j] - mx)
        l_ref += e
        o_ref = o_ref + e * V[j]
    m, l, o = od.chunk_partial(q, K, V)
    assert m == pytest.approx(mx, rel=1e-14, abs=1e-14)
    assert l == pytest.approx(l_ref, rel=1e-13)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-13)
    # the largest term of l is e^0 = 1, so 1 <= l <= n
    assert 1.0 <= l <= n


def test_chunk_partial_single_key():
    q, k, v = RNG.standard_normal(4), RNG.standard_normal((1, 4)), RNG.standard_normal((1, 4))
    m, l, o = od.chunk_partial(q, k, v)
    assert m == pytest.approx(float(q @ k[0]) / 2.0, rel=1e-14)  # sqrt(4) = 2
    assert l == 1.0
    np.testing.assert_array_equal(o, v[0])


def test_top2_margin():
    assert od.top2_margin(np.array([1.0, 5.0, 3.0])) == 2.0
    assert od.top2_margin(np.array([4.0, -1.0, 4.0])) == 0.0


def test_empty_chunk_partial():
    m, l, o = od.chunk_partial(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)))
    assert m == -np.inf and l == 0.0 and (o == 0).all()


def test_round_storage_matches_torch():
    v = RNG.standard_normal(10000) * 5
    np.testing.assert_array_equal(od.round_storage(v, "bf16"),
                                  torch.from_numpy(v).float().bfloat16().double().numpy())
    np.testing.assert_array_equal(od.round_storage(v, "f32"), v.astype(np.float32).astype(np.float64))


def test_greedy_lowest_index_on_ties():
    assert od.greedy_token(np.array([1.0, 3.0, 3.0, 2.0])) == 1
