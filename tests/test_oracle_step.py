"""The oracle's whole decode step against the independent torch formulation, and
its multi-step cache semantics."""
import numpy as np
import torch

from oracle import decode as od
from oracle.params import GeneratedParams
from synth import workloads

import torch_reference as tr


def _torch_inputs(w, p):
    P = {}
    for tid, name, shape, *_ in w.weight_specs():
        P[name] = torch.from_numpy(p.matrix(tid) if len(shape) == 2 else p.vector(tid))
    cache = {}
    for l in range(w.n_layers):
        for b in range(w.batch):
            for which, key in ((0, "k"), (1, "v")):
                cache[(l, key, b)] = torch.from_numpy(np.stack(
                    [p.cache(l, which, b, g, w.kv_capacity) for g in range(w.n_kv_heads)]))
    return P, cache


def test_tiny_step_matches_torch_formulation():
    w = workloads.tiny()
    p = GeneratedParams(w)
    ours, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p))
    P, cache = _torch_inputs(w, p)
    theirs = tr.decode_step(w, P, w.tokens(), w.positions(), cache).numpy()
    np.testing.assert_allclose(ours, theirs, rtol=1e-10, atol=1e-10)


def test_tiny_batch3_gqa_matches_torch_formulation():
    w = workloads.tiny().replace(batch=3, kv_len=(128, 40, 97), n_q_heads=8, n_kv_heads=2, kv_dtype="bf16")
    p = GeneratedParams(w)
    ours, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p))
    ours_split, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), split=True)
    P, cache = _torch_inputs(w, p)
    theirs = tr.decode_step(w, P, w.tokens(), w.positions(), cache).numpy()
    np.testing.assert_allclose(ours, theirs, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(ours_split, ours, rtol=1e-12, atol=1e-12)


def test_rows_are_independent():
    w = workloads.tiny().replace(batch=3, kv_len=(128, 40, 97))
    p = GeneratedParams(w)
    full, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p))
    one, _ = od.decode_step(w, p, w.tokens(), w.positions(), od.KVState(p), rows=[1])
    # equal up to BLAS summation order
    np.testing.assert_allclose(full[1], one[0], rtol=1e-12, atol=1e-13)


def test_multistep_greedy_matches_torch_with_persistent_cache():
    w = workloads.tiny().with_steps(4)
    p = GeneratedParams(w)
    kv = od.KVState(p)
    P, cache = _torch_inputs(w, p)
    tok = w.tokens()
    pos = np.asarray(workloads.tiny().positions())
    for _ in range(4):
        ours, _ = od.decode_step(w, p, tok, pos, kv)
        theirs = tr.decode_step(w, P, tok, pos, cache).numpy()
        np.testing.assert_allclose(ours, theirs, rtol=1e-10, atol=1e-10)
        tok = np.array([od.greedy_token(ours[0])], dtype=np.int32)
        pos = pos + 1
    # the appended slots of every layer are in the oracle's cache
    assert len(kv.written) == 4 * w.n_layers * w.n_kv_heads * 2
