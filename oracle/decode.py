"""Oracle: one transformer decode step in float64 -- TEST INFRASTRUCTURE ONLY.

What is computed follows "Mega kernel initial" (1y33.com): the decoder layer of the
graph-API section (qkv matmul with the attention RMSNorm fused, attention over the KV
cache, o projection plus residual, gate/up matmul with the MLP RMSNorm and SiLU*mul
fused, down projection plus residual), the lowering section's flash-decoding split
(partial per KV chunk, then a log-sum-exp merge) and its statement that the final
RMSNorm is fused into the lm_head matmul.

Readings where the pages are silent (both sides obey them; parity unpinned by the
pages, pinned by identities in the tests):
  * RMSNorm: y = x * (mean(x^2) + eps)^-1/2 * gamma.
  * SiLU(t) = t / (1 + e^-t); the gate is rows [0, I) of W_gate_up, up rows [I, 2I).
  * RoPE is the rotate-half form (pairs i, i + hd/2), angle pos * theta^(-2i/hd),
    applied to q and k of the new token only (the "RoPE-append" OpId); cached keys
    count as already rotated.
  * The appended k and v are stored in the cache dtype (binary32 then bfloat16,
    nearest even) before attention reads them.
  * Attention of sequence b reads cache slots [0, positions[b]] with scale 1/sqrt(hd);
    query head h uses KV head h // (n_q_heads / n_kv_heads).
  * Weight layout is row-major [out, in]; qkv rows are [q heads | k heads | v heads].
  * Every activation between ops is computed in float64 here (binary32 on the GPU).
"""
from __future__ import annotations

import numpy as np


def round_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing into a tensor of ``dtype`` (binary32, or binary32 then bfloat16),
    returned as float64."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return v32.astype(np.float64)
    u = v32.view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def rms_inv(x: np.ndarray, eps: float) -> float:
    """(mean(x^2) + eps)^(-1/2), the RMSNorm scale of one row."""
    return 1.0 / np.sqrt(np.mean(x * x) + eps)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    return x * rms_inv(x, eps) * gamma


def silu(t: np.ndarray) -> np.ndarray:
    return t / (1.0 + np.exp(-t))


def rope(v: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of the rows of v[..., hd] at position ``pos``."""
    hd = v.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Full (unsplit) attention of one query over keys K[n, hd], values V[n, hd]."""
    s = K @ q / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


def chunk_partial(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """Flash-decoding partial over one KV chunk: (m, l, o) with m = max score,
    l = sum e^(s-m), o = sum e^(s-m) v (unnormalised).  An empty chunk gives
    (-inf, 0, 0)."""
    hd = q.shape[-1]
    if K.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(hd)
    s = K @ q / np.sqrt(hd)
    m = s.max()
    e = np.exp(s - m)
    return m, e.sum(), e @ V


def combine(parts):
    """Log-sum-exp merge of (m, l, o) partials into the normalised attention output."""
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    M = ms.max()
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - M))
    lam = sum(wc * p[1] for wc, p in zip(w, parts))
    o = sum(wc * p[2] for wc, p in zip(w, parts))
    return o / lam


class KVState:
    """Oracle-side KV cache: the seeded pre-filled cache plus the slots later steps wrote."""

    def __init__(self, params):
        self.params = params
        self.written = {}  # (layer, which, b, g, slot) -> float64[hd]

    def keys_values(self, layer: int, b: int, g: int, n: int):
        K = self.params.cache(layer, 0, b, g, n).copy()
        V = self.params.cache(layer, 1, b, g, n).copy()
        for slot in range(n):
            kk = self.written.get((layer, 0, b, g, slot))
            if kk is not None:
                K[slot] = kk
            vv = self.written.get((layer, 1, b, g, slot))
            if vv is not None:
                V[slot] = vv
        return K, V


def decode_step(w, params, tokens, positions, kv: KVState, rows=None, keep: bool = False,
                split=False):
    """One decode step for the sequences in ``rows`` (default: all).

    Returns (logits[len(rows), vocab], inter) where ``inter`` (if ``keep``) maps
    activation names to per-row float64 arrays, using the names of the step's
    activation buffers (x0, and per layer qkv_out, q_rot, partials, att, h, gu, x_out),
    plus the values a graph lowered without epilogue fusion also stores: per layer xn
    (normed attention input), o (o projection before the residual), hn (normed MLP
    input), d (down projection before the residual), and xn_final.
    With ``split`` the attention is computed chunk by chunk and merged (the lowered
    form); otherwise by the plain softmax definition.
    """
    rows = list(range(w.batch)) if rows is None else list(rows)
    H, hd, Hq, Hkv, I = w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.intermediate
    grp = Hq // Hkv
    eps, theta = w.rms_eps, w.rope_theta
    inter = {} if keep else None

    x = np.stack([params.embedding_row(int(tokens[b])) for b in rows])  # [R, H]
    if keep:
        inter["x0"] = x.copy()
    for l in range(w.n_layers):
        g_attn = params.vector(w.tid_layer(l, 0))
        Wqkv = params.matrix(w.tid_layer(l, 1))
        xn = np.stack([rmsnorm(x[r], g_attn, eps) for r in range(len(rows))])
        qkv = xn @ Wqkv.T  # [R, (Hq+2Hkv) hd]
        del Wqkv
        q_rot = np.empty((len(rows), Hq * hd))
        att = np.empty((len(rows), Hq * hd))
        partials = {}
        for r, b in enumerate(rows):
            pos = int(positions[b])
            q = qkv[r, : Hq * hd].reshape(Hq, hd)
            k = qkv[r, Hq * hd:(Hq + Hkv) * hd].reshape(Hkv, hd)
            v = qkv[r, (Hq + Hkv) * hd:].reshape(Hkv, hd)
            qr = rope(q, pos, theta)
            kr = rope(k, pos, theta)
            q_rot[r] = qr.reshape(-1)
            for g in range(Hkv):
                kv.written[(l, 0, b, g, pos)] = round_storage(kr[g], w.kv_dtype)
                kv.written[(l, 1, b, g, pos)] = round_storage(v[g], w.kv_dtype)
            for g in range(Hkv):
                K, V = kv.keys_values(l, b, g, pos + 1)
                for j in range(grp):
                    h = g * grp + j
                    if split or keep:
                        parts = []
                        for c in range(w.chunks(b)):
                            lo, hi = c * w.kv_chunk, min((c + 1) * w.kv_chunk, pos + 1)
                            lo = min(lo, hi)
                            parts.append(chunk_partial(qr[h], K[lo:hi], V[lo:hi]))
                        if keep:
                            for c, p in enumerate(parts):
                                partials[(b, g, c, j)] = p
                    if split:
                        att[r, h * hd:(h + 1) * hd] = combine(parts)
                    else:
                        att[r, h * hd:(h + 1) * hd] = softmax_attention(qr[h], K, V)
        Wo = params.matrix(w.tid_layer(l, 2))
        o_proj = att @ Wo.T
        h_res = x + o_proj
        del Wo
        g_mlp = params.vector(w.tid_layer(l, 3))
        Wgu = params.matrix(w.tid_layer(l, 4))
        hn = np.stack([rmsnorm(h_res[r], g_mlp, eps) for r in range(len(rows))])
        z = hn @ Wgu.T
        del Wgu
        gu = silu(z[:, :I]) * z[:, I:]
        Wd = params.matrix(w.tid_layer(l, 5))
        d_proj = gu @ Wd.T
        x_out = h_res + d_proj
        del Wd
        if keep:
            inter[f"l{l}.xn"] = xn
            inter[f"l{l}.o"] = o_proj
            inter[f"l{l}.hn"] = hn
            inter[f"l{l}.d"] = d_proj
            inter[f"l{l}.qkv_out"] = qkv
            inter[f"l{l}.q_rot"] = q_rot
            inter[f"l{l}.partials"] = partials
            inter[f"l{l}.att"] = att
            inter[f"l{l}.h"] = h_res
            inter[f"l{l}.gu"] = gu
            inter[f"l{l}.x_out"] = x_out
        x = x_out
    g_fin = params.vector(w.tid_final_norm)
    Wlm = params.matrix(w.tid_lm)
    xn = np.stack([rmsnorm(x[r], g_fin, eps) for r in range(len(rows))])
    if keep:
        inter["xn_final"] = xn
    logits = xn @ Wlm.T
    return logits, inter


def greedy_token(logits_row: np.ndarray) -> int:
    """argmax with the lowest index on ties."""
    return int(np.argmax(logits_row))


def top2_margin(logits_row: np.ndarray) -> float:
    s = np.sort(np.asarray(logits_row, dtype=np.float64))
    return float(s[-1] - s[-2])
