"""A second, independently written statement of one decode step, in torch float64 on
the CPU (library routines: rms_norm, silu, scaled_dot_product_attention with GQA,
complex-number RoPE).  Used only to pin the numpy oracle."""
import torch
import torch.nn.functional as F


def rope_complex(x: torch.Tensor, pos: int, theta: float) -> torch.Tensor:
    """x[..., hd]: pairs (i, i + hd/2) as complex numbers rotated by pos * theta^(-2i/hd)."""
    hd = x.shape[-1]
    half = hd // 2
    freqs = torch.pow(torch.tensor(theta, dtype=torch.float64), -2.0 * torch.arange(half, dtype=torch.float64) / hd)
    rot = torch.polar(torch.ones(half, dtype=torch.float64), pos * freqs)
    z = torch.complex(x[..., :half], x[..., half:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def to_cache(v: torch.Tensor, kv_dtype: str) -> torch.Tensor:
    v32 = v.to(torch.float32)
    return (v32.to(torch.bfloat16) if kv_dtype == "bf16" else v32).to(torch.float64)


def decode_step(w, P, tokens, positions, cache):
    """P: dict name -> float64 tensor (names of Workload.weight_specs);
    cache: dict (layer, 'k'|'v', b) -> float64 tensor [kv_heads, slots, hd], updated in place."""
    H, hd, Hq, Hkv, I = w.hidden, w.head_dim, w.n_q_heads, w.n_kv_heads, w.intermediate
    x = torch.stack([P["embedding"][int(t)] for t in tokens])
    for l in range(w.n_layers):
        xn = F.rms_norm(x, (H,), P[f"l{l}.attn_norm"], eps=w.rms_eps)
        qkv = F.linear(xn, P[f"l{l}.W_qkv"])
        att = torch.empty(x.shape[0], Hq * hd, dtype=torch.float64)
        for b in range(x.shape[0]):
            pos = int(positions[b])
            q = qkv[b, : Hq * hd].view(Hq, hd)
            k = qkv[b, Hq * hd:(Hq + Hkv) * hd].view(Hkv, hd)
            v = qkv[b, (Hq + Hkv) * hd:].view(Hkv, hd)
            q, k = rope_complex(q, pos, w.rope_theta), rope_complex(k, pos, w.rope_theta)
            cache[(l, "k", b)][:, pos] = to_cache(k, w.kv_dtype)
            cache[(l, "v", b)][:, pos] = to_cache(v, w.kv_dtype)
            K = cache[(l, "k", b)][:, : pos + 1]
            V = cache[(l, "v", b)][:, : pos + 1]
            o = F.scaled_dot_product_attention(q[None, :, None, :], K[None], V[None], enable_gqa=True)
            att[b] = o[0, :, 0, :].reshape(-1)
        h = x + F.linear(att, P[f"l{l}.W_o"])
        gu = F.linear(F.rms_norm(h, (H,), P[f"l{l}.mlp_norm"], eps=w.rms_eps), P[f"l{l}.W_gate_up"])
        x = h + F.linear(F.silu(gu[:, :I]) * gu[:, I:], P[f"l{l}.W_down"])
    return F.linear(F.rms_norm(x, (H,), P["final_norm"], eps=w.rms_eps), P["W_lm"])
