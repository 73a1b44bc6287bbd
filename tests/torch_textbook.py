"""An independent textbook decoder forward in torch (CPU, float64), used only
to pin the oracle: library RMSNorm, complex-number RoPE, SDPA with an explicit
mask and grouped KV heads, and SiLU.  Shares nothing with the oracle."""
import numpy as np
import torch
import torch.nn.functional as F


def _bf16(t):
    # torch's own float -> bfloat16 conversion (via float32)
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _rope_complex(x, pos, base):
    """x [n, h, hd]; pairs (i, i + hd/2) taken as the complex number
    x_i + 1j * x_{i+hd/2}, multiplied by exp(1j * pos * base^(-2i/hd))."""
    hd = x.shape[-1]
    inv = torch.pow(torch.tensor(float(base), dtype=torch.float64),
                    -torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    ang = pos[:, None].to(torch.float64) * inv[None, :]           # [n, hd/2]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]      # [n, 1, hd/2]
    z = torch.complex(x[..., : hd // 2], x[..., hd // 2:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def textbook_logits(shape, weights, tokens, positions, allowed, lora_rows=None):
    """Logits of every row of one sequence whose rows attend by the dense
    boolean mask ``allowed`` [n, n] (rows are also the keys)."""
    bf = shape.dtype == "bf16"
    st = _bf16 if bf else (lambda t: t)
    W = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in weights.items()}
    tok = torch.as_tensor(np.asarray(tokens), dtype=torch.long)
    pos = torch.as_tensor(np.asarray(positions), dtype=torch.long)
    n = len(tokens)
    hq, hkv, hd, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_model
    mask = torch.as_tensor(np.asarray(allowed), dtype=torch.bool)
    x = W["embed"][tok]
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        y = st(F.rms_norm(x, (d,), W[p + "attn_norm"], eps=shape.rms_eps))
        q = F.linear(y, W[p + "wq"]).view(n, hq, hd)
        k = F.linear(y, W[p + "wk"]).view(n, hkv, hd)
        v = F.linear(y, W[p + "wv"]).view(n, hkv, hd)
        q, k, v = st(_rope_complex(q, pos, shape.rope_base)), st(_rope_complex(k, pos, shape.rope_base)), st(v)
        o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                           v.transpose(0, 1)[None], attn_mask=mask,
                                           enable_gqa=True)[0].transpose(0, 1).reshape(n, hq * hd)
        o = st(o)
        delta = F.linear(o, W[p + "wo"])
        if lora_rows is not None:
            lr = torch.as_tensor(np.asarray(lora_rows), dtype=torch.bool)
            mid = st(F.linear(o, W[f"lora.{l}.a"]))
            delta = delta + torch.where(lr[:, None], F.linear(mid, W[f"lora.{l}.b"]),
                                        torch.zeros_like(delta))
        x = x + delta
        y = st(F.rms_norm(x, (d,), W[p + "ffn_norm"], eps=shape.rms_eps))
        h = st(F.silu(F.linear(y, W[p + "w_gate"])) * F.linear(y, W[p + "w_up"]))
        x = x + F.linear(h, W[p + "w_down"])
    yf = st(F.rms_norm(x, (d,), W["final_norm"], eps=shape.rms_eps))
    return F.linear(yf, W["lm_head"]).numpy()
