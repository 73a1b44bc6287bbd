"""Oracle model forward (test infrastructure only).

A plain pre-norm decoder, computed row by row in float64:

    x = E[token]
    per layer:  y = RMSNorm(x); q, k, v = y Wq^T, y Wk^T, y Wv^T; RoPE(q, k; pos)
                cache[pos] = (k, v)
                o = softmax(q K[0:hi]^T / sqrt(hd)) V[0:hi]      (GQA: head h uses kv head h // (hq/hkv))
                x += o Wo^T (+ B (A o) on LoRA rows)
                y = RMSNorm(x); x += W_down (silu(W_gate y) * (W_up y))
    logits = RMSNorm(x) W_lm^T   (the V real tokens only)

The one mask is per row: a row attends to the keys [0, hi).  A clean row at
position p has hi = p + 1 (causal, the AR pathway); a row of a noisy block
[L, L + B) has hi = L + B (bidirectional inside the block, causal over the
clean prefix).  This is the block-wise attention of [Notes §3.2] and
[Digest, Method]: bidirectional within a block, causal across blocks, prefix
KV cache reused; the clean stream is strictly causal [Notes §4.3], so the
cache of committed tokens is exactly the AR cache (reading R3).

The architecture itself is not on the pages (reading R11): rotate-half RoPE
with base 10000, RMSNorm eps 1e-6 with unit gains, SwiGLU FFN, untied lm_head,
no biases.  bf16 models round at the storage points of reading R12.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

from .numerics import round_bf16


@dataclasses.dataclass
class Row:
    """One query row of a forward: token id, absolute position, exclusive key
    limit ``hi`` and whether the draft-only LoRA applies to it."""
    token: int
    pos: int
    hi: int
    lora: bool = False


class OracleModel:
    """Weights in float64 plus the shape; ``batched_linear`` trades exact
    row independence of the projections for speed on large models.

    ``proj_dtype=np.float32`` evaluates the projections (the matrix products)
    in float32 instead of float64, everything else unchanged.  It is not the
    oracle of any parity claim: it measures how far the float64 result moves
    when the products are accumulated at float32 precision, the floor any
    float32-accumulating implementation sits on."""

    def __init__(self, shape, weights: Dict[str, np.ndarray], batched_linear: bool = False,
                 keep_float32: bool = False, proj_dtype=np.float64):
        self.shape = shape
        self.bf16 = shape.dtype == "bf16"
        self.batched_linear = batched_linear
        self.proj_dtype = np.dtype(proj_dtype)
        conv = (lambda a: np.asarray(a, dtype=np.float32)) if keep_float32 else \
            (lambda a: np.asarray(a, dtype=np.float64))
        self.w = {k: conv(v) for k, v in weights.items()}
        self.has_lora = shape.lora_rank > 0 and "lora.0.a" in self.w

    def store(self, a: np.ndarray) -> np.ndarray:
        """A storage point: bf16 models keep the value as bfloat16 (reading R12)."""
        return round_bf16(a) if self.bf16 else a


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row: x / sqrt(mean(x^2) + eps) * g (reading R11)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def linear(x: np.ndarray, w: np.ndarray, batched: bool, dtype=np.float64) -> np.ndarray:
    """y = x W^T for each row of x, computed in ``dtype`` (float64 unless the
    model asks for the float32 sensitivity reference) and returned in float64.

    By default each row is its own matrix-vector product, so a row's result
    never depends on which other rows share the forward (this is what makes
    oracle self-speculation bit-identical to oracle AR).
    """
    w = np.asarray(w, dtype=dtype)
    x = np.asarray(x, dtype=dtype)
    if batched:
        y = x @ w.T
    else:
        y = np.stack([w @ xi for xi in x]) if len(x) else np.zeros((0, w.shape[0]), dtype=dtype)
    return np.asarray(y, dtype=np.float64)


def rope_angles(pos: int, head_dim: int, base: float) -> np.ndarray:
    """theta_i = pos * base^(-2i/hd), i < hd/2 (reading R11)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return pos * np.power(float(base), -2.0 * i / head_dim)


def apply_rope(v: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate-half RoPE of ``v`` [..., hd]: pairs (i, i + hd/2) rotate by theta_i."""
    hd = v.shape[-1]
    th = rope_angles(pos, hd, base)
    c, s = np.cos(th), np.sin(th)
    a, b = v[..., : hd // 2], v[..., hd // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


class KVCache:
    """Per-layer K and V of shape [max_ctx, hkv, hd] (float64 values)."""

    def __init__(self, shape, max_ctx: int):
        L, hkv, hd = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.max_ctx = max_ctx
        self.k = np.zeros((L, max_ctx, hkv, hd))
        self.v = np.zeros((L, max_ctx, hkv, hd))

    def copy(self) -> "KVCache":
        c = KVCache.__new__(KVCache)
        c.max_ctx, c.k, c.v = self.max_ctx, self.k.copy(), self.v.copy()
        return c


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, hi: int, group: int) -> np.ndarray:
    """Attention of one row: q [hq, hd] over keys [0, hi) of K, V [ctx, hkv, hd].

    Query head h reads kv head h // group.  Softmax with scale 1/sqrt(hd).
    """
    hq, hd = q.shape
    out = np.empty((hq, hd))
    for h in range(hq):
        kh = K[:hi, h // group, :]
        vh = V[:hi, h // group, :]
        s = kh @ q[h] / np.sqrt(hd)
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ vh
    return out


def forward(model: OracleModel, cache: KVCache, rows: List[Row],
            lora_enabled: bool = False, return_hidden: bool = False):
    """One forward over ``rows``; writes every row's K/V into ``cache`` at its
    position and returns float64 logits [len(rows), V].

    All rows' K/V of a layer are written before any row of that layer attends,
    so block rows see each other (bidirectional inside the block) while clean
    rows, limited to hi = pos + 1, never see anything after themselves.
    LoRA (reading R10) applies only to rows flagged ``lora`` and only when
    ``lora_enabled``: the drafter pathway, never the verifier [Notes §6].
    """
    sh, w, st = model.shape, model.w, model.store
    n = len(rows)
    if n == 0:
        return np.zeros((0, sh.vocab))
    for r in rows:
        if not (0 <= r.pos < cache.max_ctx and r.pos < r.hi <= cache.max_ctx):
            raise ValueError(f"bad row {r}")
        if not (0 <= r.token <= sh.vocab):
            raise ValueError(f"bad token {r.token}")
    hq, hkv, hd = sh.n_q_heads, sh.n_kv_heads, sh.head_dim
    group = hq // hkv
    bl = model.batched_linear
    pd = model.proj_dtype
    x = np.stack([np.asarray(w["embed"][r.token], dtype=np.float64) for r in rows])
    use_lora = lora_enabled and model.has_lora
    for l in range(sh.n_layers):
        p = f"layers.{l}."
        y = st(rms_norm(x, w[p + "attn_norm"], sh.rms_eps))
        q = linear(y, w[p + "wq"], bl, pd).reshape(n, hq, hd)
        k = linear(y, w[p + "wk"], bl, pd).reshape(n, hkv, hd)
        v = linear(y, w[p + "wv"], bl, pd).reshape(n, hkv, hd)
        for i, r in enumerate(rows):
            q[i] = apply_rope(q[i], r.pos, sh.rope_base)
            k[i] = apply_rope(k[i], r.pos, sh.rope_base)
        q, k, v = st(q), st(k), st(v)
        for i, r in enumerate(rows):
            cache.k[l, r.pos] = k[i]
            cache.v[l, r.pos] = v[i]
        o = np.stack([attend(q[i], cache.k[l], cache.v[l], r.hi, group).reshape(-1)
                      for i, r in enumerate(rows)])
        o = st(o)
        delta = linear(o, w[p + "wo"], bl, pd)
        if use_lora:
            mask = np.array([r.lora for r in rows])
            if mask.any():
                mid = st(linear(o[mask], w[f"lora.{l}.a"], bl, pd))
                delta[mask] = delta[mask] + linear(mid, w[f"lora.{l}.b"], bl, pd)
        x = x + delta
        y = st(rms_norm(x, w[p + "ffn_norm"], sh.rms_eps))
        h = st(silu(linear(y, w[p + "w_gate"], bl, pd)) * linear(y, w[p + "w_up"], bl, pd))
        x = x + linear(h, w[p + "w_down"], bl, pd)
    yf = st(rms_norm(x, w["final_norm"], sh.rms_eps))
    logits = linear(yf, w["lm_head"], bl, pd)
    if return_hidden:
        return logits, x
    return logits
