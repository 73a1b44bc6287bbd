"""Helpers of the GPU parity tests: seeded device weights, and the replay of a
GPU forward trace through the oracle (teacher forcing)."""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

import seeded
from oracle.model import KVCache, OracleModel, Row, forward


def device_weights(shape: seeded.ModelShape, arrays: Dict[str, np.ndarray], device="cuda"):
    import torch
    wdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    out = {}
    for name, a in arrays.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        t = t.to(torch.float32) if name.endswith("norm") else t.to(wdt)
        out[name] = t.to(device)
    return out


def make_model(shape: seeded.ModelShape, tensors):
    import self_speculative_lm_amd as tm
    return tm.Model(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                    shape.vocab, tensors, dtype=tm.TRI_BF16 if shape.dtype == "bf16" else tm.TRI_F32,
                    rope_base=shape.rope_base, rms_eps=shape.rms_eps, lora_rank=shape.lora_rank)


def replay(shape: seeded.ModelShape, oracle_model: OracleModel, trace: List[dict], max_ctx: int,
           prompts: Optional[List[List[int]]] = None):
    """Run every traced forward through the oracle with the GPU's rows (its
    tokens, positions, limits and LoRA flags): returns per forward the oracle
    logits (or None when the GPU forward had no lm_head).  With `prompts`, the
    oracle cache of sequence i first holds the causal prefill of prompts[i]
    (all but its last token, in one forward), as a GPU prefill leaves it."""
    caches: Dict[int, KVCache] = {}
    for i, p in enumerate(prompts or []):
        cache = caches.setdefault(i, KVCache(shape, max_ctx))
        if len(p) > 1:
            forward(oracle_model, cache, [Row(int(t), q, q + 1) for q, t in enumerate(p[:-1])])
    out = []
    for rec in trace:
        seqs = rec["seq"]
        logits = []
        for sq in sorted(set(seqs.tolist()), key=lambda s: int(np.flatnonzero(seqs == s)[0])):
            idx = np.flatnonzero(seqs == sq)
            cache = caches.setdefault(int(sq), KVCache(shape, max_ctx))
            rows = [Row(int(rec["tok"][i]), int(rec["pos"][i]), int(rec["hi"][i]), bool(rec["lora"][i])) for i in idx]
            logits.append(forward(oracle_model, cache, rows, lora_enabled=True))
        out.append(np.concatenate(logits) if rec["logits"] is not None else None)
    return out


def top2_margin(row: np.ndarray) -> float:
    s = np.sort(row)
    return float(s[-1] - s[-2])
