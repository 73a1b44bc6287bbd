"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws numbers: model shapes, random-init weights, prompts,
attention operands and draft/verify token arrays.  It holds none of the
decoding method's arithmetic (no norm, attention, sampling or acceptance
rule), so that both sides of every parity test can take identical inputs from
it while sharing no code with each other.

Random streams: every tensor gets its own ``numpy.random.SeedSequence
([seed, tensor_index, chunk_index])`` driving PCG64, with a fixed chunk size,
so a tensor's values never depend on how many threads generate it.  Default
seeds: weights 0, prompts 1, LoRA 2, attention operands 3.

Weights are drawn N(0, std^2) in float32 and, for bf16 models, rounded to the
nearest bfloat16 (ties to even).  Arrays are returned as float32 holding the
exact bf16 values, so ``torch.from_numpy(w).to(torch.bfloat16)`` is exact and
``w.astype(np.float64)`` is exact.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Iterator, List, Optional, Tuple

import numpy as np

WEIGHT_SEED = 0
PROMPT_SEED = 1
LORA_SEED = 2
ATTN_SEED = 3

_CHUNK = 1 << 22  # elements per independently seeded chunk


@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Decoder shape.  The embedding has ``vocab + 1`` rows; id ``vocab`` is [MASK]."""

    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    dtype: str = "bf16"  # "f32" or "bf16"
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    init_std: float = 0.02
    lora_rank: int = 0
    lora_std: float = 0.01
    lm_head_scale: float = 1.0  # >1 sharpens the softmax (test variant only)

    @property
    def mask_id(self) -> int:
        return self.vocab

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def n_params(self) -> int:
        return sum(int(np.prod(s)) for _, s, _ in weight_specs(self))

    def weight_bytes_per_forward(self) -> int:
        """Bytes of weights a forward streams (every layer, final norm, lm_head)."""
        esz = 2 if self.dtype == "bf16" else 4
        total = 0
        for name, shape, _ in weight_specs(self):
            if name == "embed" or name.startswith("lora."):
                continue
            n = int(np.prod(shape))
            total += n * (4 if name.endswith("norm") else esz)
        return total


# Named shapes.  The 8B/14B shapes are assumed (the write-ups give no
# architecture); the tiny one is the fp32 parity model.
TINY = ModelShape("tiny-f32", 2, 128, 4, 4, 32, 512, 512, dtype="f32")
TINY_SHARP = dataclasses.replace(TINY, name="tiny-f32-sharp", lm_head_scale=40.0)
TINY_LORA = dataclasses.replace(TINY, name="tiny-f32-lora", lora_rank=16)
SMALL_BF16 = ModelShape("small-bf16", 2, 512, 4, 2, 128, 1024, 1000, dtype="bf16")
SMALL_BF16_SHARP = dataclasses.replace(SMALL_BF16, name="small-bf16-sharp", lm_head_scale=40.0)
SMALL_BF16_LORA = dataclasses.replace(SMALL_BF16, name="small-bf16-lora", lora_rank=128)
MODEL_8B = ModelShape("8b-class", 36, 4096, 32, 8, 128, 12288, 151936, dtype="bf16")
MODEL_14B = ModelShape("14b-class", 40, 5120, 40, 8, 128, 17408, 151936, dtype="bf16",
                       lora_rank=128)

SHAPES = {s.name: s for s in (TINY, TINY_SHARP, TINY_LORA, SMALL_BF16, SMALL_BF16_SHARP,
                              SMALL_BF16_LORA, MODEL_8B, MODEL_14B)}


def weight_specs(shape: ModelShape) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Ordered (name, shape, kind) list; kind is "normal", "ones", "lm_head" or "lora".

    This order is also the order of the weight pointer array the C-ABI takes.
    """
    d, f, V = shape.d_model, shape.d_ffn, shape.vocab
    specs: List[Tuple[str, Tuple[int, ...], str]] = [("embed", (V + 1, d), "normal")]
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        specs += [
            (p + "wq", (shape.q_dim, d), "normal"),
            (p + "wk", (shape.kv_dim, d), "normal"),
            (p + "wv", (shape.kv_dim, d), "normal"),
            (p + "wo", (d, shape.q_dim), "normal"),
            (p + "w_gate", (f, d), "normal"),
            (p + "w_up", (f, d), "normal"),
            (p + "w_down", (d, f), "normal"),
            (p + "attn_norm", (d,), "ones"),
            (p + "ffn_norm", (d,), "ones"),
        ]
    specs += [("final_norm", (d,), "ones"), ("lm_head", (V, d), "lm_head")]
    if shape.lora_rank > 0:
        r = shape.lora_rank
        for l in range(shape.n_layers):
            specs += [(f"lora.{l}.a", (r, shape.q_dim), "lora"),
                      (f"lora.{l}.b", (d, r), "lora")]
    return specs


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Input preparation only (weights/operands are drawn as float32 then stored
    as bf16).  Finite inputs only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _fill_normal(seed_words: Tuple[int, ...], n: int, std: float, bf16: bool) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    n_chunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed_words) + [c])))
        v = g.standard_normal(hi - lo, dtype=np.float32)
        v *= np.float32(std)
        out[lo:hi] = bf16_round_f32(v) if bf16 else v

    if n_chunks <= 1:
        work(0)
    else:
        threads = min(n_chunks, max(1, min(16, os.cpu_count() or 1)))
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def gen_weight(shape: ModelShape, index: int, seed: Optional[int] = None) -> Tuple[str, np.ndarray]:
    """Generate weight number ``index`` of ``weight_specs(shape)``."""
    name, shp, kind = weight_specs(shape)[index]
    n = int(np.prod(shp))
    if kind == "ones":
        return name, np.ones(shp, dtype=np.float32)
    bf16 = shape.dtype == "bf16"
    if kind == "lora":
        s = LORA_SEED if seed is None else seed
        arr = _fill_normal((s, index), n, shape.lora_std, bf16)
    else:
        s = WEIGHT_SEED if seed is None else seed
        std = shape.init_std * (shape.lm_head_scale if kind == "lm_head" else 1.0)
        arr = _fill_normal((s, index), n, std, bf16)
    return name, arr.reshape(shp)


def iter_weights(shape: ModelShape, seed: Optional[int] = None) -> Iterator[Tuple[str, np.ndarray]]:
    for i in range(len(weight_specs(shape))):
        yield gen_weight(shape, i, seed)


def gen_weights(shape: ModelShape, seed: Optional[int] = None,
                names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """All weights (or the named subset) as float32 arrays keyed by name."""
    out = {}
    for i, (name, _, _) in enumerate(weight_specs(shape)):
        if names is not None and name not in names:
            continue
        out[name] = gen_weight(shape, i, seed)[1]
    return out


def prompt(n: int, vocab: int, seed: int = PROMPT_SEED, stream: int = 0) -> np.ndarray:
    """``n`` token ids uniform over [0, vocab) (the [MASK] id ``vocab`` excluded)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000 + stream])))
    return g.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def normal(shape: Tuple[int, ...], seed: int, stream: int, std: float = 1.0,
           bf16: bool = False) -> np.ndarray:
    """Seeded N(0, std^2) float32 array (bf16-exact values if ``bf16``)."""
    n = int(np.prod(shape))
    return _fill_normal((seed, 5000 + stream), n, std, bf16).reshape(shape)


def attention_operands(rows: int, prefix: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       batch: int = 1, bf16: bool = True, seed: int = ATTN_SEED):
    """Block-causal attention operands: q [batch, rows, hq, hd] and k, v
    [batch, prefix + rows, hkv, hd], all N(0, 1)."""
    q = normal((batch, rows, n_q_heads, head_dim), seed, 0, 1.0, bf16)
    k = normal((batch, prefix + rows, n_kv_heads, head_dim), seed, 1, 1.0, bf16)
    v = normal((batch, prefix + rows, n_kv_heads, head_dim), seed, 2, 1.0, bf16)
    return q, k, v


def token_pairs(batch: int, k: int, vocab: int, seed: int, match_prob: float = 0.7):
    """Draft tokens d [batch, k] and AR tokens g [batch, k+1] with a random
    matching prefix (each position copies the draft with ``match_prob``)."""
    g_ = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7000])))
    d = g_.integers(0, vocab, size=(batch, k), dtype=np.int64).astype(np.int32)
    ar = g_.integers(0, vocab, size=(batch, k + 1), dtype=np.int64).astype(np.int32)
    copy = g_.random((batch, k)) < match_prob
    ar[:, :k] = np.where(copy, d, ar[:, :k])
    return d, ar


def logits_matrix(rows: int, vocab: int, seed: int, scale: float = 1.0) -> np.ndarray:
    """Seeded float32 logits [rows, vocab] ~ N(0, scale^2)."""
    return normal((rows, vocab), seed, 9000, scale, False)
