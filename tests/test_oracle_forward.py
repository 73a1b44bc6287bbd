"""Pins for the oracle forward: an independent torch textbook forward (causal
and block-causal masks, GQA, LoRA rows), RoPE closed forms and RMSNorm."""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import seeded
from oracle.model import KVCache, OracleModel, Row, apply_rope, forward, rms_norm
from tests.torch_textbook import textbook_logits

SMALL_GQA_F32 = dataclasses.replace(seeded.SMALL_BF16, name="small-f32-gqa", dtype="f32",
                                    n_layers=1, d_model=256, head_dim=64, d_ffn=384, vocab=300)
SMALL_BF16_1L = dataclasses.replace(seeded.SMALL_BF16, name="small-bf16-1l", n_layers=1,
                                    d_model=256, head_dim=64, d_ffn=384, vocab=300, lora_rank=8)


@pytest.mark.parametrize("shape", [seeded.TINY, SMALL_GQA_F32])
def test_causal_forward_matches_textbook(shape):
    w = seeded.gen_weights(shape)
    toks = seeded.prompt(20, shape.vocab)
    m = OracleModel(shape, w)
    cache = KVCache(shape, 32)
    rows = [Row(int(t), p, p + 1) for p, t in enumerate(toks)]
    got = forward(m, cache, rows)
    ref = textbook_logits(shape, w, toks, np.arange(20), np.tril(np.ones((20, 20), bool)))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_block_forward_matches_textbook_dense_mask():
    shape = seeded.TINY
    w = seeded.gen_weights(shape)
    P, B = 9, 8
    toks = list(seeded.prompt(P, shape.vocab)) + [shape.mask_id] * B
    ids = np.array(list(range(P)) + [P] * B)
    allowed = ids[None, :] <= ids[:, None]
    m = OracleModel(shape, w)
    cache = KVCache(shape, 32)
    rows = [Row(int(toks[p]), p, p + 1) for p in range(P)] + [Row(shape.mask_id, p, P + B) for p in range(P, P + B)]
    got = forward(m, cache, rows)
    ref = textbook_logits(shape, w, toks, np.arange(P + B), allowed)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)


def test_bf16_forward_with_lora_matches_textbook():
    shape = SMALL_BF16_1L
    w = seeded.gen_weights(shape)
    P, B = 6, 5
    toks = list(seeded.prompt(P, shape.vocab)) + [shape.mask_id] * B
    ids = np.array(list(range(P)) + [P] * B)
    allowed = ids[None, :] <= ids[:, None]
    lora_rows = np.array([False] * P + [True] * B)
    m = OracleModel(shape, w)
    cache = KVCache(shape, 16)
    rows = [Row(int(toks[p]), p, p + 1) for p in range(P)] + \
        [Row(shape.mask_id, p, P + B, lora=True) for p in range(P, P + B)]
    got = forward(m, cache, rows, lora_enabled=True)
    ref = textbook_logits(shape, w, toks, np.arange(P + B), allowed, lora_rows=lora_rows)
    # torch rounds float64 -> bf16 through float32 (a double rounding); the two
    # can differ by one bf16 ulp at rare points, so compare to a loose bound.
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-3)
    # and the LoRA must matter on the flagged rows only
    cache2 = KVCache(shape, 16)
    off = forward(m, cache2, rows, lora_enabled=False)
    np.testing.assert_array_equal(got[:P], off[:P])
    assert np.abs(got[P:] - off[P:]).max() > 1e-4


def test_rope_position_zero_is_identity():
    v = np.random.default_rng(0).standard_normal((3, 32))
    np.testing.assert_array_equal(apply_rope(v, 0, 10000.0), v)


def test_rope_composes_and_preserves_norm():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((4, 128))
    for p1, p2 in [(3, 5), (100, 923), (32000, 768)]:
        # rotating by p1 then p2 is rotating by p1 + p2 (angles add per pair)
        np.testing.assert_allclose(apply_rope(apply_rope(v, p1, 1e4), p2, 1e4),
                                   apply_rope(v, p1 + p2, 1e4), atol=1e-9)
        np.testing.assert_allclose(np.linalg.norm(apply_rope(v, p1, 1e4), axis=-1),
                                   np.linalg.norm(v, axis=-1), rtol=1e-13)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    s1 = apply_rope(q, 10, 1e4) @ apply_rope(k, 3, 1e4)
    s2 = apply_rope(q, 1010, 1e4) @ apply_rope(k, 1003, 1e4)
    np.testing.assert_allclose(s1, s2, rtol=1e-10)


def test_rope_pair_rotation_closed_form():
    # hd = 2: a single pair rotated by theta = pos
    v = np.array([1.0, 0.0])
    for pos in (1, 2, 7):
        np.testing.assert_allclose(apply_rope(v, pos, 1e4), [np.cos(pos), np.sin(pos)], atol=1e-15)


def test_rms_norm_matches_torch():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 96)) * 3
    g = rng.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-6), ref, rtol=1e-13)


def test_float32_projection_reference_is_the_same_function():
    """The float32-projection mode (used only to measure the float32
    accumulation floor of large shapes) computes the same forward: on the tiny
    model it agrees with the float64 oracle to float32 rounding, and it does
    evaluate the products in float32 (the results are not bit-identical)."""
    import numpy as np
    import seeded
    from oracle.model import KVCache, OracleModel, Row, forward
    shape = seeded.TINY
    w = seeded.gen_weights(shape)
    rows = [Row(int(t), p, p + 1) for p, t in enumerate(seeded.prompt(12, shape.vocab))]
    a = forward(OracleModel(shape, w), KVCache(shape, 16), rows)
    b = forward(OracleModel(shape, w, proj_dtype=np.float32), KVCache(shape, 16), rows)
    err = float(np.abs(a - b).max())
    assert 0.0 < err < 1e-5 * max(1.0, float(np.abs(a).max()))
