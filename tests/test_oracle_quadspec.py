"""Pins for the oracle's quadratic self-speculation (reading R24: one forward
per round verifies the carried drafts and drafts the next block for every
possible accept length).  The pages name the mode and its tokens per forward
([Notes §8.1]; [Blog], performance highlights) but do not describe it, so the
layout is parity unpinned by the pages; these tests pin the oracle to its
definition and to what holds whatever the layout: losslessness against greedy
AR at temperature 0 ([Blog], LinearSpec paragraph), 1..k+1 tokens per round,
the cache after the round equal to the AR cache, and every row's logits equal
to an independent dense-mask forward of the whole round."""
import numpy as np
import pytest

import seeded
from oracle import MODE_AR, MODE_QUADSPEC, OracleModel, OracleSession, vocab_reduce
from tests.torch_textbook import textbook_logits

_cache = {}


def model(shape):
    if shape.name not in _cache:
        _cache[shape.name] = OracleModel(shape, seeded.gen_weights(shape))
    return _cache[shape.name]


def session(shape, prompt_len=16, max_ctx=400):
    s = OracleSession(model(shape), max_ctx)
    s.prefill(seeded.prompt(prompt_len, shape.vocab))
    return s


@pytest.mark.parametrize("k", [1, 4, 8])
@pytest.mark.parametrize("shape", [seeded.TINY, seeded.TINY_SHARP])
def test_quadspec_is_lossless_against_greedy_ar(shape, k):
    q = session(shape)
    got = q.generate(MODE_QUADSPEC, 30, block=k)
    ar = session(shape)
    assert got == ar.generate(MODE_AR, 30)
    # one forward per round, 1..k+1 tokens per round
    assert q.forwards == q.rounds == len(q.accepts)
    assert all(0 <= a <= k for a in q.accepts)
    assert sum(a + 1 for a in q.accepts) >= 30


def test_quadspec_with_lora_is_lossless():
    shape = seeded.TINY_LORA
    q = session(shape)
    got = q.generate(MODE_QUADSPEC, 24, block=8, lora=True)
    assert got == session(shape).generate(MODE_AR, 24)


@pytest.mark.parametrize("a_star", [0, 3, 8])
def test_quadspec_controlled_drafts_accept_exactly_and_roll_back(a_star):
    """Carried drafts replaced by the greedy AR continuation up to a forced
    mismatch at a*: the round accepts exactly a*, commits a*+1 tokens of the
    AR continuation, keeps the K/V of the accepted rows (the cache equals an AR
    prefill of the committed tokens) and carries block a*'s drafts."""
    shape, k = seeded.TINY_SHARP, 8
    ref = session(shape).generate(MODE_AR, 40)
    q = session(shape)
    q.keep_logits = True
    first = q.quad_round(k)                      # no drafts yet: the pending row + block 0
    assert first == ref[:1] and q.accepts == [0] and len(q.qdrafts) == k
    L0 = q.L
    d = list(ref[1:1 + k])
    if a_star < k:
        d[a_star] = (d[a_star] + 1) % shape.vocab
    q.qdrafts = d
    got = q.quad_round(k)
    assert q.accepts[-1] == a_star
    assert got == ref[1:1 + a_star + 1]
    assert q.kv_len == L0 + a_star and q.L == L0 + a_star + 1
    # the carried drafts are block a*'s greedy tokens at L0+a*+1 .. L0+a*+k
    blocks = q.records[-1].logits[1 + k:]        # one pending row, k draft rows, then the blocks
    blk = blocks[a_star * (k + 1):(a_star + 1) * (k + 1)]
    assert q.qdrafts == [vocab_reduce(blk[1 + i])[0] for i in range(k)]
    ar = OracleSession(model(shape), 400)
    ar.prefill(q.tokens[: q.kv_len + 1])
    np.testing.assert_array_equal(q.cache.k[:, : q.kv_len], ar.cache.k[:, : q.kv_len])
    np.testing.assert_array_equal(q.cache.v[:, : q.kv_len], ar.cache.v[:, : q.kv_len])
    # and generation continues losslessly from there
    assert q.generate(MODE_QUADSPEC, 12, block=k) == ref[2 + a_star:14 + a_star]


@pytest.mark.parametrize("shape,lora", [(seeded.TINY, False), (seeded.TINY_LORA, True)])
def test_quadspec_round_matches_dense_mask_textbook(shape, lora):
    """Every logit of one quadratic round equals an independent torch forward
    of a single sequence holding the prompt, the pending and draft rows and all
    k+1 blocks, attending by the dense mask written out from the layout: the
    clean stream is causal; block b's rows see the clean positions < L+b and
    the rows of block b, nothing else."""
    k = 4
    s = session(shape, prompt_len=12)
    s.quad_round(k, lora=lora)                   # now there are carried drafts
    s.keep_logits = True
    toks_prefix = s.tokens[: s.kv_len]
    clean, blocks = s.quad_rows(k)
    s.quad_forward(clean, blocks, lora=lora)
    got = s.records[-1].logits
    rows = [(t, p, 0, -1) for p, t in enumerate(toks_prefix)]
    rows += [(r.token, r.pos, 0, -1) for r in clean]
    for b, blk in enumerate(blocks):
        rows += [(r.token, r.pos, 1, b) for r in blk]
    n = len(rows)
    L = s.L
    allowed = np.zeros((n, n), bool)
    for i, (_, pi, bi, gi) in enumerate(rows):
        for j, (_, pj, bj, gj) in enumerate(rows):
            if bi == 0:
                allowed[i, j] = bj == 0 and pj <= pi
            else:
                allowed[i, j] = (bj == 0 and pj < L + gi) or (bj == 1 and gj == gi)
    lora_rows = np.array([b == 1 for _, _, b, _ in rows]) if lora else None
    ref = textbook_logits(shape, seeded.gen_weights(shape), [t for t, _, _, _ in rows],
                          [p for _, p, _, _ in rows], allowed, lora_rows=lora_rows)
    np.testing.assert_allclose(got, ref[len(toks_prefix):], rtol=0, atol=1e-9)


def test_quadspec_drafts_are_dropped_by_other_modes():
    shape = seeded.TINY_SHARP
    s = session(shape)
    s.quad_round(4)
    assert s.qdrafts is not None
    s.ar_step()
    assert s.qdrafts is None
    s.quad_round(4)
    s.kv_rollback(1)
    assert s.qdrafts is None
    with pytest.raises(ValueError):
        s.quad_round(64)


@pytest.mark.parametrize("a_star", [0, 2, 5])
def test_quadspec_carries_block_a_drafts_scripted(a_star):
    """Scripted logits (random-init models give every [MASK] row the same
    argmax, so they cannot tell rows apart): clean row i's greedy token is the
    i-th token of a script, block b's row at position L+b+j votes for token
    9b + j + 100.  After accepting a*, the carried drafts must be block a*'s
    votes for positions L+a*+1 .. L+a*+k, in order."""
    shape, k = seeded.TINY, 5
    s = session(shape)
    V = shape.vocab
    script = [7, 8, 9, 10, 11, 12, 13]
    s.qdrafts = [script[i] if i < a_star else 1 for i in range(k)]   # d_i = g_i for i < a*, mismatch at a*

    def fake_forward(clean, blocks, lora=False):
        L = s.L
        lg = np.zeros((len(clean), V))
        c = L - s.kv_len
        for i in range(len(clean)):
            lg[i, script[max(0, i - (c - 1))]] = 1.0
        blk = []
        for b, rows in enumerate(blocks):
            x = np.zeros((len(rows), V))
            for r_i, r in enumerate(rows):
                j = r.pos - (L + b)
                assert r.hi == L + b + k + 1 and 0 <= j <= k
                x[r_i, 100 + 9 * b + j] = 1.0
            blk.append(x)
        s.forwards += 1
        return lg, blk

    s.quad_forward = fake_forward
    L0 = s.L
    got = s.quad_round(k)
    assert got == script[: a_star + 1] and s.accepts[-1] == a_star
    assert s.qdrafts == [100 + 9 * a_star + 1 + i for i in range(k)]
    assert s.L == L0 + a_star + 1 and s.kv_len == L0 + a_star
