"""Pins for the oracle's decode modes: losslessness of self-speculation against
greedy AR, the accept range, KV rollback, the diffusion threshold edge cases,
LoRA on the drafter only, and brute-force sampler rules."""
import json
import os

import numpy as np
import pytest
import scipy.special

import seeded
from oracle import (MODE_AR, MODE_DIFFUSION, MODE_SELFSPEC, OracleModel, OracleSession,
                    accept_length, commit_set, vocab_reduce)
from oracle.model import KVCache, Row, forward

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

_cache = {}


def model(shape):
    if shape.name not in _cache:
        _cache[shape.name] = OracleModel(shape, seeded.gen_weights(shape))
    return _cache[shape.name]


def session(shape, prompt_len=16, max_ctx=96):
    s = OracleSession(model(shape), max_ctx)
    s.prefill(seeded.prompt(prompt_len, shape.vocab))
    return s


# --------------------------------------------------------------------- sampler
def test_vocab_reduce_matches_library_softmax():
    rng = np.random.default_rng(0)
    for _ in range(50):
        l = rng.standard_normal(700) * rng.uniform(0.1, 20)
        tok, conf = vocab_reduce(l)
        assert tok == int(np.argmax(l))                # numpy: first (lowest) index of the max
        assert conf == pytest.approx(scipy.special.softmax(l).max(), rel=1e-12)


def test_vocab_reduce_ties_take_lowest_id():
    l = np.zeros(10)
    l[[3, 7]] = 5.0
    assert vocab_reduce(l)[0] == 3
    assert vocab_reduce(np.full(6, -1.0)) == (0, pytest.approx(1 / 6))


def test_accept_length_against_cumulative_match():
    rng = np.random.default_rng(1)
    for _ in range(500):
        k = int(rng.integers(1, 12))
        d = rng.integers(0, 3, k)
        g = np.concatenate([np.where(rng.random(k) < 0.6, d, rng.integers(0, 3, k)), [9]])
        a_ref = int(np.cumprod(d == g[:k]).sum())     # number of leading matches
        a = accept_length(list(d), list(g))
        assert a == a_ref and 0 <= a <= k
    assert accept_length([1, 2, 3], [1, 2, 3, 4]) == 3
    assert accept_length([1, 2, 3], [0, 2, 3, 4]) == 0


def test_commit_set_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(500):
        n = int(rng.integers(1, 9))
        conf = rng.choice([0.1, 0.3, 0.5, 0.9], n)
        el = rng.random(n) < 0.7
        tau = float(rng.choice([0.0, 0.4, 0.5, 0.9, 0.95, 1.0]))  # 0.5, 0.9 equal some confs: strict ">"
        got = commit_set(conf, el, tau)
        passing = [i for i in range(n) if el[i] and conf[i] > tau]
        if not el.any():
            assert got == []
        elif passing:
            assert got == passing
        else:
            cand = [i for i in range(n) if el[i]]
            best = max(conf[i] for i in cand)
            assert got == [min(i for i in cand if conf[i] == best)]


# --------------------------------------------------------------------- modes
@pytest.mark.parametrize("shape", [seeded.TINY, seeded.TINY_SHARP])
def test_selfspec_is_lossless_against_greedy_ar(shape):
    ar = session(shape).generate(MODE_AR, 32)
    s = session(shape)
    ss = s.generate(MODE_SELFSPEC, 32, block=8)
    assert ss == ar
    # accept range: 0 <= a <= k every round, a+1 tokens per round
    assert all(0 <= a <= 8 for a in s.accepts)
    assert sum(a + 1 for a in s.accepts) >= 32
    assert s.forwards == 2 * len(s.accepts)


def test_selfspec_with_lora_is_lossless_and_lora_zero_changes_nothing():
    shape = seeded.TINY_LORA
    ar = session(shape).generate(MODE_AR, 32)
    s = session(shape)
    assert s.generate(MODE_SELFSPEC, 32, block=8, lora=True) == ar
    # B = 0 adapter: drafts identical to the drafts without the adapter
    w = dict(model(shape).w)
    for l in range(shape.n_layers):
        w[f"lora.{l}.b"] = np.zeros_like(w[f"lora.{l}.b"])
    m0 = OracleModel(shape, w)
    s1 = OracleSession(m0, 96)
    s1.prefill(seeded.prompt(16, shape.vocab))
    s2 = OracleSession(m0, 96)
    s2.prefill(seeded.prompt(16, shape.vocab))
    assert s1.draft(8, lora=True) == s2.draft(8, lora=False)
    # a non-zero adapter does change some draft logits (it is really applied)
    s3 = session(shape)
    s4 = session(shape)
    s3.keep_logits = s4.keep_logits = True
    s3.draft(8, lora=True)
    s4.draft(8, lora=False)
    assert np.abs(s3.records[-1].logits[1:] - s4.records[-1].logits[1:]).max() > 1e-6
    np.testing.assert_array_equal(s3.records[-1].logits[0], s4.records[-1].logits[0])


@pytest.mark.parametrize("mode", [MODE_SELFSPEC, MODE_DIFFUSION])
def test_cache_after_mode_equals_ar_prefill_cache(mode):
    shape = seeded.TINY_SHARP
    s = session(shape)
    s.generate(mode, 24, block=8, threshold=0.5)
    # an AR prefill of exactly the committed tokens builds the same cache
    ref = OracleSession(model(shape), 96)
    ref.prefill(s.tokens[: s.kv_len + 1])
    assert ref.kv_len == s.kv_len
    np.testing.assert_array_equal(s.cache.k[:, : s.kv_len], ref.cache.k[:, : s.kv_len])
    np.testing.assert_array_equal(s.cache.v[:, : s.kv_len], ref.cache.v[:, : s.kv_len])


def test_diffusion_threshold_zero_commits_block_at_once_equal_to_drafts():
    shape = seeded.TINY
    s = session(shape)
    f0 = s.forwards
    y = s.diffusion_block(8, 0.0)
    assert s.forwards - f0 == 1
    d = session(shape)
    _, drafts = d.draft(8)
    assert y == drafts


def test_diffusion_threshold_one_commits_one_per_forward_in_confidence_order():
    shape = seeded.TINY_SHARP
    s = session(shape)
    s.keep_logits = True
    f0 = s.forwards
    L = s.L
    y = s.diffusion_block(8, 1.0)
    assert s.forwards - f0 == 8
    # replay: each forward committed exactly the most confident remaining position
    done = set()
    for rec in s.records[-8:]:
        block = rec.logits[-8:]
        confs = {i: vocab_reduce(block[i])[1] for i in range(8) if i not in done}
        best = max(confs.values())
        i = min(i for i, c in confs.items() if c == best)
        assert y[i] == vocab_reduce(block[i])[0]
        done.add(i)
    assert len(done) == 8 and s.L == L + 8


def test_diffusion_block_one_commits_one_token_per_forward():
    shape = seeded.TINY
    s = session(shape)
    out = s.generate(MODE_DIFFUSION, 5, block=1, threshold=0.9)
    assert len(out) == 5 and s.forwards == 5


def test_diffusion_sharp_threshold_fires_and_counts():
    shape = seeded.TINY_SHARP
    s = session(shape)
    out = s.generate(MODE_DIFFUSION, 32, block=8, threshold=0.9)
    assert len(out) == 32
    assert 4 <= s.forwards <= 32
    assert all(t < shape.vocab for t in out)        # a [MASK] is never committed (R1)


def test_ar_step_row_is_causal_and_invariant_to_batching():
    # a row's logits do not depend on which other rows share its forward
    shape = seeded.TINY
    m = model(shape)
    toks = seeded.prompt(10, shape.vocab)
    c1 = KVCache(shape, 16)
    full = forward(m, c1, [Row(int(t), p, p + 1) for p, t in enumerate(toks)])
    c2 = KVCache(shape, 16)
    forward(m, c2, [Row(int(t), p, p + 1) for p, t in enumerate(toks[:9])])
    last = forward(m, c2, [Row(int(toks[9]), 9, 10)])
    np.testing.assert_array_equal(full[9], last[0])


def test_tpf_definition_matches_published_ratio():
    """TPF counts the draft and the verify forward separately (golden fixture)."""
    with open(os.path.join(GOLDEN, "tpf_definition.json")) as f:
        g = json.load(f)
    # the SOL-vs-linear-self-speculation TPF ratio is the published "+76.5%"
    assert g["sol_tpf"] / g["linear_selfspec_tpf"] == pytest.approx(1 + g["gain_percent"] / 100, abs=1e-3)
    # with two forwards per round, tokens per round is twice TPF
    shape = seeded.TINY_SHARP
    s = session(shape)
    out = s.generate(MODE_SELFSPEC, 32, block=8)
    tpf = len(out) / s.forwards
    tpr = len(out) / len(s.accepts)
    assert tpr == pytest.approx(g["forwards_per_round"] * tpf)


# ------------------------------------------------ scheduled commit counts
def test_scheduled_diffusion_reduces_to_the_threshold_edge_cases():
    shape = seeded.TINY_SHARP
    for stream in range(3):
        p = seeded.prompt(14, shape.vocab, stream=stream)
        a, b = OracleSession(model(shape), 96), OracleSession(model(shape), 96)
        a.prefill(p)
        b.prefill(p)
        assert a.diffusion_block_scheduled(8, [1]) == b.diffusion_block(8, 1.0)   # one per forward
        assert a.forwards == b.forwards == 8 and a.tokens == b.tokens
        c, d = OracleSession(model(shape), 96), OracleSession(model(shape), 96)
        c.prefill(p)
        d.prefill(p)
        assert c.diffusion_block_scheduled(8, [8]) == d.diffusion_block(8, 0.0)   # the whole block at once
        assert c.forwards == d.forwards == 1


def test_scheduled_diffusion_commits_the_most_confident_counts():
    shape = seeded.TINY_SHARP
    rng = np.random.default_rng(4)
    for trial in range(4):
        counts = [int(c) for c in rng.integers(1, 5, size=int(rng.integers(1, 4)))]
        s = session(shape, prompt_len=12)
        s.keep_logits = True
        n0 = len(s.records)
        L = s.L
        y = s.diffusion_block_scheduled(10, counts)
        recs = s.records[n0:]
        done = set()
        for t, rec in enumerate(recs):
            block = rec.logits[-10:]
            masked = [i for i in range(10) if i not in done]
            confs = sorted(masked, key=lambda i: (-vocab_reduce(block[i])[1], i))
            now = confs[: counts[t % len(counts)]]
            for i in now:
                assert y[i] == vocab_reduce(block[i])[0]
                assert rec.rows[-10 + i].token == shape.mask_id
            done.update(now)
        assert len(done) == 10 and s.L == L + 10
        # forwards: the fewest t with sum of the cycled counts >= 10
        need, t = 10, 0
        while need > 0:
            need -= counts[t % len(counts)]
            t += 1
        assert len(recs) == t


def test_scheduled_diffusion_rejects_bad_counts():
    s = session(seeded.TINY)
    for bad in ([], [0], [2, -1]):
        with pytest.raises(ValueError):
            s.diffusion_block_scheduled(8, bad)
