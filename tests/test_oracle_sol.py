"""Pins for the oracle's speed-of-light (SOL) analysis (reading R20 of the
SOL section of the technical notes): closed forms on scripted predictors
(a dependency forest needs 1 + its height in forwards; a planted fallback),
every decision of a real model's passes replayed through the independent
textbook forward, and the serial pass against the diffusion block at
threshold 1."""
import numpy as np
import pytest

import seeded
from oracle import OracleModel, OracleSession, vocab_reduce
from oracle.sol import fork, serial_denoise, sol_block, sol_pass
from tests.torch_textbook import textbook_logits

_cache = {}


def model(shape):
    if shape.name not in _cache:
        _cache[shape.name] = OracleModel(shape, seeded.gen_weights(shape))
    return _cache[shape.name]


def session(shape, prompt_len=12, max_ctx=96, stream=0):
    s = OracleSession(model(shape), max_ctx)
    s.prefill(seeded.prompt(prompt_len, shape.vocab, stream=stream))
    return s


# ------------------------------------------------------- scripted predictors
class _Shape:
    def __init__(self, vocab):
        self.vocab = vocab
        self.mask_id = vocab


class _Model:
    def __init__(self, vocab):
        self.shape = _Shape(vocab)


class ScriptedSession:
    """Stands in for a session: the block rows' logits come from
    ``pred(i, committed) -> (token, logit)``, where ``committed`` maps the
    already committed block positions to their tokens."""

    def __init__(self, vocab, pred, L=5):
        self.model = _Model(vocab)
        self.pred = pred
        self.tokens = list(range(L))
        self.kv_len = L - 1
        self.forwards = 0
        self.rounds = 0
        self.accepts = []
        self.records = []
        self.cache = self

    def copy(self):          # the cache protocol used by fork()
        return self

    @property
    def L(self):
        return len(self.tokens)

    def clean_rows(self):
        return [None] * (self.L - self.kv_len)

    def kv_append(self, n):
        self.kv_len += n

    def run(self, rows):
        self.forwards += 1
        V, mask = self.model.shape.vocab, self.model.shape.mask_id
        block = [r for r in rows if r is not None]
        committed = {r.pos - self.L: r.token for r in block if r.token != mask}
        out = np.zeros((len(rows), V))
        for j, r in enumerate(rows):
            if r is None or r.token != mask:
                continue
            tok, logit = self.pred(r.pos - self.L, committed)
            out[j, tok] = logit
        return out


def forest_predictor(parent, target, vocab):
    """Position i predicts its target once its parent is committed (roots at
    once); otherwise a wrong token with little confidence."""
    def pred(i, committed):
        if parent[i] < 0 or parent[i] in committed:
            return target[i], 20.0 + i * 0.01          # distinct: no confidence ties
        return (target[i] + 1) % vocab, 1.0
    return pred


def test_dependency_forest_needs_one_plus_height_forwards():
    rng = np.random.default_rng(7)
    for trial in range(60):
        B = int(rng.integers(1, 17))
        perm = rng.permutation(B)                 # dependencies not left to right
        parent = [-1] * B
        for r in range(1, B):
            if rng.random() < 0.8:
                parent[perm[r]] = int(perm[rng.integers(0, r)])
        target = [int(t) for t in rng.integers(0, 50, B)]
        depth = [0] * B
        for r in range(B):
            i = perm[r]
            depth[i] = 0 if parent[i] < 0 else depth[parent[i]] + 1
        s = ScriptedSession(50, forest_predictor(parent, target, 50))
        res = sol_block(s, B)
        assert res["target"] == target
        assert res["sol_forwards"] == 1 + max(depth)
        assert res["step"] == depth                   # each position one forward after its parent
        assert s.forwards == B and s.L == 5 + B       # the session took the serial block
        # the serial order commits a parent before its child
        seen = set()
        for i in res["order"]:
            assert parent[i] < 0 or parent[i] in seen
            seen.add(i)


def test_planted_fallback_commits_the_next_serial_position():
    # serial: 0 (a), then 1 (b), then 2 (c).  With nothing committed, 2 already
    # predicts c but 1 does not predict b; with {0, 2} committed, 1 predicts a
    # wrong token, so the SOL pass must fall back to the serial order.
    a, b, c, x, z = 3, 4, 5, 6, 7

    def pred(i, C):
        C = set(C)
        if i == 0:
            return a, 30.0
        if i == 1:
            return (b, 20.0) if C == {0} else (z if 2 in C else x, 1.0)
        return (c, 10.0 if C == {0, 1} else 2.0)

    res = sol_block(ScriptedSession(10, pred), 3)
    assert res["target"] == [a, b, c]
    assert res["order"] == [0, 1, 2]
    assert res["step"] == [0, 1, 0]
    assert res["sol_forwards"] == 2


def test_planted_fallback_follows_the_serial_order_not_the_position():
    # serial order 0, 3, 1, 2.  The SOL pass commits {0, 2} first; then neither
    # 1 nor 3 is right, and the fallback must take 3 (next in serial order),
    # after which 1 becomes right.
    a, b, c, d, w, x, yy = 1, 2, 3, 4, 5, 6, 7

    def pred(i, C):
        C = set(C)
        if i == 0:
            return a, 30.0
        if i == 3:
            return (d, 20.0) if C == {0} else (w, 1.0)
        if i == 1:
            return (b, 15.0) if 3 in C else (x, 1.0)
        if C == {0, 1, 3}:
            return c, 10.0
        return (c, 2.0) if not C else (yy, 1.0)

    res = sol_block(ScriptedSession(12, pred), 4)
    assert res["target"] == [a, b, c, d]
    assert res["order"] == [0, 3, 1, 2]
    assert res["step"] == [0, 2, 0, 1]
    assert res["sol_forwards"] == 3


def test_no_position_ever_predicts_early_means_serial_forwards():
    # a chain in serial order: position i is right only once i-1 is committed
    B = 9
    parent = [-1] + list(range(B - 1))
    res = sol_block(ScriptedSession(40, forest_predictor(parent, list(range(B)), 40)), B)
    assert res["sol_forwards"] == B and res["tokens_per_forward"] == 1.0


# --------------------------------------------------------- a real model
def _textbook_block(shape, s0, y):
    """Textbook logits of the block rows for the committed prefix of ``s0`` and
    block tokens ``y`` (prefix causal, block bidirectional over itself)."""
    toks = list(s0.tokens) + list(y)
    P, B = s0.L, len(y)
    ids = np.array(list(range(P)) + [P] * B)
    allowed = ids[None, :] <= ids[:, None]
    return textbook_logits(shape, seeded.gen_weights(shape), toks, np.arange(P + B), allowed)[P:]


@pytest.mark.parametrize("shape,B", [(seeded.TINY_SHARP, 8), (seeded.TINY, 6)])
def test_every_decision_replays_through_the_textbook_forward(shape, B):
    s = session(shape)
    s0 = fork(s)
    res = sol_block(s, B)
    mask = shape.mask_id
    target, order, step = res["target"], res["order"], res["step"]
    # serial pass: each forward commits the most confident masked position
    y = [mask] * B
    for i in order:
        lg = _textbook_block(shape, s0, y)
        conf = {j: vocab_reduce(lg[j])[1] for j in range(B) if y[j] == mask}
        best = max(conf.values())
        assert i == min(j for j, c in conf.items() if c == best)
        assert target[i] == vocab_reduce(lg[i])[0]
        y[i] = target[i]
    assert s.tokens[s0.L:] == target
    # SOL pass: the set of each forward is exactly the positions already right
    y = [mask] * B
    for f in range(res["sol_forwards"]):
        lg = _textbook_block(shape, s0, y)
        right = [j for j in range(B) if y[j] == mask and vocab_reduce(lg[j])[0] == target[j]]
        now = [j for j in range(B) if step[j] == f]
        if right:
            assert now == right
        else:
            assert now == [next(j for j in order if y[j] == mask)]
        for j in now:
            y[j] = target[j]
    assert y == target


def test_serial_pass_is_the_diffusion_block_at_threshold_one():
    shape = seeded.TINY_SHARP
    for stream in range(3):
        a, b = session(shape, stream=stream), session(shape, stream=stream)
        f0 = a.forwards
        target, order = serial_denoise(a, 8)
        assert b.diffusion_block(8, 1.0) == target
        assert a.forwards - f0 == 8 and sorted(order) == list(range(8))
        assert a.tokens == b.tokens and a.kv_len == b.kv_len


def test_invariants_over_a_generation():
    shape = seeded.TINY_SHARP
    s = session(shape, prompt_len=10)
    for _ in range(4):
        res = sol_block(s, 8)
        F = res["sol_forwards"]
        assert 1 <= F <= 8
        assert sorted(set(res["step"])) == list(range(F))      # every forward commits one or more
        assert res["step"][res["order"][0]] == 0                 # the serial first pick is right at once
        assert all(t < shape.vocab for t in res["target"])
    assert s.L == 10 + 32 and s.forwards == 32


def test_sol_pass_leaves_the_fork_with_the_target_prefix_run():
    shape = seeded.TINY
    s = session(shape)
    start = fork(s)
    res = sol_block(s, 6)
    kv0 = start.kv_len
    F, _ = sol_pass(start, 6, res["target"], res["order"])
    assert F == res["sol_forwards"]
    assert start.kv_len == kv0 + 1 and start.L == s.L - 6      # pending row adopted, block not committed
