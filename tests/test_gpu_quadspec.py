"""GPU parity of quadratic self-speculation (TRI_QUADSPEC, reading R24)
against the oracle: free-running tokens equal the oracle's quadratic rounds
and greedy AR, every traced forward (clean rows plus all hypothesis blocks)
matches the oracle teacher-forced, controlled drafts are accepted exactly,
and the draft LoRA changes drafts only."""
import numpy as np
import pytest

import seeded
from oracle import MODE_AR, MODE_QUADSPEC, OracleModel, OracleSession
from oracle.model import KVCache, Row, forward
from tests.gpu_util import device_weights, make_model

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
_models = {}


def get(shape):
    if shape.name not in _models:
        arrays = seeded.gen_weights(shape)
        tens = device_weights(shape, arrays)
        _models[shape.name] = (arrays, tens, make_model(shape, tens), OracleModel(shape, arrays))
    return _models[shape.name]


def replay_quad(shape, om, trace, max_ctx, prompts, k):
    """Oracle logits of every traced quadratic forward on the GPU's rows:
    [MASK] rows with a common key limit form one hypothesis block (limit
    L+b on the GPU: the clean prefix, plus the block's own keys); the clean
    rows run into the sequence's cache, each block on a copy of it."""
    caches = {}
    for i, p in enumerate(prompts):
        c = caches.setdefault(i, KVCache(shape, max_ctx))
        if len(p) > 1:
            forward(om, c, [Row(int(t), q, q + 1) for q, t in enumerate(p[:-1])])
    out = []
    for rec in trace:
        lg = np.zeros_like(rec["logits"], dtype=np.float64)
        for sq in sorted(set(rec["seq"].tolist())):
            idx = np.flatnonzero(rec["seq"] == sq)
            cache = caches[int(sq)]
            clean = [i for i in idx if rec["tok"][i] != shape.mask_id]
            lg[clean] = forward(om, cache, [Row(int(rec["tok"][i]), int(rec["pos"][i]), int(rec["hi"][i])) for i in clean])
            blk = [i for i in idx if rec["tok"][i] == shape.mask_id]
            for j in range(0, len(blk), k + 1):
                rows = blk[j:j + k + 1]
                hi = int(rec["hi"][rows[0]])
                assert all(int(rec["hi"][i]) == hi for i in rows) and len(rows) == k + 1
                assert [int(rec["pos"][i]) for i in rows] == list(range(hi, hi + k + 1))
                lg[rows] = forward(om, cache.copy(),
                                   [Row(shape.mask_id, int(rec["pos"][i]), hi + k + 1, bool(rec["lora"][i])) for i in rows],
                                   lora_enabled=True)
        out.append(lg)
    return out


def run_quad(shape, k, n_new, prompts, max_ctx, lora=False, trace=True):
    import self_speculative_lm_amd as tm
    _, _, model, _ = get(shape)
    rows = max(64, len(prompts) * (1 + k + (k + 1) ** 2))
    sess = tm.Session(model, max_batch=len(prompts), max_ctx=max_ctx, max_rows=rows)
    for i, p in enumerate(prompts):
        sess.prefill(i, p)
    if lora:
        sess.set_lora(True)
    if trace:
        sess.set_trace(True)
    outs = [[] for _ in prompts]
    stats = []
    while min(len(o) for o in outs) < n_new:
        toks, st = sess.decode_step(tm.TRI_QUADSPEC, k)
        stats.append(st)
        for i in range(len(prompts)):
            outs[i] += [int(t) for t in toks[i] if t >= 0]
    return [o[:n_new] for o in outs], stats, sess


@pytest.mark.parametrize("shape,k", [(seeded.TINY, 4), (seeded.TINY_SHARP, 8), (seeded.TINY_LORA, 4)])
def test_tiny_quadspec_matches_oracle(shape, k):
    lora = shape.lora_rank > 0
    prompts = [seeded.prompt(16, shape.vocab), seeded.prompt(11, shape.vocab, stream=3)]
    max_ctx = 200
    got, stats, sess = run_quad(shape, k, 24, prompts, max_ctx, lora=lora)
    _, _, _, om = get(shape)
    for i, p in enumerate(prompts):
        o = OracleSession(om, max_ctx)
        o.prefill(p)
        assert got[i] == o.generate(MODE_QUADSPEC, 24, block=k, lora=lora)
        o2 = OracleSession(om, max_ctx)
        o2.prefill(p)
        assert got[i] == o2.generate(MODE_AR, 24)
    assert all(s[1] == 1 and 0 <= s[2] <= k and s[0] == s[2] + 1 for st in stats for s in st)
    ref = replay_quad(shape, om, sess.trace(), max_ctx, prompts, k)
    err = max(float(np.abs(r - t["logits"]).max()) for r, t in zip(ref, sess.trace()))
    print(f"[parity quadratic {shape.name} k={k}] forwards {len(ref)}, max |logit err| {err:.2e}")
    assert err <= TOL_F32 * shape.lm_head_scale, err


@pytest.mark.parametrize("shape", [seeded.SMALL_BF16, seeded.SMALL_BF16_LORA])
def test_small_bf16_quadspec_teacher_forced_and_equals_ar(shape):
    """head_dim 128 in bf16: the split-partial attention with the block keys
    folded in by the combine, the large-M GEMMs (1 + 8 + 81 rows) and the
    draft LoRA on the block rows."""
    import self_speculative_lm_amd as tm
    k = 8
    lora = shape.lora_rank > 0
    prompts = [seeded.prompt(40, shape.vocab)]
    max_ctx = 160
    got, stats, sess = run_quad(shape, k, 16, prompts, max_ctx, lora=lora)
    _, _, model, om = get(shape)
    ar = tm.Session(model, max_batch=1, max_ctx=max_ctx, max_rows=128)
    ar.prefill(0, prompts[0])
    want = [int(ar.decode_step(tm.TRI_AR, 1)[0][0, 0]) for _ in range(16)]
    assert got[0] == want
    ref = replay_quad(shape, om, sess.trace(), max_ctx, prompts, k)
    err = max(float(np.abs(r - t["logits"]).max()) for r, t in zip(ref, sess.trace()))
    print(f"[parity quadratic {shape.name} k={k}] forwards {len(ref)}, max |logit err| {err:.3e}")
    assert err <= TOL_BF16 * shape.lm_head_scale, err


@pytest.mark.parametrize("a_star", [0, 3, 8])
def test_quadspec_controlled_drafts_accept_exactly(a_star):
    """Carried drafts replaced by the greedy AR continuation with a forced
    mismatch at a*: every round after the first accepts exactly a* and
    commits a*+1 tokens of that continuation."""
    import self_speculative_lm_amd as tm
    shape, k = seeded.SMALL_BF16, 8
    _, _, model, _ = get(shape)
    prompt = seeded.prompt(24, shape.vocab, stream=5)
    max_ctx = 256
    ar = tm.Session(model, max_batch=1, max_ctx=max_ctx, max_rows=128)
    ar.prefill(0, prompt)
    for _ in range(60):
        ar.decode_step(tm.TRI_AR, 1)
    ref = ar.state(0)[0]
    sess = tm.Session(model, max_batch=1, max_ctx=max_ctx, max_rows=1 + k + (k + 1) ** 2)
    sess.prefill(0, prompt)
    sess.set_draft_override(0, ref, a_star)
    for r in range(4):
        _, st = sess.decode_step(tm.TRI_QUADSPEC, k)
        n, f, acc, _ = st[0]
        assert f == 1 and n == acc + 1
        if r > 0:
            assert acc == a_star
    got = sess.state(0)[0]
    assert got == ref[: len(got)]
