"""GPU parity of the speed-of-light analysis (tri_sol_block) against the
oracle's sol_block: float32 targets, serial orders and parallel commit steps
equal over chained blocks of a ragged batch; in bfloat16 every traced forward
matches the oracle teacher-forced, every parallel decision is exactly the
rule applied to the GPU's own logits, and the serial pass equals the
diffusion step at threshold 1."""
import numpy as np
import pytest

import seeded
from oracle import MODE_DIFFUSION, OracleSession
from oracle.sol import sol_block
from tests.test_gpu_model import TOL_BF16, TOL_F32, get, gpu_generate, teacher_forced_error

pytestmark = pytest.mark.gpu


def gpu_sol(shape, prompts, block, n_blocks, max_ctx=160, trace=False):
    import self_speculative_lm_amd as tm
    _, _, model, _ = get(shape)
    sess = tm.Session(model, max_batch=len(prompts), max_ctx=max_ctx, max_rows=(2 * block + 1) * len(prompts))
    if trace:
        sess.set_trace(True)
    for i, p in enumerate(prompts):
        sess.prefill(i, p)
    return [sess.sol_block(block) for _ in range(n_blocks)], sess


def test_tiny_sol_matches_oracle_over_chained_blocks():
    shape = seeded.TINY_SHARP
    prompts = [seeded.prompt(n, shape.vocab, stream=90 + i) for i, n in enumerate((16, 7, 21))]
    res, sess = gpu_sol(shape, prompts, 8, 3, trace=True)
    _, _, _, om = get(shape)
    for i, p in enumerate(prompts):
        o = OracleSession(om, 160)
        o.prefill(p)
        for r in res:
            want = sol_block(o, 8)
            assert r["target"][i].tolist() == want["target"], i
            assert r["order"][i].tolist() == want["order"], i
            assert r["step"][i].tolist() == want["step"], i
            assert int(r["forwards"][i]) == want["sol_forwards"], i
        assert sess.state(i)[0] == o.tokens
    err, _, _ = teacher_forced_error(shape, sess, max_ctx=160)
    assert err <= TOL_F32, err


def test_tiny_sol_block_one_and_full_width():
    shape = seeded.TINY
    p = seeded.prompt(12, shape.vocab, stream=95)
    _, _, _, om = get(shape)
    for B in (1, 64):
        res, _ = gpu_sol(shape, [p], B, 1, max_ctx=128)
        o = OracleSession(om, 128)
        o.prefill(p)
        want = sol_block(o, B)
        assert res[0]["target"][0].tolist() == want["target"]
        assert res[0]["step"][0].tolist() == want["step"]
        assert int(res[0]["forwards"][0]) == want["sol_forwards"]


def test_small_bf16_sol_decisions_follow_the_gpu_logits():
    shape = seeded.SMALL_BF16_SHARP
    B = 32
    prompt = seeded.prompt(40, shape.vocab, stream=97)
    res, sess = gpu_sol(shape, [prompt], B, 2, trace=True)
    err, tr, _ = teacher_forced_error(shape, sess, max_ctx=160)
    assert err <= TOL_BF16 * shape.lm_head_scale, err
    mask = shape.vocab
    t = next(i for i, f in enumerate(tr) if f["logits"] is not None)     # after the prefill forwards
    for r in res:
        target, order, step, F = r["target"][0], r["order"][0], r["step"][0], int(r["forwards"][0])
        # serial pass: B forwards, each committing the position it names with its greedy token
        for j in range(B):
            lg = tr[t]["logits"][-B:]
            i = order[j]
            assert int(np.argmax(lg[i])) == target[i]
            assert tr[t]["tok"][-B + i] == mask
            t += 1
        # parallel pass: each forward commits exactly the masked positions whose
        # greedy token on the GPU's logits equals the target, else the serial next
        y = np.full(B, mask)
        for f in range(F):
            rows = tr[t]
            np.testing.assert_array_equal(rows["tok"][-B:], y)
            g = np.argmax(rows["logits"][-B:], axis=1)
            right = [i for i in range(B) if y[i] == mask and g[i] == target[i]]
            now = [i for i in range(B) if step[i] == f]
            assert now == (right or [next(i for i in order if y[i] == mask)])
            y[now] = target[now]
            t += 1
        assert (y == target).all()
    assert t == len(tr)
    # the serial pass is the diffusion step at threshold 1
    got, _, _ = gpu_generate(shape, MODE_DIFFUSION, 2 * B, B, tau=1.0, prompts=[prompt], max_ctx=160)
    assert got[0] == res[0]["target"][0].tolist() + res[1]["target"][0].tolist()


def test_sol_errors_leave_state_unchanged():
    import self_speculative_lm_amd as tm
    shape = seeded.TINY
    _, _, model, _ = get(shape)
    sess = tm.Session(model, max_batch=2, max_ctx=64, max_rows=40)
    with pytest.raises(tm.TriError):
        sess.sol_block(8)                                  # nothing prefilled
    sess.prefill(0, seeded.prompt(20, shape.vocab))
    before = sess.state(0)
    for B in (0, 65):
        with pytest.raises(tm.TriError):
            sess.sol_block(B)
    with pytest.raises(tm.TriError):
        sess.sol_block(50)                                 # 20 + 50 > max_ctx
    assert sess.state(0) == before
    r = sess.sol_block(8)
    assert r["forwards"][1] == -1 and (r["target"][1] == -1).all()
    assert sess.state(0)[0][-8:] == r["target"][0].tolist()


def test_sol_ignores_a_commit_schedule():
    """The serial pass is the threshold-1 rule whatever commit schedule the
    sequence carries (the schedule is a diffusion-step measurement hook)."""
    import self_speculative_lm_amd as tm
    shape = seeded.TINY_SHARP
    _, _, model, _ = get(shape)
    p = seeded.prompt(14, shape.vocab, stream=99)
    outs = []
    for sched in (None, [3, 2]):
        sess = tm.Session(model, max_batch=1, max_ctx=96, max_rows=40)
        sess.prefill(0, p)
        if sched:
            sess.set_commit_schedule(0, sched)
        r = sess.sol_block(8)
        outs.append((r["target"][0].tolist(), r["order"][0].tolist(), r["step"][0].tolist()))
    assert outs[0] == outs[1]
