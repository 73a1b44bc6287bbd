"""End-to-end GPU parity of tri_decode_step in the three modes against the
oracle: free-running token sequences, teacher-forced logits (every traced
forward replayed through the oracle), batch invariance (GPU self-speculation
equals GPU AR), LoRA on the drafter only, ragged batches and state errors."""
import numpy as np
import pytest

import seeded
from oracle import MODE_AR, MODE_DIFFUSION, MODE_SELFSPEC, OracleModel, OracleSession
from oracle.sampler import vocab_reduce
from tests.gpu_util import device_weights, make_model, replay, top2_margin

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


def gpu_generate(shape, mode, n_new, block, tau=0.9, prompt_len=16, max_ctx=128, lora=False, trace=False,
                 prompts=None):
    import self_speculative_lm_amd as tm
    arrays, tens, model, om = get(shape)
    prompts = prompts or [seeded.prompt(prompt_len, shape.vocab)]
    sess = tm.Session(model, max_batch=len(prompts), max_ctx=max_ctx, max_rows=64 * len(prompts))
    if lora:
        sess.set_lora(True)
    if trace:
        sess.set_trace(True)
    for i, p in enumerate(prompts):
        sess.prefill(i, p)
    outs = [[] for _ in prompts]
    stats = []
    gmode = {MODE_AR: tm.TRI_AR, MODE_DIFFUSION: tm.TRI_DIFFUSION, MODE_SELFSPEC: tm.TRI_SELFSPEC}[mode]
    while min(len(o) for o in outs) < n_new:
        toks, st = sess.decode_step(gmode, block, tau)
        stats.append(st)
        for i in range(len(prompts)):
            outs[i] += [int(t) for t in toks[i] if t >= 0]
    return [o[:n_new] for o in outs], stats, sess


def oracle_generate(shape, mode, n_new, block, tau=0.9, prompt_len=16, max_ctx=128, lora=False, prompt=None):
    _, _, _, om = get(shape)
    o = OracleSession(om, max_ctx)
    o.prefill(prompt if prompt is not None else seeded.prompt(prompt_len, shape.vocab))
    return o.generate(mode, n_new, block=block, threshold=tau, lora=lora), o


def teacher_forced_error(shape, sess, max_ctx=128):
    _, _, _, om = get(shape)
    tr = sess.trace()
    ref = replay(shape, om, tr, max_ctx)
    err = 0.0
    for r, t in zip(ref, tr):
        if r is not None:
            err = max(err, float(np.abs(r - t["logits"]).max()))
    return err, tr, ref


@pytest.mark.parametrize("shape", [seeded.TINY, seeded.TINY_SHARP])
@pytest.mark.parametrize("mode", [MODE_AR, MODE_DIFFUSION, MODE_SELFSPEC])
def test_tiny_f32_free_running_matches_oracle(shape, mode):
    got, _, sess = gpu_generate(shape, mode, 32, 8, trace=True)
    want, _ = oracle_generate(shape, mode, 32, 8)
    err, _, _ = teacher_forced_error(shape, sess)
    assert err <= TOL_F32, err
    assert got[0] == want


def test_tiny_selfspec_equals_ar_and_accept_range():
    shape = seeded.TINY_SHARP
    ar, _, _ = gpu_generate(shape, MODE_AR, 40, 1)
    ss, stats, _ = gpu_generate(shape, MODE_SELFSPEC, 40, 8)
    assert ss == ar
    for st in stats:
        n, f, a, _ = st[0]
        assert 0 <= a <= 8 and n == a + 1 and f == 2


def test_tiny_lora_drafter_is_lossless():
    shape = seeded.TINY_LORA
    ar, _, _ = gpu_generate(shape, MODE_AR, 32, 1)
    ss, _, sess = gpu_generate(shape, MODE_SELFSPEC, 32, 8, lora=True, trace=True)
    assert ss == ar
    err, tr, _ = teacher_forced_error(shape, sess)
    assert err <= TOL_F32, err
    assert any(t["lora"].any() for t in tr)
    want, _ = oracle_generate(shape, MODE_SELFSPEC, 32, 8, lora=True)
    assert ss[0] == want


def test_tiny_ragged_batch_diffusion_and_selfspec():
    shape = seeded.TINY_SHARP
    prompts = [seeded.prompt(16, shape.vocab, stream=i) for i in range(3)]
    prompts[1] = prompts[1][:9]
    for mode in (MODE_DIFFUSION, MODE_SELFSPEC, MODE_AR):
        got, _, _ = gpu_generate(shape, mode, 24, 8, prompts=prompts)
        for i, p in enumerate(prompts):
            want, _ = oracle_generate(shape, mode, 24, 8, prompt=p)
            assert got[i] == want, (mode, i)


@pytest.mark.parametrize("shape", [seeded.SMALL_BF16, seeded.SMALL_BF16_SHARP])
def test_small_bf16_teacher_forced_and_batch_invariant(shape):
    ar, _, sess_ar = gpu_generate(shape, MODE_AR, 24, 1, prompt_len=40, trace=True)
    ss, _, sess_ss = gpu_generate(shape, MODE_SELFSPEC, 24, 32, prompt_len=40, trace=True)
    assert ss == ar                                      # GPU batch invariance: bit-identical decisions
    tol = TOL_BF16 * shape.lm_head_scale                 # logits scale with the lm_head
    for sess in (sess_ar, sess_ss):
        err, tr, ref = teacher_forced_error(shape, sess)
        assert err <= tol, err
        # a greedy decision of the GPU differs from the oracle's only where the
        # oracle's top-2 margin is within twice the logit error (a near-tie)
        decisions = flips = 0
        for r, t in zip(ref, tr):
            if r is None:
                continue
            for i in range(len(r)):
                decisions += 1
                if int(np.argmax(t["logits"][i])) != vocab_reduce(r[i])[0]:
                    assert top2_margin(r[i]) <= 2 * err
                    flips += 1
        assert flips <= 0.1 * decisions


def test_small_bf16_diffusion_teacher_forced():
    shape = seeded.SMALL_BF16_SHARP
    got, stats, sess = gpu_generate(shape, MODE_DIFFUSION, 64, 32, tau=0.7, prompt_len=64, trace=True)
    err, _, _ = teacher_forced_error(shape, sess)
    assert err <= TOL_BF16 * shape.lm_head_scale, err
    assert all(t < shape.vocab for t in got[0])


def test_small_bf16_lora_lossless():
    shape = seeded.SMALL_BF16_LORA
    ar, _, _ = gpu_generate(shape, MODE_AR, 16, 1, prompt_len=32)
    ss, _, sess = gpu_generate(shape, MODE_SELFSPEC, 16, 32, prompt_len=32, lora=True, trace=True)
    assert ss == ar
    err, _, _ = teacher_forced_error(shape, sess)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("shape,plen,max_rows", [(seeded.TINY, 45, 8), (seeded.SMALL_BF16, 100, 16),
                                                  (seeded.SMALL_BF16, 301, 300),   # one 300-row chunk
                                                  (seeded.SMALL_BF16, 571, 300)])  # 300 + 270 rows
def test_prefill_in_many_chunks_matches_oracle(shape, plen, max_rows):
    """A prompt longer than max_rows is prefilled in back-to-back chunks whose
    metadata uploads are queued asynchronously (no tracing, so nothing
    synchronises in between); the next step must see a correct cache."""
    import self_speculative_lm_amd as tm
    _, _, model, om = get(shape)
    prompt = seeded.prompt(plen, shape.vocab, stream=7)
    sess = tm.Session(model, max_batch=1, max_ctx=plen + 16, max_rows=max_rows)
    sess.prefill(0, prompt)
    sess.set_trace(True)
    out, _ = sess.decode_step(tm.TRI_AR, 1)
    tr = sess.trace()
    o = OracleSession(om, plen + 16, prefill_chunk=max_rows)
    o.prefill(prompt)
    o.keep_logits = True
    tok = o.ar_step()
    err = float(np.abs(o.records[-1].logits - tr[-1]["logits"]).max())
    tol = TOL_F32 if shape.dtype == "f32" else TOL_BF16
    assert err <= tol, err
    if top2_margin(o.records[-1].logits[-1]) > 2 * tol:
        assert out[0, 0] == tok[0]


def test_small_bf16_wide_batch_teacher_forced():
    """Ten sequences decoded together: the forwards have 330 rows, so every
    projection, including the 1000-wide (ragged) lm_head, runs on the
    large-M GEMM; the logits of every traced forward match the oracle."""
    shape = seeded.SMALL_BF16_SHARP
    prompts = [seeded.prompt(20 + 3 * i, shape.vocab, stream=20 + i) for i in range(10)]
    _, _, sess = gpu_generate(shape, MODE_DIFFUSION, 32, 32, tau=0.7, prompts=prompts, trace=True)
    err, tr, _ = teacher_forced_error(shape, sess)
    assert max(len(t["logits"]) for t in tr if t["logits"] is not None) >= 256
    assert err <= TOL_BF16 * shape.lm_head_scale, err


def test_small_bf16_lora_wide_batch_lossless():
    """Eight sequences in self-speculation with the drafter LoRA: the draft
    forward has 264 rows, so the rank-128 LoRA projections (N = 128: most
    waves of the large-M workgroup fall past the last feature block; K = 128:
    one short split) run on the large-M GEMM.  Still lossless against AR, and
    the teacher-forced logits match the oracle."""
    shape = seeded.SMALL_BF16_LORA
    prompts = [seeded.prompt(24 + 2 * i, shape.vocab, stream=40 + i) for i in range(8)]
    ar, _, _ = gpu_generate(shape, MODE_AR, 12, 1, prompts=prompts)
    ss, _, sess = gpu_generate(shape, MODE_SELFSPEC, 12, 32, prompts=prompts, lora=True, trace=True)
    assert ss == ar
    err, tr, _ = teacher_forced_error(shape, sess)
    assert max(len(t["logits"]) for t in tr if t["logits"] is not None) >= 256
    assert any(t["lora"].any() for t in tr)
    assert err <= TOL_BF16, err


def gpu_mixed(shape, prompts, schedule, block, lora=False, trace=False, max_ctx=200):
    """Mixed steps: schedule[t][i] is the mode of sequence i at step t (-1: left out)."""
    import self_speculative_lm_amd as tm
    _, _, model, _ = get(shape)
    sess = tm.Session(model, max_batch=len(prompts), max_ctx=max_ctx, max_rows=(block + 2) * len(prompts))
    if lora:
        sess.set_lora(True)
    if trace:
        sess.set_trace(True)
    for i, p in enumerate(prompts):
        sess.prefill(i, p)
    outs = [[] for _ in prompts]
    stats = []
    for modes in schedule:
        toks, st = sess.decode_step_mixed(modes, block)
        stats.append(st)
        for i in range(len(prompts)):
            outs[i] += [int(t) for t in toks[i] if t >= 0]
    return outs, stats, sess


def oracle_mixed(shape, prompts, schedule, block, lora=False, max_ctx=200):
    _, _, _, om = get(shape)
    outs = []
    for i, p in enumerate(prompts):
        o = OracleSession(om, max_ctx)
        o.prefill(p)
        out = []
        for modes in schedule:
            if modes[i] >= 0:
                out += o.mixed_step(modes[i], block, lora)
        outs.append(out)
    return outs


def mixed_schedule(n_seq, n_steps, seed):
    rng = np.random.default_rng(seed)
    sched = []
    for _ in range(n_steps):
        m = rng.choice([-1, MODE_AR, MODE_SELFSPEC], size=n_seq, p=[0.15, 0.4, 0.45])
        if (m < 0).all():
            m[0] = MODE_AR
        sched.append(m.astype(np.int32).tolist())
    return sched


def test_tiny_mixed_steps_match_oracle():
    """AR and self-speculation sequences (and sequences left out) in the same
    steps: every sequence commits exactly the oracle's tokens for its own
    modes, with the per-mode stats, and every traced forward matches."""
    shape = seeded.TINY_SHARP
    prompts = [seeded.prompt(n, shape.vocab, stream=60 + i) for i, n in enumerate((16, 9, 23, 16))]
    sched = mixed_schedule(len(prompts), 8, seed=5)
    got, stats, sess = gpu_mixed(shape, prompts, sched, 8, trace=True)
    want = oracle_mixed(shape, prompts, sched, 8)
    assert got == want
    for modes, st in zip(sched, stats):
        for m, (n, f, a, _) in zip(modes, st):
            if m == MODE_AR:
                assert (n, f, a) == (2, 2, -1)
            elif m == MODE_SELFSPEC:
                assert 0 <= a <= 8 and n == a + 1 and f == 2
            else:
                assert (n, f) == (0, 0)
    err, _, _ = teacher_forced_error(shape, sess, max_ctx=200)
    assert err <= TOL_F32, err


def test_small_bf16_lora_mixed_batch_lossless():
    """Six sequences, AR and self-speculation with the drafter LoRA in the same
    forwards (up to 200 rows: the large-M GEMM): every sequence commits the
    greedy AR continuation and the traced logits match the oracle."""
    shape = seeded.SMALL_BF16_LORA
    prompts = [seeded.prompt(24 + 3 * i, shape.vocab, stream=80 + i) for i in range(6)]
    sched = [[MODE_SELFSPEC, MODE_AR] * 3, [MODE_AR, MODE_SELFSPEC] * 3, [MODE_SELFSPEC] * 6,
             [MODE_AR, -1, MODE_SELFSPEC, MODE_SELFSPEC, -1, MODE_AR]]
    got, _, sess = gpu_mixed(shape, prompts, sched, 32, lora=True, trace=True)
    n = min(len(g) for g in got)
    # the same session shape (sequences, capacity), so the same key split
    ar, _, _ = gpu_generate(shape, MODE_AR, n, 1, prompts=prompts, max_ctx=200)
    for i in range(len(prompts)):
        assert got[i][:n] == ar[i], i
    err, tr, _ = teacher_forced_error(shape, sess, max_ctx=200)
    assert max(len(t["logits"]) for t in tr if t["logits"] is not None) >= 128
    assert any(t["lora"].any() for t in tr)
    assert err <= TOL_BF16, err


def test_small_bf16_rows_bit_identical_alone_and_in_a_wide_batch():
    """Batch invariance across the GEMM kernels: eight sequences stepped
    together (264 draft rows and 256 verify rows: every projection on the
    large-M kernel) give bit-identical logits for every row, and the same
    tokens, as each sequence stepped alone (33 / 32 rows: the decode kernel)."""
    import self_speculative_lm_amd as tm
    shape = seeded.SMALL_BF16
    _, _, model, _ = get(shape)
    prompts = [seeded.prompt(20 + 5 * i, shape.vocab, stream=120 + i) for i in range(8)]
    sessions = []
    for _ in range(2):
        sess = tm.Session(model, max_batch=8, max_ctx=160, max_rows=8 * 34)
        for i, p in enumerate(prompts):
            sess.prefill(i, p)
        sess.set_trace(True)
        sessions.append(sess)
    together, alone = sessions
    SS = tm.TRI_SELFSPEC
    for step in range(3):
        out_t, _ = together.decode_step_mixed([SS] * 8, 32)
        for i in range(8):
            out_a, _ = alone.decode_step_mixed([SS if j == i else -1 for j in range(8)], 32)
            assert (out_a[i] == out_t[i]).all(), (step, i)
    tr_t, tr_a = together.trace(), alone.trace()
    assert len(tr_a) == 8 * len(tr_t)
    for f, rec in enumerate(tr_t):
        assert len(rec["seq"]) >= 256
        step, which = divmod(f, 2)
        for i in range(8):
            solo = tr_a[(step * 8 + i) * 2 + which]
            rows = rec["seq"] == i
            assert (solo["seq"] == i).all()
            for key in ("tok", "pos", "hi"):
                assert (rec[key][rows] == solo[key]).all()
            assert np.array_equal(rec["logits"][rows], solo["logits"]), (f, i)


def test_small_bf16_ragged_mixed_step_rows_bit_identical_alone():
    """The attention's compacted grid (one workgroup per query group that
    holds rows, for steps whose sequences carry different row counts): six
    sequences stepped together in mixed AR / self-speculation steps give, row
    for row, the logits and tokens of each sequence stepped alone (one slot:
    the regular grid)."""
    import self_speculative_lm_amd as tm
    shape = seeded.SMALL_BF16
    _, _, model, _ = get(shape)
    prompts = [seeded.prompt(18 + 7 * i, shape.vocab, stream=150 + i) for i in range(6)]
    AR, SS = tm.TRI_AR, tm.TRI_SELFSPEC
    sched = [[SS, AR, AR, SS, AR, AR], [AR, AR, SS, AR, AR, AR], [AR, SS, AR, AR, SS, SS]]
    sessions = []
    for _ in range(2):
        sess = tm.Session(model, max_batch=6, max_ctx=200, max_rows=6 * 34)
        for i, p in enumerate(prompts):
            sess.prefill(i, p)
        sess.set_trace(True)
        sessions.append(sess)
    together, alone = sessions
    for modes in sched:
        out_t, _ = together.decode_step_mixed(modes, 32)
        for i in range(6):
            out_a, _ = alone.decode_step_mixed([modes[i] if j == i else -1 for j in range(6)], 32)
            assert (out_a[i] == out_t[i]).all(), (modes, i)
    tr_t, tr_a = together.trace(), alone.trace()
    assert len(tr_a) == 6 * len(tr_t)
    for f, rec in enumerate(tr_t):
        step, which = divmod(f, 2)
        for i in range(6):
            solo = tr_a[(step * 6 + i) * 2 + which]
            rows = rec["seq"] == i
            assert (solo["seq"] == i).all()
            for key in ("tok", "pos", "hi"):
                assert (rec[key][rows] == solo[key]).all()
            assert np.array_equal(rec["logits"][rows], solo["logits"]), (f, i)


def test_small_bf16_1500_rows_bit_identical_to_50_row_chunks():
    """Batch invariance where the large-M GEMM keeps one slot for several K
    splits (the down projection's two splits chained in split order, at
    1500 rows): a 1500-row teacher-forced forward gives logits bit-identical
    to the same rows run as thirty 50-row forwards on the decode kernel."""
    import torch
    import self_speculative_lm_amd as tm
    shape = seeded.SMALL_BF16
    _, _, model, _ = get(shape)
    n, c = 1500, 50
    toks = seeded.prompt(n, shape.vocab, stream=140)
    pos = np.arange(n, dtype=np.int32)
    seq = np.zeros(n, dtype=np.int32)
    sess = tm.Session(model, max_batch=1, max_ctx=n + 64, max_rows=n)
    big = torch.empty((n, shape.vocab), dtype=torch.float32, device="cuda")
    sess.forward(seq, toks, pos, pos + 1, logits=big)
    small = torch.empty((c, shape.vocab), dtype=torch.float32, device="cuda")
    for i in range(0, n, c):
        sess.forward(seq[i:i + c], toks[i:i + c], pos[i:i + c], pos[i:i + c] + 1, logits=small)
        torch.cuda.synchronize()
        assert torch.equal(big[i:i + c], small), i


def test_mixed_step_errors_leave_state_unchanged():
    import self_speculative_lm_amd as tm
    shape = seeded.TINY
    _, _, model, _ = get(shape)
    sess = tm.Session(model, max_batch=2, max_ctx=64, max_rows=16)
    AR, SS = tm.TRI_AR, tm.TRI_SELFSPEC
    with pytest.raises(tm.TriError) as e:
        sess.decode_step_mixed([AR, -1], 8)
    assert e.value.code == tm._lib.TRI_ESTATE               # not prefilled
    sess.prefill(0, seeded.prompt(30, shape.vocab))
    before = sess.state(0)
    for modes, block, code in (([-1, -1], 8, tm._lib.TRI_ESTATE),          # nothing to step
                               ([tm.TRI_DIFFUSION, -1], 8, tm._lib.TRI_EINVAL),
                               ([AR, AR], 8, tm._lib.TRI_ESTATE),           # sequence 1 not prefilled
                               ([SS, -1], 16, tm._lib.TRI_ECAPACITY),       # 1 + 16 rows > max_rows 16
                               ([SS, -1], 40, tm._lib.TRI_ECAPACITY),       # 30 + 41 > max_ctx 64
                               ([AR, -1], 0, tm._lib.TRI_EINVAL)):
        with pytest.raises(tm.TriError) as e:
            sess.decode_step_mixed(modes, block)
        assert e.value.code == code, (modes, block)
        assert sess.state(0) == before
    with pytest.raises(ValueError):
        sess.decode_step_mixed([AR], 8)
    out, st = sess.decode_step_mixed([AR, -1], 8)
    assert st[0][:2] == (2, 2) and (out[0, :2] >= 0).all() and (out[0, 2:] == -1).all()
    toks, kv = sess.state(0)
    assert len(toks) == 32 and kv == 31 and toks[30:] == out[0, :2].tolist()   # g1 stays pending


def test_state_errors_and_kv_bookkeeping():
    import self_speculative_lm_amd as tm
    shape = seeded.TINY
    _, _, model, _ = get(shape)
    sess = tm.Session(model, max_batch=2, max_ctx=40, max_rows=16)
    with pytest.raises(tm.TriError) as e:
        sess.decode_step(tm.TRI_AR, 1)
    assert e.value.code == tm._lib.TRI_ESTATE
    sess.prefill(0, seeded.prompt(30, shape.vocab))
    toks, kv = sess.state(0)
    assert len(toks) == 30 and kv == 29
    with pytest.raises(tm.TriError):
        sess.kv_append(0, 1)                      # nothing written beyond the prefix
    sess.kv_rollback(0, 4)
    assert sess.state(0)[1] == 25
    with pytest.raises(tm.TriError):
        sess.kv_rollback(0, 26)
    with pytest.raises(tm.TriError):
        sess.decode_step(tm.TRI_SELFSPEC, 32)      # 30 + 33 > max_ctx
    with pytest.raises(tm.TriError):
        sess.decode_step(tm.TRI_DIFFUSION, 8, 1.5)  # bad threshold
    # a rollback makes tokens pending again: the next AR step re-runs them
    out, st = sess.decode_step(tm.TRI_AR, 1)
    assert st[0][0] == 1
    toks2, kv2 = sess.state(0)
    assert len(toks2) == 31 and kv2 == 30
    # same result as a fresh session that never rolled back
    s2 = tm.Session(model, max_batch=1, max_ctx=40, max_rows=16)
    s2.prefill(0, seeded.prompt(30, shape.vocab))
    out2, _ = s2.decode_step(tm.TRI_AR, 1)
    assert out2[0, 0] == out[0, 0]


def test_tiny_scheduled_commit_rate_matches_oracle():
    """The controlled commit rate of diffusion mode: a scheduled sequence
    commits the oracle's top-n positions per forward while a sequence in the
    same forwards keeps the threshold rule; a prefill switches the schedule off."""
    import self_speculative_lm_amd as tm
    shape = seeded.TINY_SHARP
    _, _, model, om = get(shape)
    prompts = [seeded.prompt(n, shape.vocab, stream=70 + i) for i, n in enumerate((16, 11, 13))]
    counts = [[3, 1, 2], None, [2]]
    sess = tm.Session(model, max_batch=3, max_ctx=96, max_rows=3 * 24)
    sess.set_trace(True)
    for i, p in enumerate(prompts):
        sess.prefill(i, p)
        if counts[i]:
            sess.set_commit_schedule(i, counts[i])
    got = [[] for _ in prompts]
    fw = [[] for _ in prompts]
    for _ in range(3):
        toks, st = sess.decode_step(tm.TRI_DIFFUSION, 8, 0.9)
        for i in range(3):
            got[i] += toks[i][:8].tolist()
            fw[i].append(st[i][1])
    for i, p in enumerate(prompts):
        o = OracleSession(om, 96)
        o.prefill(p)
        want, wf = [], []
        for _ in range(3):
            f0 = o.forwards
            want += o.diffusion_block_scheduled(8, counts[i]) if counts[i] else o.diffusion_block(8, 0.9)
            wf.append(o.forwards - f0)
        assert got[i] == want, i
        assert fw[i] == wf, i
    assert fw[0] == [4, 4, 4] and fw[2] == [4, 4, 4]
    err, _, _ = teacher_forced_error(shape, sess, max_ctx=96)
    assert err <= TOL_F32, err
    sess.prefill(0, prompts[0])                          # the schedule is gone
    toks, _ = sess.decode_step(tm.TRI_DIFFUSION, 8, 0.9)
    o = OracleSession(om, 96)
    o.prefill(prompts[0])
    assert toks[0][:8].tolist() == o.diffusion_block(8, 0.9)
    with pytest.raises(tm.TriError):
        sess.set_commit_schedule(0, [2, 0])


def test_fp16_v_cache_out_of_range_fails_the_step():
    """A bf16 session keeps V in fp16 form (exact for |v| <= 65504).  A value
    outside that range is not saturated silently: the prefill or step that
    writes it fails with TRI_ENUMERIC and leaves the sequence as it was
    (reading R23).  Wv scaled by 2^18 (bf16-exact) puts |v| near 1e5."""
    import torch
    import self_speculative_lm_amd as tm
    shape = seeded.SMALL_BF16
    arrays, tens, _, _ = get(shape)
    big = dict(tens)
    big["layers.1.wv"] = (tens["layers.1.wv"].float() * 2.0 ** 18).to(torch.bfloat16)
    model = make_model(shape, big)
    sess = tm.Session(model, max_batch=1, max_ctx=64, max_rows=64)
    with pytest.raises(tm.TriError) as e:
        sess.prefill(0, seeded.prompt(16, shape.vocab))
    assert e.value.code == tm._lib.TRI_ENUMERIC and "fp16" in str(e.value)
    # a one-token prompt writes no V; the AR step's pending row does
    sess.prefill(0, seeded.prompt(1, shape.vocab))
    before = sess.state(0)
    with pytest.raises(tm.TriError) as e:
        sess.decode_step(tm.TRI_AR, 1)
    assert e.value.code == tm._lib.TRI_ENUMERIC
    after = sess.state(0)
    assert list(after[0]) == list(before[0]) and after[1] == before[1]
    # the flag was cleared: the same session still runs a model in range
    ok = tm.Session(get(shape)[2], max_batch=1, max_ctx=64, max_rows=64)
    ok.prefill(0, seeded.prompt(16, shape.vocab))
    ok.decode_step(tm.TRI_AR, 1)
