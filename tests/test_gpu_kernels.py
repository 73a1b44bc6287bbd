"""GPU parity of the kernel-level C-ABI entry points against the oracle:
block_causal_attn, sample_commit and verify_accept."""
import math

import numpy as np
import pytest

import seeded
from oracle.model import attend
from oracle.sampler import accept_length, commit_set, vocab_reduce

pytestmark = pytest.mark.gpu

# bf16 attention bound: the output is rounded to bf16 (<= 2^-9 relative of
# max|v|) and the probabilities enter P.V rounded (fp16 in the kernel, <=
# 2^-12; the bound keeps bf16's 2^-9); with N(0,1) values max|v| < 6, so
# |err| <= 2 * 2^-9 * 6 ~ 2.3e-2.
ATT_TOL_BF16 = 2.5e-2
ATT_TOL_F32 = 2e-5


def _attn_case(prefixes, nrows, hq, hkv, hd, bf16, causal=False, kv_split=0, seed=3, sample=None, vf16=False,
               v_scale=1.0, return_max=False):
    """Max |GPU - oracle| over the sampled rows.  vf16: the V cache is passed in
    the session's fp16 form (TRI_BF16_V16) of the same bf16 values; v_scale
    (a power of two) scales V exactly."""
    import torch
    import self_speculative_lm_amd as tm
    b = len(prefixes)
    maxlen = max(p + n for p, n in zip(prefixes, nrows))
    ctx = (maxlen + 63) // 64 * 64
    R = max(nrows)
    q, k, v = seeded.attention_operands(R, max(prefixes), hq, hkv, hd, batch=b, bf16=bf16, seed=seed)
    if v_scale != 1.0:
        v = v * np.float32(v_scale)
    # k, v: [b, Pmax + R, hkv, hd]; sequence s uses positions [0, P_s + n_s)
    tdt = torch.bfloat16 if bf16 else torch.float32
    kc = torch.zeros((b, hkv, ctx, hd), dtype=tdt)
    vc = torch.zeros((b, hkv, hd, ctx), dtype=torch.float16 if vf16 else tdt)
    qs, his, starts = [], [], [0]
    for s in range(b):
        L = prefixes[s] + nrows[s]
        kc[s, :, :L] = torch.from_numpy(k[s, :L]).permute(1, 0, 2).to(tdt)
        vc[s, :, :, :L] = torch.from_numpy(v[s, :L]).permute(1, 2, 0).to(tdt).to(vc.dtype)
        qs.append(q[s, : nrows[s]])
        for i in range(nrows[s]):
            his.append(prefixes[s] + i + 1 if causal else L)
        starts.append(starts[-1] + nrows[s])
    qn = np.concatenate(qs)
    dev = "cuda"
    tq = torch.from_numpy(qn).to(tdt).to(dev)
    out = torch.zeros_like(tq)
    seq_start = torch.tensor(starts, dtype=torch.int32, device=dev)
    row_hi = torch.tensor(his, dtype=torch.int32, device=dev)
    tm.block_causal_attn(tq, kc.to(dev), vc.to(dev), seq_start, row_hi, out, 1.0 / math.sqrt(hd),
                         max_rows_per_seq=R, max_hi=max(his), kv_split=kv_split)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rows = list(range(len(his))) if sample is None else sample
    err = vmax = 0.0
    cache = {}
    for r in rows:
        s = int(np.searchsorted(starts, r, side="right") - 1)
        if s not in cache:
            cache = {s: (k[s].astype(np.float64), v[s].astype(np.float64))}
        K, V = cache[s]
        ref = attend(qn[r].astype(np.float64), K, V, his[r], hq // hkv)
        err = max(err, float(np.abs(ref - got[r]).max()))
        vmax = max(vmax, float(np.abs(ref).max()))
    return (err, vmax) if return_max else err


@pytest.mark.parametrize("prefixes,nrows,causal,kv_split", [
    ([0], [33], False, 64),
    ([37], [33], False, 64),
    ([31], [33], False, 0),
    ([700], [32], True, 256),
    ([200], [1], False, 0),
    ([5, 130, 300], [1, 33, 8], False, 128),
    ([64, 1], [64, 63], True, 64),
    ([3000], [4], True, 0),                     # one query tile, long prefix
    ([5000], [33], True, 0),                    # nine query tiles past 4K keys: two tiles per wave
    ([4500, 300], [33, 40], False, 512),        # mixed lengths, two query tiles per wave
])
def test_block_causal_attn_bf16_matches_oracle(prefixes, nrows, causal, kv_split):
    err = _attn_case(prefixes, nrows, 32, 8, 128, True, causal, kv_split)
    assert err <= ATT_TOL_BF16, err


@pytest.mark.parametrize("prefixes,nrows,kv_split", [
    ([100], [33], 64),
    ([6000], [33], 0),                  # 165 query vectors past 4K keys: two query groups of two tiles per wave
    ([5000, 700, 4200], [33, 32, 5], 1024),   # three sequences, query groups 8 workgroup ids apart
])
def test_block_causal_attn_bf16_group5(prefixes, nrows, kv_split):
    """Five query heads per kv head (the 14B-class head layout)."""
    rng = np.random.default_rng(sum(prefixes))
    n = sum(nrows)
    sample = sorted(set(rng.integers(0, n, 8).tolist() + [0, n - 1]))
    assert _attn_case(prefixes, nrows, 40, 8, 128, True, False, kv_split, sample=sample) <= ATT_TOL_BF16


@pytest.mark.parametrize("prefixes,nrows,hq,causal,kv_split", [
    ([16384], [33], 40, False, 1024),           # the 14B-class draft forward behind a 16K prefix
    ([16384], [32], 40, True, 1024),            # its verify forward (causal rows)
    ([32768], [33], 40, False, 1024),
    ([32768] * 8, [32] * 8, 32, False, 0),      # eight sequences of 32K keys
])
def test_block_causal_attn_fp16_v_cache_matches_oracle(prefixes, nrows, hq, causal, kv_split):
    """The V cache form a bf16 session keeps (fp16 bits of the bf16 values),
    at the long-prefix launch shapes the sessions use: 1024-key splits and two
    query tiles per slot (a 33-row block of 5-head groups is 165 query
    vectors)."""
    rng = np.random.default_rng(sum(prefixes) + len(prefixes))
    n = sum(nrows)
    sample = sorted(set(rng.integers(0, n, 6).tolist() + [0, n - 1]))
    err = _attn_case(prefixes, nrows, hq, 8, 128, True, causal, kv_split, sample=sample, vf16=True)
    print(f"fp16-V attention {prefixes[0]} keys x {len(prefixes)}, {hq}q: max |err| {err:.3e}")
    assert err <= ATT_TOL_BF16, err


def test_block_causal_attn_fp16_v_cache_subnormal_values():
    """V values below fp16's normal range (2^-20 * N(0,1), about 1e-6) become
    fp16 subnormals in the cache: each loses at most half a subnormal step,
    2^-25, so a convex combination of them moves by at most 2^-25.  With the
    bf16 output rounding (2^-9 of the output) and the fp16 P (2^-12 of the
    values) the bound is 2^-25 + 2^-8 * max|out| + 2^-11 * max|v|."""
    scale = 2.0 ** -20
    err, omax = _attn_case([700], [33], 32, 8, 128, True, False, 256, vf16=True, v_scale=scale, return_max=True)
    bound = 2.0 ** -25 + 2.0 ** -8 * omax + 2.0 ** -11 * 6 * scale
    print(f"subnormal V: max |err| {err:.3e}, bound {bound:.3e}")
    assert err <= bound, (err, bound)


@pytest.mark.parametrize("prefix,nrows,kv_split", [(600, 33, 256), (5000, 33, 512), (130, 40, 64), (6000, 33, 4096),
                                                   (0, 300, 4096)])
def test_block_causal_attn_row_independent_of_batch(prefix, nrows, kv_split):
    """A row's bf16 output is bit-identical whether it is computed inside a
    causal block of nrows rows or alone (same q, same keys, same kv_split):
    the kernel's rounding may depend on kv_split only, never on which other
    queries share a workgroup or a wave."""
    import torch
    import self_speculative_lm_amd as tm
    hq, hkv, hd = 32, 8, 128
    q, k, v = seeded.attention_operands(nrows, prefix, hq, hkv, hd, batch=1, bf16=True, seed=11)
    L = prefix + nrows
    # Exact power-of-two scalings (bf16 stays bf16) that give the scores a wide
    # range, growing along the keys at a different rate per row, so that the
    # online softmax moves its base at different tiles for different queries.
    q = q * (2.0 ** (np.arange(nrows) % 4))[None, :, None, None]
    k = k * np.where(np.arange(L) >= L // 2, 4.0, 1.0)[None, :, None, None]
    ctx = (L + 63) // 64 * 64
    kc = torch.zeros((1, hkv, ctx, hd), dtype=torch.bfloat16)
    vc = torch.zeros((1, hkv, hd, ctx), dtype=torch.bfloat16)
    kc[0, :, :L] = torch.from_numpy(k[0, :L]).permute(1, 0, 2).to(torch.bfloat16)
    vc[0, :, :, :L] = torch.from_numpy(v[0, :L]).permute(1, 2, 0).to(torch.bfloat16)
    kc, vc = kc.cuda(), vc.cuda()
    tq = torch.from_numpy(q[0, :nrows]).to(torch.bfloat16).cuda()

    def run(rows, his):
        out = torch.zeros((len(rows), hq, hd), dtype=torch.bfloat16, device="cuda")
        ss = torch.tensor([0, len(rows)], dtype=torch.int32, device="cuda")
        hi = torch.tensor(his, dtype=torch.int32, device="cuda")
        tm.block_causal_attn(tq[rows].contiguous(), kc, vc, ss, hi, out, 1.0 / math.sqrt(hd),
                             max_rows_per_seq=len(rows), max_hi=max(his), kv_split=kv_split)
        torch.cuda.synchronize()
        return out.cpu()

    his = [prefix + i + 1 for i in range(nrows)]
    full = run(list(range(nrows)), his)
    # long splits: every row (each launch shape adds its own sums; two query
    # tiles per wave once differed in single elements)
    rows = range(nrows) if kv_split >= 4096 and nrows <= 40 else sorted({0, 1, nrows // 2, nrows - 1})
    for i in rows:
        alone = run([i], [his[i]])
        assert torch.equal(alone[0], full[i]), f"row {i} differs alone vs in the block"
    if nrows >= 256:  # a prefill-sized block against its halves (other launch shapes)
        h = nrows // 2
        assert torch.equal(run(list(range(h)), his[:h]), full[:h])
        assert torch.equal(run(list(range(h, nrows)), his[h:]), full[h:])
    pair = run([nrows - 1, 0], [his[-1], his[0]])           # other rows, other order
    assert torch.equal(pair[0], full[nrows - 1]) and torch.equal(pair[1], full[0])


@pytest.mark.parametrize("short,long_,kv_split", [(40, 700, 256), (100, 3000, 128)])
def test_block_causal_attn_short_row_same_bits_beside_a_long_one(short, long_, kv_split):
    """A sequence whose keys fit in one split gets the same bits alone (one
    split: the kernel normalises in its epilogue) and beside a sequence that
    needs several splits (the launch then merges split partials for every
    row, one partial for the short sequence's rows)."""
    import torch
    import self_speculative_lm_amd as tm
    hq, hkv, hd, nr = 32, 8, 128, 8
    L = long_ + nr
    ctx = (L + 63) // 64 * 64
    q, k, v = seeded.attention_operands(nr, long_, hq, hkv, hd, batch=2, bf16=True, seed=21)
    kc = torch.zeros((2, hkv, ctx, hd), dtype=torch.bfloat16)
    vc = torch.zeros((2, hkv, hd, ctx), dtype=torch.bfloat16)
    kc[:, :, :L] = torch.from_numpy(k).permute(0, 2, 1, 3).to(torch.bfloat16)
    vc[:, :, :, :L] = torch.from_numpy(v).permute(0, 2, 3, 1).to(torch.bfloat16)
    kc, vc = kc.cuda(), vc.cuda()
    tq = torch.from_numpy(q.reshape(2 * nr, hq, hd)).to(torch.bfloat16).cuda()
    his_a = [short - nr + i + 1 for i in range(nr)]          # sequence 0: keys [0, short)
    his_b = [long_ + i + 1 for i in range(nr)]               # sequence 1: several splits
    assert max(his_a) <= kv_split < max(his_b)

    def run(n_seq, his, kc_, vc_, qq):
        out = torch.zeros((len(his), hq, hd), dtype=torch.bfloat16, device="cuda")
        ss = torch.tensor([nr * i for i in range(n_seq + 1)], dtype=torch.int32, device="cuda")
        hi = torch.tensor(his, dtype=torch.int32, device="cuda")
        tm.block_causal_attn(qq, kc_, vc_, ss, hi, out, 1.0 / math.sqrt(hd), max_rows_per_seq=nr,
                             max_hi=max(his), kv_split=kv_split)
        torch.cuda.synchronize()
        return out.cpu()

    both = run(2, his_a + his_b, kc, vc, tq)
    alone = run(1, his_a, kc[:1].contiguous(), vc[:1].contiguous(), tq[:nr].contiguous())
    assert torch.equal(alone, both[:nr])


@pytest.mark.parametrize("prefixes,nrows,hq,hkv,hd,causal", [
    ([0], [8], 4, 4, 32, False), ([50], [9], 4, 4, 32, True), ([20, 70], [9, 16], 4, 2, 64, False),
    ([100], [3], 2, 1, 128, False),
])
def test_block_causal_attn_f32_matches_oracle(prefixes, nrows, hq, hkv, hd, causal):
    err = _attn_case(prefixes, nrows, hq, hkv, hd, False, causal)
    assert err <= ATT_TOL_F32, err


@pytest.mark.parametrize("prefix,batch,causal", [(512, 1, False), (2048, 8, False), (8192, 1, True),
                                                 (32768, 1, False), (32768, 8, False)])
def test_block_causal_attn_full_size_sampled(prefix, batch, causal):
    """Attention-alone shapes (32 q / 8 kv heads, hd 128, 32-row block) at the
    benchmark's launch configuration, checked on sampled rows."""
    rng = np.random.default_rng(prefix + batch)
    sample = sorted(set(rng.integers(0, 32 * batch, 6).tolist() + [0, 32 * batch - 1]))
    err = _attn_case([prefix] * batch, [32] * batch, 32, 8, 128, True, causal, 0, sample=sample)
    assert err <= ATT_TOL_BF16, err


def test_block_causal_attn_rejects_bad_arguments():
    import torch
    import self_speculative_lm_amd as tm
    q = torch.zeros((4, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, 2, 100, 128), dtype=torch.bfloat16, device="cuda")  # ctx not a multiple of 64
    vc = torch.zeros((1, 2, 128, 100), dtype=torch.bfloat16, device="cuda")
    ss = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    hi = torch.full((4,), 10, dtype=torch.int32, device="cuda")
    with pytest.raises(tm.TriError):
        tm.block_causal_attn(q, kc, vc, ss, hi, torch.zeros_like(q), 0.1, max_rows_per_seq=4, max_hi=10)


# ----------------------------------------------------------------- sampler
def _sampler_case(rows, vocab, seed, kinds, blocks, tau, plant=None):
    import torch
    import self_speculative_lm_amd as tm
    lg = seeded.logits_matrix(rows, vocab, seed, 1.0)
    if plant:
        plant(lg)
    dev = "cuda"
    tl = torch.from_numpy(lg).to(dev)
    kind = torch.tensor(kinds, dtype=torch.int32, device=dev)
    bs = torch.tensor(blocks, dtype=torch.int32, device=dev) if blocks else None
    ot = torch.zeros(rows, dtype=torch.int32, device=dev)
    oc = torch.zeros(rows, dtype=torch.float32, device=dev)
    om = torch.zeros(rows, dtype=torch.int32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    tm.sample_commit(tl, kind, bs, tau, ot, oc, om, st)
    torch.cuda.synchronize()
    return lg, ot.cpu().numpy(), oc.cpu().numpy(), om.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("vocab", [1000, 151936])
@pytest.mark.parametrize("tau", [0.0, 0.5, 0.9, 1.0])
def test_sample_commit_matches_oracle(vocab, tau):
    rows = 33
    kinds = [1] + [2] * 20 + [3, 2, 2, 3, 2, 2, 3, 2, 2, 2, 2, 2]
    blocks = [1, 17, 33]

    def plant(lg):
        lg[3, 7] = lg[3].max() + 30.0     # very confident: passes any tau < 1
        lg[20, 11] = lg[20].max() + 2.0
        lg[25, 100] = lg[25, 200] = lg[25].max() + 25.0   # exact tie: lowest id, conf ~ 0.5
        lg[30, :] = 0.0                                   # all equal: id 0, conf 1/V

    lg, tok, conf, com, st = _sampler_case(rows, vocab, 17 + vocab, kinds, blocks, tau, plant)
    assert st == 0
    ref = [vocab_reduce(lg[r].astype(np.float64)) if kinds[r] else (0, 0.0) for r in range(rows)]
    for r in range(rows):
        if kinds[r] == 0:
            continue
        assert tok[r] == ref[r][0], r
        assert conf[r] == pytest.approx(ref[r][1], rel=2e-6), r
    assert com[0] == 1
    for b in range(len(blocks) - 1):
        lo, hi = blocks[b], blocks[b + 1]
        el = [kinds[r] == 2 for r in range(lo, hi)]
        cf = [ref[r][1] for r in range(lo, hi)]
        flagged = any(abs(c - tau) < 1e-6 for c, e in zip(cf, el) if e)
        want = set(lo + i for i in commit_set(cf, el, tau))
        gotc = set(r for r in range(lo, hi) if com[r])
        if not flagged:
            assert gotc == want, (b, gotc, want)


def test_sample_commit_flags_non_finite_rows():
    kinds = [1, 1, 2, 2]

    def plant(lg):
        lg[1, 5] = np.nan

    _, tok, conf, com, st = _sampler_case(4, 512, 5, kinds, [2, 4], 0.5, plant)
    assert st == 1 and com[1] == 0 and tok[1] == -1
    assert com[0] == 1


# ------------------------------------------------------------------ verify
@pytest.mark.parametrize("k", [1, 8, 32, 64])
def test_verify_accept_matches_oracle(k):
    import torch
    import self_speculative_lm_amd as tm
    b = 16
    d, g = seeded.token_pairs(b, k, 50, seed=k, match_prob=0.85)
    d[0] = g[0, :k]          # all match -> a = k
    d[1, 0] = (g[1, 0] + 1) % 50   # immediate mismatch -> a = 0
    dev = "cuda"
    td = torch.from_numpy(d).to(dev)
    tg = torch.from_numpy(g).to(dev)
    acc = torch.zeros(b, dtype=torch.int32, device=dev)
    com = torch.zeros((b, k + 1), dtype=torch.int32, device=dev)
    kvl = torch.arange(b, dtype=torch.int32, device=dev) * 10
    tm.verify_accept(td, tg, acc, com, kvl)
    torch.cuda.synchronize()
    acc, com, kvl = acc.cpu().numpy(), com.cpu().numpy(), kvl.cpu().numpy()
    for i in range(b):
        a = accept_length(list(d[i]), list(g[i]))
        assert acc[i] == a
        assert list(com[i, : a + 1]) == list(g[i, : a + 1])
        assert (com[i, a + 1:] == -1).all()
        assert kvl[i] == 10 * i + a
        assert 1 <= a + 1 <= k + 1
    assert acc[0] == k and acc[1] == 0
