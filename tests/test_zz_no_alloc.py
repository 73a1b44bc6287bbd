"""The allocation-free attention entry point (block_causal_attn_noalloc):
through the C-ABI, bit-identical to block_causal_attn with a caller
workspace, on two calls in a row (the second smaller, after the first left
its partials in the static scratch), and a request beyond the scratch is
refused."""
import math

import numpy as np
import pytest

import seeded

pytestmark = pytest.mark.gpu


def _case(prefix, nrows, hq, hkv, kv_split, seed):
    import torch
    hd = 128
    q, k, v = seeded.attention_operands(nrows, prefix, hq, hkv, hd, batch=1, bf16=True, seed=seed)
    L = prefix + nrows
    ctx = (L + 63) // 64 * 64
    kc = torch.zeros((1, hkv, ctx, hd), dtype=torch.bfloat16)
    vc = torch.zeros((1, hkv, hd, ctx), dtype=torch.bfloat16)
    kc[0, :, :L] = torch.from_numpy(k[0, :L]).permute(1, 0, 2).to(torch.bfloat16)
    vc[0, :, :, :L] = torch.from_numpy(v[0, :L]).permute(1, 2, 0).to(torch.bfloat16)
    tq = torch.from_numpy(q[0, :nrows]).to(torch.bfloat16).cuda()
    his = [prefix + i + 1 for i in range(nrows)]
    ss = torch.tensor([0, nrows], dtype=torch.int32, device="cuda")
    hi = torch.tensor(his, dtype=torch.int32, device="cuda")
    return tq, kc.cuda(), vc.cuda(), ss, hi, max(his)


@pytest.mark.parametrize("first,second", [((3000, 33, 32, 8, 128), (700, 9, 32, 8, 128)),
                                          ((5000, 33, 40, 8, 0), (200, 4, 40, 8, 0))])
def test_noalloc_equals_workspace_entry_on_consecutive_calls(first, second):
    import torch
    import self_speculative_lm_amd as tm
    for n, (prefix, nrows, hq, hkv, kv_split) in enumerate((first, second)):
        tq, kc, vc, ss, hi, mh = _case(prefix, nrows, hq, hkv, kv_split, seed=20 + n)
        a = torch.zeros_like(tq)
        b = torch.full_like(tq, float("nan"))
        tm.block_causal_attn(tq, kc, vc, ss, hi, a, 1.0 / math.sqrt(128), max_rows_per_seq=nrows, max_hi=mh,
                             kv_split=kv_split)
        tm.block_causal_attn_noalloc(tq, kc, vc, ss, hi, b, 1.0 / math.sqrt(128), max_rows_per_seq=nrows, max_hi=mh,
                                     kv_split=kv_split)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (n, prefix, nrows)


def test_noalloc_refuses_partials_beyond_the_scratch():
    import torch
    import self_speculative_lm_amd as tm
    tq, kc, vc, ss, hi, mh = _case(4096, 64, 32, 8, 64, seed=30)
    out = torch.zeros_like(tq)
    # 64-key splits of 4160 keys: 65 splits x 64 rows x 32 heads x 130 floats > 32 MiB
    with pytest.raises(tm.TriError) as e:
        tm.block_causal_attn_noalloc(tq, kc, vc, ss, hi, out, 0.1, max_rows_per_seq=64, max_hi=mh, kv_split=64)
    assert e.value.code == tm._lib.TRI_ECAPACITY
