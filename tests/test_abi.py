"""The C-ABI library loads, exports every function include/trimode.h declares,
and validates arguments on the host (no GPU needed: nothing here launches)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trimode.h")


@pytest.fixture(scope="module")
def L():
    from self_speculative_lm_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from self_speculative_lm_amd.build import build
        build()
    return _lib.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([A-Za-z_]\w*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "sizeof")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tri_decode_step", "block_causal_attn", "sample_commit", "verify_accept", "kv_append", "kv_rollback"):
        assert n in names


def test_library_exports_every_declared_function(L):
    from self_speculative_lm_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    # and the Python binding declares a signature for each of them
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def _desc(**kw):
    from self_speculative_lm_amd._lib import ModelDesc, TRI_BF16
    d = dict(n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=2, head_dim=128, d_ffn=1024, vocab=1024,
             rope_base=10000.0, rms_eps=1e-6, dtype=TRI_BF16, lora_rank=0)
    d.update(kw)
    return ModelDesc(**d)


def _create(L, desc, n=None, null_at=None, buf=0x100000, nbytes=1 << 40):
    n_w = 1 + 9 * desc.n_layers + 2 + (2 * desc.n_layers if desc.lora_rank else 0)
    ptrs = [0x1000 * (i + 1) for i in range(n_w if n is None else n)]
    if null_at is not None:
        ptrs[null_at] = 0
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    h = ctypes.c_void_p()
    return L.tri_model_create(ctypes.byref(desc), arr, len(ptrs), buf, nbytes, None, ctypes.byref(h))


def _bytes(L, desc):
    n = ctypes.c_size_t()
    rc = L.tri_model_bytes(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


def test_model_descriptor_and_buffer_validation_on_host(L):
    from self_speculative_lm_amd._lib import TRI_ECAPACITY, TRI_EINVAL, TRI_F32
    rc, small = _bytes(L, _desc())
    assert rc == 0 and small > 0
    rc, more = _bytes(L, _desc(n_layers=3))
    assert rc == 0 and more > small                          # one more layer of weights
    rc, lora = _bytes(L, _desc(lora_rank=64))
    assert rc == 0 and lora > small                          # the adapter is stored too
    # bf16 projection rows are padded to 128 in the packed layout
    rc, b1 = _bytes(L, _desc(vocab=1000))
    rc2, b2 = _bytes(L, _desc(vocab=1024))
    assert rc == rc2 == 0 and b1 <= b2
    assert _bytes(L, _desc(head_dim=64))[0] == TRI_EINVAL    # bf16 needs hd 128
    assert _bytes(L, _desc(n_q_heads=3))[0] == TRI_EINVAL    # hq % hkv
    assert _bytes(L, _desc(dtype=7))[0] == TRI_EINVAL
    assert _bytes(L, _desc(dtype=TRI_F32, head_dim=32, d_model=128, n_q_heads=4, n_kv_heads=4))[0] == 0
    # creation is refused before any device work for bad pointers and buffers
    assert _create(L, _desc(), n=5) == TRI_EINVAL            # pointer count
    assert _create(L, _desc(), null_at=3) == TRI_EINVAL      # null weight
    assert _create(L, _desc(), buf=0) == TRI_EINVAL          # null model buffer
    assert _create(L, _desc(), nbytes=small - 1) == TRI_ECAPACITY
    assert _create(L, _desc(), buf=0x100010) == TRI_EINVAL   # misaligned buffer
    assert b"aligned" in L.tri_last_error()


def test_kernel_entry_points_validate_on_host(L):
    from self_speculative_lm_amd._lib import TRI_ECAPACITY, TRI_EINVAL
    n = ctypes.c_size_t()
    assert L.block_causal_attn_ws_bytes(33, 32, 128, 32800, 0, ctypes.byref(n)) == 0
    assert n.value > 33 * 32 * 128 * 4
    assert L.block_causal_attn_ws_bytes(33, 32, 128, 32800, 100, ctypes.byref(n)) == TRI_EINVAL
    assert L.sample_commit_ws_bytes(33, 151936, ctypes.byref(n)) == 0
    fake = ctypes.c_void_p(0x1000)
    # threshold out of range, then a workspace that is too small: rejected before any launch
    assert L.sample_commit(fake, 4, 100, fake, fake, 1, 1.5, fake, fake, fake, fake, fake, 1 << 20, None) == TRI_EINVAL
    assert L.sample_commit(fake, 4, 100, fake, fake, 1, 0.5, fake, fake, fake, fake, fake, 1, None) == TRI_ECAPACITY
    assert L.verify_accept(None, fake, 1, 4, fake, fake, None, None) == TRI_EINVAL
    assert L.block_causal_attn(fake, fake, fake, 1, fake, fake, 4, 4, 10, 8, 2, 128, 100, 0.1, 1, 0, fake, fake, 1 << 20,
                               None) == TRI_EINVAL      # ctx % 64 != 0
