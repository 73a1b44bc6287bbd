"""bfloat16 rounding for the oracle (test infrastructure only).

The bf16 models store weights, the KV cache and every GEMM input operand as
bfloat16 and accumulate in float32 or wider; the oracle reproduces those
storage points by rounding its float64 values to the nearest bfloat16.
"""
import numpy as np

_BF16_MIN_NORMAL_EXP = -126   # smallest normal exponent
_BF16_MANT_BITS = 8           # significant bits including the implicit one
_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each float64 entry, ties to even (returned as float64).

    Written from the format's definition: 8 significant bits for normal
    numbers, a fixed quantum 2^-133 below 2^-126, and infinity once the
    rounded magnitude would exceed the largest finite bfloat16.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    _, e = np.frexp(xf)                      # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, _BF16_MIN_NORMAL_EXP + 1)  # subnormal range keeps a fixed quantum
    quantum = np.ldexp(1.0, e - _BF16_MANT_BITS)
    r = np.rint(xf / quantum) * quantum      # np.rint rounds half to even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xf), r)
    out[finite] = r
    return out
