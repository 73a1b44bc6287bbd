"""CPU oracle of the tri-mode decode step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its Python
binding) never calls it and fails loudly when its native library is missing.

It is a plain, slow NumPy implementation in float64 of what the GPU path
computes, written from the public write-ups of Nemotron-Labs-Diffusion:

* [Notes] "Nemotron-Labs-Diffusion 技术报告：统一 AR、Diffusion 与
  Self-Speculation 的三模式语言模型" (ranhao.site technical notes), sections 3-7.
* [Digest] "Nemotron-Labs-Diffusion: A Tri-Mode Language Model Unifying
  Autoregressive, Diffusion, and Self-Speculation Decoding" (r9-hu paper
  digest), sections Method and Key Contributions.
* [Blog] "Nemotron-Labs 扩散语言模型实现光速级文本生成" (shilu.ai translation
  of the Hugging Face blog), sections "一个模型中的三种生成模式" and
  "通过 SGLang 进行部署和推理".
* [Abstract] the arXiv abstract page (aihot.42aifuture), arXiv:2607.05722.

Where the pages leave a step open, the reading taken is named in the function
that takes it (R1..R20 in the design notes use the same numbering).

Pins (tests run with ``-m "not gpu"``) tie every function here to something
other than itself: brute-force masked attention, an independent torch-CPU
textbook forward, RoPE closed forms, a brute-force acceptance loop, the
losslessness of self-speculation against greedy AR (also in mixed AR /
self-speculation steps), KV-rollback equality with an AR cache, the diffusion
threshold edge cases, closed forms of the mode choice by concurrency, and
closed forms plus a textbook replay of the speed-of-light analysis, and the
quadratic self-speculation round against a dense-mask textbook forward of all
its rows plus its losslessness.  Parity unpinned by the pages: the diffusion
trajectory itself for thresholds strictly inside (0, 1), for which the pages
print no worked example, and the quadratic self-speculation layout (reading
R24), which the pages name but do not describe; only its invariants pin it.
"""
from .numerics import round_bf16  # noqa: F401
from .model import OracleModel, Row, KVCache, forward  # noqa: F401
from .sampler import vocab_reduce, commit_set, accept_length  # noqa: F401
from .decode import OracleSession, MODE_AR, MODE_DIFFUSION, MODE_SELFSPEC, MODE_QUADSPEC  # noqa: F401
from .policy import choose_modes, forward_ms, step_rate  # noqa: F401
from .sol import sol_block  # noqa: F401
