"""ORACLE — plain, slow CPU implementation of the MoE expert-offload layer.

Test infrastructure only: ``tests/``, the smoke check in ``__graft_entry__`` and
the CPU-baseline leg of ``bench.py`` may import it. The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes, and the passage each part follows (pages: "FreeToken:
Efficient Edge-Native MoE Serving with Bandwidth-Adaptive Execution", as
explained on papers.ananclaw.com, zhichai.net and juejin.cn):

* ``router``    — fp32 router logits in a fixed order, top-k, softmax weights.
* ``formats``   — fp32 / bf16 / MXFP4 / NVFP4 / FP8 expert-block decoding
                  (juejin.cn overview, section 5, the format list; zhichai.net
                  article, section 5).
* ``moe``       — SwiGLU expert FFN in fp64 and the weighted layer output,
                  plus a brute-force dense evaluation used to pin it.
* ``residency`` — the global LRU expert cache and the bandwidth-ratio miss
                  split q* = m * B_P / B_H (zhichai.net article, section 2,
                  the Decode and LRU paragraphs).
* ``streaming`` — the full-layer double-buffered prefill timing model
                  (zhichai.net article, section 2, the Prefill paragraph).

Readings of points the pages leave open are listed in each module's header.
"""
from . import formats, moe, residency, router, streaming  # noqa: F401
