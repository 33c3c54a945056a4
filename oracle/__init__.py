"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or runs anything here, and this package
imports nothing from the product.

Modules
  attention       materialised forward / analytic backward (the definition)
  tiled           block-by-block forward and backward in the pages' step order,
                  used only to test that tiling does not change the result
  online_softmax  the single-row running state (m, l, a) and its block ledger
  decode          one query token per sequence against a KV cache (definition),
                  and the pages' split-KV merge, used only to pin that rule
  fp8             E4M3 encoding, per-block quantization, the FP8 attention
                  reference (exact attention on dequantized inputs) and its
                  error bound

Every function says which passage of the source pages it follows.  Pages:
  [P1] "解析 FlashAttention（4）：FlashAttention-v2" (my-webpage-adu.pages.dev)
  [P2] FlashAttention-1 notes, BHHXX's Blog (bhhxx.wiki)
  [P3] "分块 Attention：重建概率，累计梯度" (glenzli.com, attention-kernels)
  [P4] Chapter 18 "FlashAttention" of an AI-algorithms book (theaiera.top)
"""
from . import attention, decode, fp8, online_softmax, tiled  # noqa: F401
