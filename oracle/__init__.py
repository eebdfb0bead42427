"""CPU oracle for the FlashAttention forward pass.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``flashattention_forward_amd`` never imports, links or runs anything here,
and this package imports nothing from it: the two share no code.

Everything is plain numpy in fp64 (exact integer arithmetic for the
quantised scores), evaluated the obvious way so a reader can check it
against the sources by eye.

Sources, cited by short name in the modules:
  [trading post]  "Can a full trading day of context beat one minute? Flash
                  attention and the sequence-length question" (marketmaker.cc
                  blog, Thai edition) -- sections "Why attention is bound to
                  memory", "The Flash Attention algorithm", "The online softmax
                  recurrence", "Backward: recompute instead of store",
                  "FA2", "Causal masking", "Integration in eight lines",
                  "Validation".
  [FA4 post]      "FlashAttention 4: fast, memory-efficient attention for LLMs"
                  (linux-konsole.com, Vietnamese) -- "Introduction", "Why
                  attention kernels still dominate".
  [INT-FA post]   "INT-FlashAttention: an INT8 quantisation architecture
                  compatible with FlashAttention" (hoodcat.net, Spanish).
  [FP4 summary]   summary of "Hardware-Aware FP4 FlashAttention-4"
                  (gist.science, Chinese) -- summary and explainer.

Modules:
  attention   -- the plain definition (two-pass softmax, fp64).
  recurrence  -- the tiled online-softmax recurrence exactly as the trading
                 post's algorithm section states it, plus the merge of
                 partial states over disjoint key ranges.
  quant       -- int8 per-token and OCP e4m3 quantisation emulation and the
                 quantised-attention oracle.
  backward    -- the gradients dQ, dK, dV of attention by the chain rule
                 through the plain definition.
  variants    -- grouped-query heads (GQA/MQA) and packed variable-length
                 batches, by head mapping and slicing of the definition.
  rotated     -- FP8 attention with Q and K rotated by a random-sign Hadamard
                 matrix before block quantisation ([trading post], "FA3:
                 Hopper mechanisms", FP8 with incoherent processing).
  fp4         -- the same FP8 attention with P in MXFP4 (E2M1 codes, one
                 power-of-two scale per 32 keys of a row) ([FP4 summary]).

Parity status of every function is stated in its module header.
"""
from . import attention, backward, fp4, quant, recurrence, rotated, variants  # noqa: F401
