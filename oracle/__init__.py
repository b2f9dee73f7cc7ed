"""CPU oracle for the resident-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy float64 definition of what the layer
computes, step by step, following the TideLM README's "How adaptive expert
loading works" section (items 1-3) and the colibri cluster page's wire-protocol
paragraphs (rows named by index; replies added in a fixed order).  It shares no
code with the GPU path or with the input generators' weight packer: it decodes
packed bytes with its own decoder and quantises activations with its own
encoder.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product path never calls it.

Parity status per function (pins live in tests/test_oracle_*.py):
  mxfp4.decode / mxfp4.encode     pinned (exhaustive closed form, hand-worked golden blocks)
  mxfp6.decode / mxfp6.encode     pinned (exhaustive table, hand-worked packing and ties, brute force)
  moe.router_logits               pinned (correctly rounded fsum on small shapes)
  moe.softmax / moe.renormalise   pinned (sums, closed forms, k=1)
  moe.topk / moe.masked_topk      pinned (brute force; literal miss-replacement procedure)
  moe.demand                      pinned (sum and mask-independence invariants)
  moe.bucket                      pinned (bijection, counts, stable order)
  moe.expert_ffn                  pinned (scalar-loop brute force, textbook SwiGLU cases)
  moe.combine                     pinned (identical-experts invariant)
  plan.hot_read / plan.replan     pinned (constructed cases, brute force)
  softmax router, bias placement, score used for demand, activation format,
  SwiGLU form: parity unpinned by the pages (fixed by the readings recorded in
  the design notes).
"""
from . import mxfp4, mxfp6, moe, plan  # noqa: F401
