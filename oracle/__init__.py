"""Oracle for the Dual-AR decoder (Fast-AR frame, Slow-AR step) — TEST INFRASTRUCTURE ONLY.

A plain, slow, literal CPU implementation of what the Fast-AR decoder
computes, written from the s2.cpp analysis pages ("Fast-AR codebook decoding
and the generation main loop", sections 1-5; "Overall architecture & Dual-AR
data flow", sections 2-3) and the Mizuoto "Fish Speech" engine page
(section "What matches upstream": float32 RMSNorm, adjacent-pair RoPE with a bf16-rounded
table, the draw argmax(probs / -log u), top-k fixed at 30).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or run anything in this package.  It shares
no code with the HIP path and never imports it; the product path must not
route through it.

Modules:
  fast_ar  - float32 numpy forward (full recompute of every window, no KV
             cache) and the frame decode loop; weight-only int8 matrices
             (one float32 scale per output row) are dequantized first.
  sampler  - the per-request sampler (temperature, top-k, softmax, top-p,
             exponential race with SplitMix64 per-candidate uniforms).
  brute    - an independent float64 scalar-loop forward for small shapes,
             used only to pin ``fast_ar``.
  slow_ar  - the Slow-AR side ("Overall architecture & Dual-AR data flow",
             sections 3-4; main-loop page, sections 5-6): the input combine,
             the cached decode step, prefill, the masked tied head, the
             main-token draw with the repetition check, and the full frame
             (Slow-AR step, then the Fast-AR frame).

Parity status of each function is listed in the module headers.  Nothing
here is "parity unpinned" except the end-to-end logits at the 2560-wide
shape, which no page prints and no trained weights exist for (the same code
is pinned at the small shapes by brute force, library routines and
invariants).
"""
