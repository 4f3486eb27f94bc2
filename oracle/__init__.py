"""Plain fp64 CPU oracle for the quantized recurrent-state write-back step.

TEST INFRASTRUCTURE, NOT PRODUCT. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package. It
shares no code with the HIP library (no kernels, headers, helpers, tables or
constant generators) and imports nothing from it; both sides consume the seeded
inputs of the stand-alone ``synth`` module.

Every function is written from the pages' definitions in the order they state them,
in float64, with numpy primitives only where a primitive is a single textbook step
(a matrix product, rint, a sort). No blocking, fusion or algebraic re-forming: where
the GPU uses a faster equivalent form (rotated-domain Hadamard rows, a chunked
prefill), this oracle uses the plain definition, so that the equivalence is tested.

Pages cited (title, then the section, paragraph, equation or figure):
  [WB]    "When Quantization Breaks Memory: Recurrent-State Write-Back in
          Low-Precision Temporal Inference" -- English summary page.
  [WB-zh] The Chinese-language summary page of the same paper.
  [LBRS]  "Low-Bit Recurrent States in Hybrid Language Models" -- HTML excerpt of
          the paper (paragraphs between "Related work" and "Limitations").
  [LBRS-x] "Allocate low-bit recurrent state precision by channel decay" --
          explainer of the same paper.
  [DAMP]  Summary page of "DAMP: Decay-Aware Mixed-Precision recurrent-state
          quantization" (arXiv 2608.27513).

Parity unpinned (pinned only by agreement of two independent implementations, or
by nothing beyond a reading of the pages): the clipping-fit tie rule, the greedy
width-adjustment tie rule, the Philox counter mapping of stochastic rounding, the
exact byte packing of every layout, and the chunk-boundary cadence of prefill.
Every other function has a pin in ``tests/test_oracle_*.py``.
"""
