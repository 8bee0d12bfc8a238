"""CPU oracle for the FP8 MoE prefill path -- test infrastructure only.

This package is a plain, slow, obviously-correct NumPy (float64) statement of what the
FP8 grouped-expert prefill path computes. It exists to check the HIP library, never to
stand in for it: only the test suite, the smoke check and the bench's CPU-baseline leg
may import it. It shares no code with the GPU path (``fp8_moe_prefill_amd``), and it
imports nothing from there; both sides receive their inputs from ``synth``.

Sources (cited by page title and section in each function):

* "FP8 grouped-expert prefill with on-chip int4-to-e4m3 dequant" (octopusresearch.org),
  section 1 Contribution -- the method: FP8 e4m3 dense q/k/v/o projections, one grouped
  expert GEMM per layer instead of per-token dispatch, int4 weights turned into e4m3
  without unpacking the resident bank, one dynamic activation scale per token and K group
  applied inside the fp32 accumulation; sections 3-4 -- the logit-cosine parity gate.
* FreeToken PR #389 "load-time per-tensor FP8 dense projections (W8A8 via _scaled_mm)",
  sections "What this adds", "Limits", "Testing" -- per-tensor e4m3 weights with one
  fp32 scale, a dynamic per-tensor activation scale, the zero-input scale floor.
* memra-engine ``fp8_ffi`` module docs (docs.rs), module text and ``Fp8Scratch`` -- the
  activation scale is amax/448 (so the format is OCP e4m3fn, max 448); the scale block
  holds amax, the quantising multiplier and the folded scale.

Where the pages are silent the plainest reading is taken; each such reading is named
in the docstring of the function that makes it.

Parity status: every function here is pinned by a ``-m "not gpu"`` test against closed
forms, brute force, library routines or invariants (see ``tests/test_oracle_*.py``),
except where a docstring says "parity unpinned".
"""
