"""Plain fp64 CPU oracle for the multi-tenant LoRA layer over a low-precision base GEMM.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the ``precision_gemm_amd``
package and its HIP library) imports, calls or links this package; only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code, tables or helpers with the GPU path.

What it computes (cited by page title and passage):

* "Punica: Serving multiple LoRA finetuned LLM as one" (GitHub README, Overview):
  with W of shape [H1, H2], A of shape [H1, r] and B of shape [r, H2], a LoRA'd
  layer computes y = x@(W + A@B) = x@W + x@A@B; for a batch X = (x1, ..., xn)
  whose parts map to n LoRA models, Y = X@W + (x1@A1@B1, ..., xn@An@Bn).  The
  grouping of the batch by model is what the README calls "Segmented" in SGMV.
* "EpiLoRA" abstract: the base GEMM runs in a low-precision format (FP8 or 4-bit
  weights); the adapter's down-projection feeds only the GEMM's epilogue, which adds
  every tenant's up-projection before the output is written.

Modules:

* ``codecs``   -- e4m3fn, e2m1, e8m0 and bf16 decoders/encoders written from the
  format definitions (OCP 8-bit floating point spec; OCP Microscaling Formats v1.0).
* ``mxquant``  -- MXFP8 quantisation of the bf16 activations (32-element K-blocks).
* ``segments`` -- grouping of tokens by adapter: CSR offsets and a stable order.
* ``layer``    -- the unfused layer in fp64: dequantised base GEMM plus per-segment
  LoRA terms, with a run-time exactness guard on the base sum.

Every function is pinned by ``tests/test_oracle_*.py`` against facts fixed by the
pages and by the mathematics (exhaustive code tables, closed forms, invariants,
brute force with exact rationals); see the docstrings for which pin covers what.
"""

from . import codecs, mxquant, segments, layer  # noqa: F401
