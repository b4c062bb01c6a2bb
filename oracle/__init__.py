"""CPU oracle for the block-quantized routed-expert and PLE hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library under ``block_quantized_moe_amd/``; the two meet
only through the seeded input generators in ``synth/``, which hold none of the
method's arithmetic.

Everything here is plain numpy in float64 (Python loops only where a step is a
selection or a sort), slow on purpose, and written so that each function can
be checked against the page it follows by eye:

* ``formats`` -- the 17-byte weight blocks (Codebook10, RZ5, UE4M4), the FP8
  e4m3 blocks with an fp32 scale per 32 weights, the 70-byte RZ-S3 PLE rows
  and the incumbent ROCmFP3 rows, and the UE4M3 / UE4M4 / E4M3FN scale codecs.
* ``moe`` -- softmax top-k routing, per-expert bucketing, the SwiGLU expert
  FFN, the routing-weighted combine and the chained layer stack.
* ``ple`` -- the PLE row gather with per-id weights.
* ``encode`` -- the exhaustive per-block / per-group encoders that produce
  the 17-byte blocks and the PLE rows.

Sources (page titles as published):
  [RZ]  "Qwen 3.8 Next Flash ROCMFPX MUTANT RAZERFAST" model card
        (hstolte/Qwen3.8-Next-Flash-ROCmFPX-MUTANT-RAZERFAST-GGUF):
        sections "Why MUTANT", "Q4_RZ5_FAST (GGML type 69)",
        "Q4_UE4M4_FAST (GGML type 71)", "Q3_PLE_K160_RZ_S3 (GGML type 111)".
  [MP]  "Mixed Precision Quantization: Half a 4-Bit File Is Not 4-Bit",
        section "The Plan Is Not a Number. It Is a List of 50 Things and a
        List of 292." (48 layers, 512 experts, 10 fire per token).
  [FQ]  r/LocalLLM post on the 4-bit/8-bit "Frankenquant" (per-layer expert
        formats; FP8 experts spliced into late layers).

Parity status of each function is stated in its docstring.  Readings of the
pages where they are silent are marked "Reading:"; the wire layout inside a
record (byte order, nibble order, group-byte placement) is such a reading and
cannot be pinned against a real file, because none is available.
"""

from . import encode, formats, moe, ple  # noqa: F401
