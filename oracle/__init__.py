"""CPU oracle for the DiffusionGemma parallel dense-MLP + routed-MoE FFN block.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything in this package; only the test
suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of the
bench do.  The oracle shares no code with the GPU path.

Everything here is plain numpy in float64, except the two decisions that turn a
float into an integer and that the GPU must reproduce bit-exactly: the affine
quantiser's codes and the nvfp4 quantiser's codes and scale bytes (taken in
float32, the precision the kernels use) and nothing else.  Router top-k is taken on float64 logits; positions whose k-th/(k+1)-th
logit margin is below 1e-4 are the only ones where a float32 GPU may pick a
different set, and the parity tests excuse exactly those.

Modules:
  quant  -- affine group-64 / group-32 quantiser, the q4/q4g32/q8 byte
            layouts, dequantisation
  fp4    -- the nvfp4 expert format: E2M1 codes, E4M3 block scales, a tensor
            scale; its quantiser, layout and exact dequantisation
  block  -- RMSNorm, router, GeGLU MLP, the parallel dense + MoE block
  head   -- the tied embedding table at both ends of a forward: the
            self-conditioned canvas input and the tail (final norm, tied head,
            softcap, temperature, entropy / argmax / softmax normalisers)
  attention -- the denoise attention of one layer: QK-norm, weightless
            V-norm, split-half RoPE (full or partial), unit scale, the
            canvas over [committed window | canvas]

Sources (the web pages this method is described on):
  [ARCH]  "diffgemma -- architecture & implemented contract", Part II
          section 2.1 "Forward-pass details" (Norms; MoE order), section 1
          "Model constants", Part III "Precision policy" and
          "Standing design decisions".
  [BLOG]  "DiffusionGemma Explained" (ML@Berkeley), sections "RMSNorm" and
          "MLP and mixture-of-experts block" (classes MLP and MOEBlock), and
          "Complete DiffusionGemma model" (the layer_scalar multiply).
  [PORT]  mlx-bun "DiffusionGemma port -- plan & parity strategy", Reference
          dossier D0 section 1 "Weight schema & quant map" and section 2
          "Decoder architecture" (DecoderLayer, MLP, Router, Experts).
  [GGUF]  "Independent GGUF Forward Pass and Bit-Identical Cross-Backend
          Consistency for a 26B Text-Diffusion Model", section 4, facts 6, 7, 9.

Parity status per function is stated in each docstring; every function here is
pinned by a CPU test in tests/test_oracle_*.py except where a docstring says
"parity unpinned".
"""
