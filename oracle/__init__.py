"""The CPU oracle of the JEPA ViT encoder forward pass.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import anything from this package.  The HIP library
never calls it, shares no code with it, and fails loudly instead of falling
back to it.

What it computes is the plain definition of the encoder, in float64, on the
stored weights (f32, f16 or bfloat16 widened exactly; q8_0 / q4_0 blocks
dequantized exactly).  The pages never write the network out as equations;
the readings taken where they are silent are listed in each function's
docstring.  The sources followed:
  * LeVJEPA ViT-L/16 model card, opening paragraph: tubelet 1; a mask under
    which a patch token sees its own and earlier temporal slots and never
    the CLS token, while CLS sees every token; the CLS token as the feature.
  * V-JEPA 2 ViT-L/16 SSv2 card, opening paragraph: tubelet 2, 256x256.
  * jepa.cpp Quantization page, "The rule" and "File sizes": the tensor
    schema, which tensors are re-typed, 8.5 / 4.5 bits per weight for
    q8_0 / q4_0; "How the accuracy was measured": the per-token cosine,
    rel_max and rel_fro metrics.
  * LeVJEPA card, "Run it": pooling modes cls / mean / none.

Modules:
  quant    q8_0 / q4_0 quantizer and dequantizer, widening of f16 / bfloat16.
  encoder  normalisation, patchify, LayerNorm, GELU, masked attention, the
           encoder forward and pooling.
  head     the attentive-pool classifier head (V-JEPA 2 SSv2 card).
  metrics  the comparison metrics.
"""
