"""CPU oracle for the LoRA / QLoRA adapted linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain reference that the
HIP library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the library itself
never does, and it never imports the library.  It shares no code, header,
table or constant generator with the HIP path: the NF4 codebook, thresholds
and every formula below are derived here on their own.

Sources (web pages on LoRA / QLoRA, cited by title and section):

* "Low-Rank Adaptation (LoRA) and QLoRA: Mathematical Foundations, Intrinsic
  Rank Dynamics, NF4 Quantization, and Parameter-Efficient Fine-Tuning"
  (llms.blog) -- forward pass, gradients, NF4 levels, block absmax, double
  quantization, static merge, segmented multi-adapter serving.
* "Large Language Model Fine-tuning and LoRA" (aicomputerinstitute.com) --
  NF4 block size 64, DQ block size 256, storage rates, trainable-parameter
  formula and calculator, merge FLOP count, multi-tenant serving.
* "LoRA and QLoRA fine-tuning under the hood" (codingpancake.com) and
  "LLMs part 08: Parameter-Efficient Fine-Tuning" (shakilmahmud.com) and
  "Lesson 26: LoRA / QLoRA theory" (teology.holyping.network) -- the same
  forward / merge formulas and the B = 0 initialisation.

Precision: LoRA products are computed in float64 from the exact values the
device receives; the NF4 codec is computed in float32 with one IEEE rounding
per operation, because its integer outputs (codes, 8-bit constants) are
decided by float32 comparisons and roundings on both sides.

Modules:
    nf4   -- codebook, quantize / dequantize with double quantization
    lora  -- forward, backward, merge, segmented multi-adapter forward
             (uniform or per-adapter ranks and scales), LoRA-input dropout,
             DoRA forward and backward, trainable-parameter counts
    optim -- AdamW step on the adapter factors (float32 master, m, v)

Parity unpinned: none of the functions here is without a pin; what pins
each one is listed in the test files under ``tests/`` (``test_oracle_*``).
The NF4 codebook's truncation constant and the 8-bit integer format of the
second-level constants are readings of the pages (see the ``nf4`` module
docstring); they are pinned to the pages' properties, not to an external
NF4 implementation, which none of the pages prints.
"""
from . import lora, nf4, optim  # noqa: F401
