"""CPU oracle for the MXFP8 block-scaled grouped MLP.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (``mxfp8_block_scaled_mx_amd``) never does: it fails
loudly when its HIP library is missing instead of falling back here.

The oracle is plain numpy in float64 (exact integer bit operations where the
method defines an integer result).  It shares no code, table or constant
generator with the HIP path.  Every function cites the passage it follows.
Pages cited:

* "Efficient MoE training for biological foundation models" (bpdata news
  article on the BioNeMo MoE recipe), section "Key technical approaches in the
  recipe", items 1) fragmented expert kernels (GroupedLinear over per-expert
  split_sizes), 2) model size and activation memory (MXFP8: one scaling factor
  per block of 32 consecutive values, 8 bits per value) and 3) quantization
  overhead (GroupedLinear -> ScaledSwiGLU -> GroupedLinear with routing-weight
  scaling, a fused forward and a corresponding fused backward op, 16-bit master
  weights quantized each step).
* "TransformerEngine-accelerated Llama 3 training with native PyTorch training
  loop" (BioNeMo recipes docs), section "MXFP8 vs BF16 throughput on
  Llama-3.1": the recipe is MXFP8BlockScaling with E4M3 elements.

What the pages leave open is fixed by the readings listed in this package's
module ``mx_oracle`` (exponent rule floor(log2 amax) - 8, saturating
round-to-nearest-even, layouts, SwiGLU halves, backward dataflow).
"""
from .mx_oracle import *  # noqa: F401,F403
