"""CPU oracle for the paged decode / prefill path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy restatement of what the path computes, written
from the pages of the code series "An Inference Engine in 1,500 Lines of
CUDA: The Map" (jaehun.me, English page and its Korean original) and the
public definitions those pages name (PagedAttention, online softmax, GQA,
Llama-3-scaled RoPE).  It exists so that tests, the smoke check and the
bench's CPU baseline can compare the HIP kernels against something obviously
correct.  Nothing in the product imports it; it imports nothing from the
product.

Modules:
  bf16       -- decoding bfloat16 bit patterns to float64, float64 -> bf16 RNE
  rope       -- Llama-3 frequency scaling and the half-split rotation
  paging     -- append, gather and block-allocation validity through a block table
  attention  -- single-query decode attention and causal prefill attention,
                two-pass softmax in float64
  layer      -- the rest of a Llama decode layer around the attention:
                RMSNorm, projections, gated SiLU MLP, residual adds

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: library routines (torch's float64 scaled_dot_product_attention,
transformers' Llama-3 RoPE parameters and rotate-half, transformers' Llama
RMSNorm, MLP and decoder layer), closed forms,
invariants, brute force and the constants the pages print.
"""
from . import bf16, rope, paging, attention, layer  # noqa: F401
