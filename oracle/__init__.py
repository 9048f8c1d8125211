"""CPU oracle for DiT joint self-attention. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product library never calls it, and it shares no
code with the HIP path: the two meet only through the seeded inputs of
``dit_workloads``.

What it computes, in float64, as the plain definition with no tiling:

* RoPE (``oracle.rope``): multi-axis rotary position embedding on Q and K.
  The source pages never write RoPE out. The xDiT paper (catalogue page,
  abstract) and the AMD RDNA 4 xDiT blog (section "Understanding the Inference
  Pipeline") describe DiTs that attend over text and patchified-latent tokens.
  Axis layout, pairing and frequencies follow the readings listed in the
  design notes: interleaved pairs (2i, 2i+1), per-axis frequencies
  theta^(-2i/d_a), and text tokens at position 0.
* Attention (``oracle.attention``): non-causal softmax(s * Q K^T) V over the
  whole joint sequence, with s = 1/sqrt(D) unless given. The formula is the
  one in "Attention Is All You Need" and FlashAttention-2, both in the xDiT
  paper's reference list (catalogue page, "Other references"). The joint
  text+image sequence is the one the xDiT abstract describes as growing with
  resolution.
* Ring blocks (``oracle.ring``): attention of a query shard over one key/value
  block with the row log-sum-exp, and the exact merge of two such partial
  results (ring attention, in the same reference list).
* MXFP4 (``oracle.mx``): OCP MX quantisation and the block-scaled linear
  layer (MXFP4/Quark on MI350 blog).
* DBCache (``oracle.dbcache``): the relative L1 residual difference and the
  reuse decision against the threshold (RDNA 4 xDiT blog, step caching).
* ``oracle.brute``: the same steps as pure-Python scalar loops, used to pin
  the numpy version on tiny inputs.

Every function is pinned by the CPU tests against something other than
itself: brute force, torch's float64 SDPA, a complex-number RoPE, closed
forms and invariants.
"""
from .rope import rope_angles, rope_apply
from .attention import attention, joint_attention, softmax_probs, lse
from .ring import block_attention, merge_lse

__all__ = ["rope_angles", "rope_apply", "attention", "joint_attention", "softmax_probs", "lse", "block_attention",
           "merge_lse"]
