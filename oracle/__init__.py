"""CPU oracle for exact tiled attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the bench's CPU-baseline leg may import this
package.  The product path (the HIP library and its Python binding) never imports, calls or links
anything here, and this package imports nothing from the product.

What it computes, in float64 on the CPU, straight from the definitions:

* ``attention_ref`` / ``attention_rows`` — scaled-dot-product attention softmax(scale*Q*K^T [+ causal
  mask]) * V and the row log-sum-exp, with full score rows (no key tiling, no running maximum).
  The pages say the tiled method returns the same output as this plain softmax formula
  (FlashAttention 2 + 3 — speicherbewusste Attention-Kernels, "Kernpunkte" and "Worum es geht";
  Flash Attention glossary, "/01 Was ist Flash Attention?").
* ``attention_probs`` — the score and probability matrices of one head, as the unfused comparison path
  holds them in memory.
* ``attention_rect`` — the same definition for Nq queries against Nk keys, the queries sitting at
  positions q_start .. q_start + Nq - 1 of the key sequence for the causal mask (default: the last Nq
  positions, the decode shape; a middle range is one GPU's share of a sequence-sharded forward).
* ``attention_bwd_ref`` / ``attention_bwd_rows`` — the gradients dQ, dK, dV of that definition for a
  given output gradient dO (the pages name the backward pass but do not write it out; the derivative
  of the definition is the plain result the kernels must reproduce).
* ``fp8`` — the OCP e4m3 codec, the Sylvester Walsh-Hadamard transform and the per-block absmax
  quantisation of the FP8 path (FlashAttention-3 article, "Drei technische Hebel", item 3
  "FP8-Blockquantisierung"; concept card, "Kernpunkte", FP8 with absmax scaling).

Pins (tests marked ``not gpu``): brute force with ``math.fsum`` on tiny inputs, torch's float64
CPU scaled_dot_product_attention and scipy's logsumexp/hadamard as independent library routines,
central finite differences and torch autograd for the gradients,
closed forms (Q = 0, constant V, causal row 0, two keys), invariances (joint key/value permutation,
per-row score shift), and torch's float8_e4m3fn conversion for the codec.  No function here is
"parity unpinned".
"""

from .attention import (  # noqa: F401
    attention_bwd_ref,
    attention_bwd_rows,
    attention_probs,
    attention_rect,
    attention_ref,
    attention_rows,
)
from .fp8 import (  # noqa: F401
    E4M3_MAX,
    dequantize_blocks,
    e4m3_decode,
    e4m3_encode,
    fp8_prep_ref,
    fwht_f32,
    fp8_attention_ref,
)
