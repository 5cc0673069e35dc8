"""CPU oracle for INT4 KV-cache quantize-append and regional INT4/INT8 decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the GPU library is checked against.  Only the test suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the HIP library and its Python binding) never does, and shares
no code, table or constant with it.

What it computes, and where each step comes from:

* rotation -- block-diagonal Sylvester-Hadamard of block size h applied to each
  key vector, queries rotated the same way (SAW-INT4, section 2 "Block-Diagonal
  Hadamard Rotatie"; KV4-RL, "Methodology in Plain English": keys stored in a
  Hadamard-rotated basis, queries rotated to match);
* quantization -- one affine group per 128-dim token-head vector with an FP16
  scale and FP16 offset, INT4 for the main cache and INT8 for the side cache
  (KV4-RL, "Methodology in Plain English" and "Key Contributions" item 4);
* regions -- the first s positions and the most recent w positions live in the
  INT8 side cache, everything else is attended from INT4; the two disjoint
  regions are merged through softmax statistics (KV4-RL, "Key Contributions"
  item 4 and "Methodology in Plain English");
* attention -- exact softmax attention in fp64 over the dequantized cache.

Parity status of each function is listed in the module that defines it; every
function here is pinned by tests under ``tests/`` against closed forms,
library routines or brute force; none is "parity unpinned".
"""

from . import numerics, hadamard, quant, regions, attention, cache  # noqa: F401
