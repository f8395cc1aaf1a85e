"""CPU oracle for the block-quantised weight x activation products.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links
or executes this package: only the tests, the smoke check of the entry module
and the CPU-baseline leg of the bench may use it.  It shares no code with the
HIP library.

What it computes, in float64, from the canonical GGUF block bytes:

* `quant`  - Q4_0 / Q8_0 block decoding by the block definition, dense
  dequantisation, and the byte image of the library's repacked layout
  written out from that layout's definition.
* `requant` - Q4_1 / Q5_0 / Q5_1 blocks decoded by the public GGUF layouts
  and requantised to Q8_0 in float32 steps (byte-exact reference).
* `ops`    - y = W x (and y += W x), RMSNorm, the fused gate/up SiLU, LM-head argmax
  and LM-head top-k candidates with lowest-index ties, router top-k,
  softmax, the MoE FFN, and the tolerances and argmax / top-k certification
  used by the parity tests.

Pins (tests/test_oracle.py) tie every function to something other than
itself: hand-worked blocks, exact rational brute force, closed forms,
library special cases and invariants.  Parity unpinned: none.
"""
from . import quant, ops, requant  # noqa: F401
