"""Plain fp64 CPU oracle for the SimSD verification pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and it never imports that
library.

What it computes, and where the method is defined (page "SimSD - Simple
Speculative Decoding in Diffusion Language Models", gist.science summary):

* ``attention``  -- the single verification forward's attention: a paired
  data section D and mask section D~ after the prompt (section 1, input
  layout), the token-level temporal mask driven by the stage map tau
  (section 2), and RoPE copy, where D~_k reuses D_k's position (section 3).
* ``acceptance`` -- standard rejection sampling walked in the drafted
  temporal order, committing the longest accepted prefix (section 4,
  pipeline, "acceptance" bullet).
* ``philox``     -- the Philox4x64-10 counter-based generator of Salmon et
  al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11), which the
  acceptance walk draws its uniforms from.

Every function is the plain definition written out in float64; see each
module's header for its pins (the tests that tie it to something other than
itself).  No function here is "parity unpinned".
"""

from .attention import (  # noqa: F401
    MASK_FULL,
    MASK_TEMPORAL,
    block_visibility,
    rope_rotate,
    verify_attn_ref,
    verify_status_ref,
)
from .acceptance import accept_ref, accept_status_ref  # noqa: F401
from .philox import philox4x64_10, uniform24, uniform53  # noqa: F401
