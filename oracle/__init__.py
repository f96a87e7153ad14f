"""CPU oracle for the rotation + low-bit KV-cache codec.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the package smoke
check and the bench's CPU-baseline leg may import or call anything in this
package; the GPU library never does, and shares no code, table or constant
generator with it.

Everything here is plain, slow and meant to be checked by eye against the
pages: numpy in float64, one function per step of the method, each step citing
the passage it follows.  Steps the pages leave open take the reading stated in
the docstring of the function that implements them.

Page short names used in citations:

* "RoPE-KV page"  -- RoPE-inspired KV-cache compression (jsqmd.com news 754920).
* "EliteKV page"  -- EliteKV: RoPE frequency selection and low-rank projection.
* "IsoQuant page" -- KV-cache compression: IsoQuant in large language models
                     (jsqmd.com news 793725).
* "RotateKV page" -- RotateKV: accurate and robust 2-bit KV cache quantization
                     via outlier-aware adaptive rotations (arXiv 2501.16383).

Parity pins: every function is pinned by a CPU test against something other
than itself (closed forms, library routines, brute force, textbook values);
see the tests named ``test_oracle_*``.
"""
from .codec import CodecParams, append, decode, encode, widen  # noqa: F401
from .attention import attend, attend_decoded  # noqa: F401
from .lloyd import fit_gaussian  # noqa: F401
