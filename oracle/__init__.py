"""fp64 CPU checker for the spatiotemporal self-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke entry point
and the benchmark's CPU-baseline leg use it.  It shares no code, tables or
constants with the HIP library and does not import that package.

Contents
--------
``oracle.attention``  the plain definition O = softmax(scale * Q K^T) V in
                      fp64 (row-blocked, row-sampled), a pure-Python
                      brute force for tiny cases, and the masked variants.
``oracle.fp8``        an E4M3 encoder/decoder written from the format's
                      definition, the fp8 pre-pass (quantise + smooth) in
                      the precision the kernels take their decisions in, and
                      the fp64 quantisation model of the fp8 attention.

Every function cites the passage of the pages it follows.  Functions that no
test pins to something outside this package are marked "parity unpinned" in
their docstring; at present there are none.
"""

from . import attention, fp8  # noqa: F401
