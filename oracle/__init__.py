"""fp64 CPU oracle for the POET-X linear layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The library (HIP kernels, C ABI,
Python binding) never calls it, and it never calls the library.
"""

from .poetx_oracle import *  # noqa: F401,F403
