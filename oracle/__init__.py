"""CPU oracle for Positional-LSH ALiBi attention.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, links or executes anything
here, and this package imports nothing from the product path.
"""

from .plsh_oracle import *  # noqa: F401,F403
