"""fp64 CPU oracle for block-sparse top-k attention.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the bench's
CPU-baseline leg may import it. It shares no code with the HIP path.
"""
from .bsattn_oracle import *  # noqa: F401,F403
