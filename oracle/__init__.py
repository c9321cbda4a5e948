"""CPU oracle for the online-quantized W8A8 / W4A8 linear layer.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. The HIP library and its
Python binding never import it, and the two share no code.

`cider_oracle` is the vectorised numpy oracle; `brute` is an independent
exact-rational brute force used to pin it on tiny inputs.
"""
from . import brute, cider_oracle  # noqa: F401
from .cider_oracle import *  # noqa: F401,F403
