"""Float64 CPU oracle for MLA paged latent decode -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  It shares no code with the GPU library.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import __all__  # noqa: F401
