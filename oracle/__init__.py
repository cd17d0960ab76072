"""fp64 CPU oracle for BAM attention.  TEST INFRASTRUCTURE ONLY.

Imported only by tests/, the package smoke check and the benchmark's CPU-baseline
leg.  The HIP product path never imports, links or executes anything here.
"""
from .bam_oracle import *  # noqa: F401,F403
from .bam_oracle import PreconditionError  # noqa: F401
