"""Plain fp64 CPU oracle for the SparsePR attention call.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP implementation.
"""
from .sparsepr_oracle import *  # noqa: F401,F403
