"""Float64 CPU oracle for the LiftQuant layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg; the product path never imports it and it never
imports the product package.
"""
from .lq_oracle import *  # noqa: F401,F403
from .lq_oracle import __all__  # noqa: F401
