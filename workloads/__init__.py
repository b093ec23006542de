"""Seeded synthetic workloads shared by the CPU oracle's tests and the GPU path.

This package holds random draws, their shapes and the configuration table only.
No step of the quantizer or of the inner-product estimator lives here.
"""
from .gen import *  # noqa: F401,F403
