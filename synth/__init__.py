"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This package holds input generation only: shapes, seeds and value
distributions.  It contains none of the method's arithmetic (no absmax, no
scale, no quantization, no contraction, no epilogue, no hash) and imports
neither ``oracle`` nor ``int8_gemm_amd``.
"""
from .inputs import *  # noqa: F401,F403
