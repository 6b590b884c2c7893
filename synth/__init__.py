"""Seeded synthetic inputs shared by the oracle (tests) and the HIP path.

This package draws random numbers and stores them in the storage dtypes the
method uses (bf16/fp16 bit patterns, packed int4 words).  It holds none of the
method's arithmetic: no dequantisation, GEMV, routing, activation or LoRA math.
"""
from .gen import *  # noqa: F401,F403
