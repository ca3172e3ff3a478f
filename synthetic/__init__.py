"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This package holds no quantization arithmetic: it only draws random tensors and rounds them to
BF16. The same bytes are fed to the GPU library and to the CPU oracle.
"""
from .workloads import *  # noqa: F401,F403
