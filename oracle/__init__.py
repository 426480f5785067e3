"""CPU oracle for the post-router MoE layer (test infrastructure only).

Imported by tests/, the package's smoke() entry and the benchmark's
cpu_baseline leg; never by the HIP library or its Python binding.
"""
from .moe_oracle import *  # noqa: F401,F403
