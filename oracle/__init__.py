"""CPU oracle for PagedAttention decode: test infrastructure only.

Imported by tests/, by the smoke check and by the benchmark's CPU-baseline leg;
never by the library or its binding.
"""
from .pa_oracle import *  # noqa: F401,F403
