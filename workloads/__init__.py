"""Seeded synthetic inputs for KDA prefill (shared by the oracle-side tests and the GPU path).

This package draws random numbers and lays them out; it holds none of the
method's arithmetic (no normalisation, no decay, no recurrence).
"""
from .gen import *  # noqa: F401,F403
