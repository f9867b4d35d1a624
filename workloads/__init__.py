"""Seeded synthetic inputs shared by the oracle-side tests and the GPU-side tests/bench."""
from .synth import *  # noqa: F401,F403
