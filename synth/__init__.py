"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and by the oracle."""
from .inputs import *  # noqa: F401,F403
