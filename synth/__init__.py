"""Seeded synthetic inputs (generator G) shared by the oracle and the HIP path."""
from .gen import *  # noqa: F401,F403
