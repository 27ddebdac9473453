"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

This package draws random numbers and lays them out; it holds none of the
drafting method's arithmetic (no norms, projections, attention or argmax).
"""
from .inputs import *  # noqa: F401,F403
