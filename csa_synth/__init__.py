"""Seeded synthetic inputs for the CSA / HCA path (shared by tests, bench and smoke).

This package only draws random numbers and lays them out in the storage
formats the library takes.  It holds none of the method's arithmetic (no
pooling, no scoring, no selection, no attention), so the oracle and the GPU
library can both be fed from it without sharing code.
"""
from .gen import *  # noqa: F401,F403
