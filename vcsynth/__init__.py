"""Seeded synthetic inputs for the draft/verify attention workloads.

This package is the only code shared by the product path and the oracle: it draws numbers
(counter-based, layout-independent) and describes the five workloads.  It performs none of
the method's arithmetic.
"""
from . import rng, configs  # noqa: F401
from .normal_table import normal_table  # noqa: F401
