"""Seeded synthetic workloads shared by the oracle and the product.

Holds shapes, page sizes and random draws only; none of the method's
arithmetic lives here.
"""
from .configs import CONFIGS, MoEConfig, ViewSpec  # noqa: F401
from . import gen  # noqa: F401
