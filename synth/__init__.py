"""Seeded synthetic workloads: parameter-shape lists and random draws.

Shared by the CPU oracle side and the GPU side; holds none of the update's
arithmetic.
"""
from . import gen, shapes  # noqa: F401
