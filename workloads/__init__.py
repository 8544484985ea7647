"""Seeded synthetic inputs for paged decode attention.

This package draws random numbers and describes sequence set-ups; it holds none
of the method's arithmetic (no slot or table computation, no attention).  Both
the CPU oracle and the HIP path consume what it produces.
"""
from .configs import Case, make_case, CONFIG_NAMES, small_case  # noqa: F401
