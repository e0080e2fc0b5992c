"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This package draws random numbers and describes shapes.  It holds none of the
method's arithmetic (no truncation, no lens rules, no products), so both the
CPU oracle and the HIP library can consume what it produces without sharing
code with each other.
"""

from .synth import *  # noqa: F401,F403
