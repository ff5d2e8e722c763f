"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

Holds input generation only (lengths, page assignment, tensor values); none of
the attention method's arithmetic lives here.
"""
from . import rng, workloads  # noqa: F401
