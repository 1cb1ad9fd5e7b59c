"""Seeded synthetic workloads (parameter shapes and gradient generators).

Shared by the oracle tests, the GPU tests and the bench. It holds no step of the
bucketed-reduction method itself.
"""
from . import shapes, gen, configs  # noqa: F401
