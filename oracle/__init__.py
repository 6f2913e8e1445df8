"""fp64 CPU oracle of the ButterflyMoE expert layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the HIP library never does.
"""
from . import ref  # noqa: F401
