"""CPU oracle of the DFlash block draft-and-verify step (test infrastructure).

Only tests, the smoke check and the bench's CPU-baseline leg import this package.
The HIP library and its Python binding never import it, and it imports nothing
from them; the two share only the seeded input generators.
"""
from . import dflash_oracle, bruteforce  # noqa: F401
