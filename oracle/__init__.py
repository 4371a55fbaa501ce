"""CPU oracle for the DFlash / DFlash2 draft block step (test infrastructure).

Plain, slow, fp64 numpy code that states what each call of the library
computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the library never does, and it imports nothing from the
library.
"""
from .dflash_oracle import *  # noqa: F401,F403
