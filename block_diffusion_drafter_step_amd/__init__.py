"""MI355X-native DFlash / DFlash2 draft block step.

The compute lives in the HIP library ``libdflash.so`` (C-ABI, declared in
``include/dflash.h``); ``block_diffusion_drafter_step_amd.dflash`` is the thin
Python binding over it.  Importing the package loads nothing; the binding
loads the library on first use and raises if it is missing.
"""
