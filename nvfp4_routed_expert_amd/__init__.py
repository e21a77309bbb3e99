"""NVFP4 routed-expert (MoE) FFN for MI355X (gfx950).

The computation lives in the HIP library ``libnvfp4moe.so`` (C ABI in
``include/nvfp4moe.h``); ``native`` is its thin Python binding, ``synth``
draws the seeded synthetic inputs and ``weights`` prepares NVFP4 expert
weights on the device.  Importing the package loads nothing; the first
library call loads the library and raises if it is not built.
"""
__all__ = ["native", "synth", "weights", "build"]
