"""MI355X-native Psi-Spec draft-and-verify decode step (diffusion-augmented LLMs, Uno).

The compute lives in ``libuno.so`` (HIP, gfx950) behind the C ABI of
``include/uno.h``; ``diffusion_drafted_lora_amd.uno`` is the ctypes binding.
Importing this package loads nothing; the binding loads the library on first use
and raises if it is missing.
"""
from . import configs  # noqa: F401

__all__ = ["configs"]
