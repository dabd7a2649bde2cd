"""MI355X-native trellis-coded (eschamoe) MoE expert path.

``escha`` is the Python binding over the C-ABI library ``libescha.so``
(hand-written HIP kernels for gfx950). ``synth`` builds seeded synthetic
inputs. Importing the package loads nothing; ``escha`` raises if the HIP
library is missing.
"""
__all__ = ["escha", "synth"]
