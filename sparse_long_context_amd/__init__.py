"""MI355X-native Lighthouse Attention layer.

The layer's stages run as hand-written HIP kernels for gfx950 behind the
C-ABI library liblighthouse.so (declared in include/lighthouse.h).  This
package holds the library sources (csrc/), its build step, the ctypes
binding and the autograd wrapper.  Importing the package does not load the
library; `lib()` does, and raises if it is missing.
"""
from ._lib import lib, LighthouseError  # noqa: F401
