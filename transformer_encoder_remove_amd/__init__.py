"""MI355X-native Transformer encoder-layer forward with padding removal.

The compute lives in libtel.so (HIP kernels for gfx950, C ABI in include/tel.h); this
package is its Python binding (``binding``) and its build script (``build``).
Importing the package raises ImportError when the library has not been built.
"""
from .binding import *  # noqa: F401,F403
from .binding import lib, LIB_PATH, EXPORTS, TelError  # noqa: F401
