"""Layer-sliding fine-tuning step for MI355X (gfx950).

The library (libsf.so, built in-tree by ``build.py``) holds every kernel and
the sliding engine behind a C ABI (``include/sf.h``); ``sf`` is its ctypes
binding and ``runtime`` the torch-side buffer plumbing.  Importing this
package does not load the library; ``sf.load()`` does, and raises if it has
not been built -- there is no fallback path.
"""

from . import sf  # noqa: F401
