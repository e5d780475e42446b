"""ric: ragged input compilation for MI355X (gfx950).

The product is the C-ABI library ``libric.so`` (declared in ``include/ric.h``),
built in-tree by ``python -m ragged_input_compilation_amd.build``.  The Python
side is a thin ctypes binding (``_ric``) plus a step driver (``runner``) that
allocates device memory and streams with PyTorch and calls the library.
Importing ``_ric`` fails loudly when the library has not been built: there is no
fallback implementation."""
import importlib

__all__ = ["ric", "runner"]

_LAZY = {"ric": "._ric", "runner": ".runner"}


def __getattr__(name):
    if name in _LAZY:
        return importlib.import_module(_LAZY[name], __name__)
    raise AttributeError(name)
