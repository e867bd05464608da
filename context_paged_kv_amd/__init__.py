"""Decode Context Parallelism over a paged KV cache, for MI355X (gfx950).

The compute path is libdcpkv.so (hand-written HIP kernels behind a C ABI,
include/dcpkv.h); this package is its thin ctypes binding (``_lib``) plus the
in-tree build script (``build``).  Accessing any entry point loads the library
and raises if it has not been built: there is no other path.
"""

_API = None


def _load():
    global _API
    if _API is None:
        import importlib
        _API = importlib.import_module(__name__ + "._lib")
    return _API


def __getattr__(name):
    if name.startswith("__") or name in ("_lib", "build"):
        raise AttributeError(name)
    api = _load()
    try:
        return getattr(api, name)
    except AttributeError:
        raise AttributeError(f"context_paged_kv_amd has no attribute {name!r}") from None
