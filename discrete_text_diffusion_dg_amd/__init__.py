"""DiffusionGemma-style block-diffusion denoise step on MI355X (gfx950).

The hot path lives in libdg.so (hand-written HIP, include/dg.h).  This package
holds the ctypes binding (``_lib``), a torch-backed engine (``runtime``) and the
build script (``build``).  Importing ``Engine`` loads the library and raises if
it has not been built.
"""


def __getattr__(name):
    if name in ("Engine", "upload_weights"):
        from . import runtime
        return getattr(runtime, name)
    raise AttributeError(name)
