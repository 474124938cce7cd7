"""MI355X-native paged KV cache: decode attention, chunked prefill and the
KV scatter, as hand-written HIP kernels for gfx950 behind a C-ABI library
(``libpa.so``).  The binding in :mod:`paged_kv_cache_326_amd.pa` marshals
torch tensors into that library; importing this package does not load it.
"""

__version__ = "0.1.0"


def __getattr__(name):
    # The binding is loaded on first use so that CPU-only tooling (the input
    # generator, host-side tests) imports without a GPU.
    if name in ("pa",):
        import importlib

        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
