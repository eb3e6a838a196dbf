"""Veda-style learned block-sparse attention on MI355X (gfx950).

The compute path lives in ``libveda.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/veda.h``); this package only marshals torch tensors
into that ABI.  ``inputs`` draws the seeded synthetic workloads.

Attributes of the binding (``select``, ``sparse_attn``, ``dequant_fp8_e4m3``,
``Layer`` ...) are loaded on first use, so importing the package does not load
the shared library.
"""

__all__ = ["select", "sparse_attn", "layer_attn", "dequant_fp8_e4m3", "project", "Layer", "VedaError",
           "lib_path", "build"]


def __getattr__(name):
    if name in ("select", "sparse_attn", "dequant_fp8_e4m3", "project", "Layer", "layer_attn",
                "VedaError", "lib_path", "layer_from_workload", "select_workspace_bytes",
                "status_string", "abi_version"):
        from . import binding
        return getattr(binding, name)
    if name == "build":
        # importlib, not "from . import build": that form looks the name up on this
        # package first and would re-enter this function
        import importlib
        return importlib.import_module(__name__ + ".build").build
    raise AttributeError(name)
