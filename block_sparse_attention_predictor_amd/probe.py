"""ctypes binding of libveda_probe.so (include/veda_probe.h): measurement aids for the
benchmark, kept out of the method's library.  Raises when the library is not built."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libveda_probe.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               "`python -m block_sparse_attention_predictor_amd.build` (needs hipcc)")
        lib = ctypes.CDLL(lib_path)
        lib.veda_probe_mfma_peak.restype = ctypes.c_int
        lib.veda_probe_mfma_peak.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        _lib = lib
    return _lib


def exported_symbols():
    return ["veda_probe_mfma_peak"]


def mfma_peak(iters: int = 2000, workgroups: int = 2048, stream=None):
    """Launch the MFMA-only loop on the current stream; returns (checksum buffer, flops)."""
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    if stream is None:
        stream = torch.cuda.current_stream()
    st = _load().veda_probe_mfma_peak(ctypes.c_void_p(out.data_ptr()), int(iters), int(workgroups),
                                      ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"veda_probe_mfma_peak returned {st}")
    return out, 2097152.0 * iters * workgroups
