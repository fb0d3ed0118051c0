"""ctypes binding of ``libattn_probes.so`` (include/attn_probes.h): the unit
microbenchmarks the benchmark reports as measured ceilings.  Argument
marshalling only; a missing library raises."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_probes.so")
EXPORTED = ("attn_probe_stream_read", "attn_probe_exp", "attn_probe_lds_read", "attn_probe_mfma")

_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"probe library not built: {LIB_PATH} is missing")
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.attn_probe_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ci, vp]
    lib.attn_probe_exp.argtypes = [vp, ci, ci, vp]
    lib.attn_probe_lds_read.argtypes = [vp, ci, ci, ci, vp]
    lib.attn_probe_mfma.argtypes = [vp, ci, ci, vp]
    for n in EXPORTED:
        getattr(lib, n).restype = ci
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        raise RuntimeError(f"probe launch failed ({st})")


def stream_read(src, out, blocks: int, stream):
    _check(load_library().attn_probe_stream_read(src.data_ptr(), src.numel() * src.element_size(),
                                                 out.data_ptr(), blocks, stream.cuda_stream))


def exp_rate(out, blocks: int, iters: int, stream):
    _check(load_library().attn_probe_exp(out.data_ptr(), blocks, iters, stream.cuda_stream))


def lds_read(out, blocks: int, iters: int, transposed: bool, stream):
    _check(load_library().attn_probe_lds_read(out.data_ptr(), blocks, iters, int(transposed),
                                              stream.cuda_stream))


def mfma_rate(out, blocks: int, iters: int, stream):
    _check(load_library().attn_probe_mfma(out.data_ptr(), blocks, iters, stream.cuda_stream))
