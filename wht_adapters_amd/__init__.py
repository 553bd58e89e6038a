"""MI355X (gfx950) batched Walsh-Hadamard transforms: orthonormal FWHT,
RHT + per-group RTN quantisation and its inverse, the QWHA adapter forward
and a HARP-style structured rotation.

The compute lives in the HIP shared library ``libwhtq.so`` (C ABI declared in
``include/whtq.h``); ``wht_adapters_amd.whtq`` is the thin ctypes binding over
it.  Attribute access on this package loads the binding lazily so that the
input generators in ``wht_adapters_amd.synth`` import without the library.
"""

_API = ("wht_batched", "rht_quantize_rtn", "rht_dequantize_inverse",
        "qwha_adapter_forward", "harp_rotate", "WhtqError", "lib_path",
        "abi_version")


def __getattr__(name):
    if name in _API:
        from . import whtq
        return getattr(whtq, name)
    raise AttributeError(name)
