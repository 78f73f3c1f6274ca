"""ctypes binding of libpact_nvfp4.so: argument marshalling only.

Every computation runs in the HIP library; this module only turns torch
tensors into device pointers and sizes, passes torch's current HIP stream,
and raises on a non-zero status.  If the library is not built, importing the
package raises: there is no CPU fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpact_nvfp4.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pact_nvfp4.h")

_lib = None

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_float = ctypes.c_float
c_vp = ctypes.c_void_p
c_size_p = ctypes.POINTER(ctypes.c_size_t)

# argument signatures (ctypes) of every entry point in include/pact_nvfp4.h
SIGNATURES = {
    "pact_last_error": ([], ctypes.c_char_p),
    "pact_abi_version": ([], c_int),
    "pact_nvfp4_sizes": ([c_i64, c_i64, c_size_p, c_size_p, c_size_p], c_int),
    "pact_gemm_tile": ([c_i64, c_i64, c_i64, ctypes.POINTER(c_int), ctypes.POINTER(c_int)], c_int),
    "pact_gemm_multi_tile": ([c_i64, c_i64, ctypes.POINTER(c_int), ctypes.POINTER(c_int)], c_int),
    "nvfp4_quantize": ([c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp], c_int),
    "rmsnorm_quant": ([c_vp, c_vp, c_float, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp], c_int),
    "rmsnorm_quant_ex": ([c_vp, c_vp, c_float, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp, c_vp, c_vp], c_int),
    "silu_mul_quant": ([c_vp, c_vp, c_i64, c_i64, c_i64] + [c_vp] * 9 + [c_vp], c_int),
    "nvfp4_gemm_fwd": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64,
                        c_vp, c_vp, c_i64, c_float, c_vp], c_int),
    "nvfp4_gemm_dgrad": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_int,
                          c_vp, c_vp, c_i64, c_vp], c_int),
    "nvfp4_gemm_fwd_ex": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64,
                           c_vp, c_vp, c_i64, c_float, c_int, c_vp], c_int),
    "nvfp4_gemm_dgrad_ex": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_int,
                             c_vp, c_vp, c_i64, c_int, c_vp], c_int),
    "lora_bwd_dt": ([c_vp, c_i64, c_i64, c_vp, c_i64, c_float, c_vp, c_vp], c_int),
    "lora_bwd_ab": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_i64, c_float, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp,
                     ctypes.c_size_t, c_vp], c_int),
    "lora_bwd_ab_batch": ([c_int] + [c_vp] * 3 + [c_i64, c_vp, c_vp, c_vp, c_vp, c_float] + [c_vp] * 7 + [c_vp],
                          c_int),
    "lora_down": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp], c_int),
    "pact_lora_bwd_workspace_size": ([c_i64, c_i64, c_i64, c_i64, c_size_p], c_int),
    "lora_bwd": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_float, c_vp, c_i64,
                  c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp], c_int),
    "lora_bwd_noalloc": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_float, c_vp, c_i64,
                          c_vp, c_vp, c_vp, c_vp], c_int),
    "silu_mul_bwd": ([c_vp] * 7 + [c_i64, c_i64, c_vp, c_vp, c_vp], c_int),
    "rmsnorm_bwd": ([c_vp] * 6 + [c_i64, c_i64, c_vp, c_vp], c_int),
    "nvfp4_quantize_ex": ([c_vp, c_i64, c_i64, c_i64, c_int, c_int, c_vp, c_vp, c_vp, c_vp, c_vp], c_int),
    "nvfp4_quantize_batch": ([c_int] + [c_vp] * 7 + [c_vp], c_int),
    "nvfp4_gemm_dgrad_fwd_layout": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_i64,
                                     c_int, c_vp, c_vp, c_i64, c_vp], c_int),
    "pact_nvfp4_row_exp_max": ([c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp], c_int),
    "pact_selftest_arith": ([c_vp, c_vp], c_int),
    "pact_mfma_probe": ([c_int, c_int, c_vp, c_i64, c_vp, c_i64, c_vp], c_int),
    "nvfp4_gemm_dgrad_multi": ([c_int] + [c_vp] * 7 + [c_i64, c_i64, c_vp, c_i64, c_int] + [c_vp] * 3 + [c_vp],
                               c_int),
    "silu_mul_bwd_quant": ([c_vp] * 7 + [c_i64, c_i64] + [c_vp] * 9, c_int),
    "rmsnorm_bwd_residual": ([c_vp] * 7 + [c_i64, c_i64] + [c_vp] * 5, c_int),
    "pact_mxfp4_sizes": ([c_i64, c_i64, c_size_p, c_size_p], c_int),
    "mxfp4_quantize": ([c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_vp, c_vp], c_int),
    "mxfp4_rmsnorm_quant": ([c_vp, c_vp, c_float, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp], c_int),
    "mxfp4_silu_mul_quant": ([c_vp, c_vp, c_i64, c_i64, c_i64] + [c_vp] * 6 + [c_vp], c_int),
    "mxfp4_silu_mul_bwd_quant": ([c_vp] * 5 + [c_i64, c_i64] + [c_vp] * 6 + [c_vp], c_int),
    "mxfp4_rmsnorm_bwd_residual": ([c_vp] * 6 + [c_i64, c_i64] + [c_vp] * 3 + [c_vp], c_int),
    "mxfp4_gemm": ([c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_i64, c_int, c_vp], c_int),
}

STATUS = {0: "PACT_OK", -1: "PACT_EINVAL", -2: "PACT_ESHAPE", -3: "PACT_EALIGN", -4: "PACT_EHIP",
          -5: "PACT_EUNSUPPORTED"}


class PactError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def header_functions() -> list:
    """Names of the functions declared in include/pact_nvfp4.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const\s+char\s*\*)\s*\*?\s*([a-z_0-9]+)\s*\(",
                       text, flags=re.M)
    return names


def load():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python frozen_weight_gemms_amd/build.py "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def check(status: int):
    if status != 0:
        msg = _lib.pact_last_error().decode()
        raise PactError(status, msg)


def gemm_tile(M: int, Nout: int, Kr: int):
    """(bm, bn) workgroup tile the GEMM launches for this output shape."""
    lib = load()
    bm, bn = c_int(), c_int()
    check(lib.pact_gemm_tile(M, Nout, Kr, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def gemm_multi_tile(M: int, Nout: int):
    """(bm, bn) workgroup tile the segmented input-gradient GEMM launches for this output shape."""
    lib = load()
    bm, bn = c_int(), c_int()
    check(lib.pact_gemm_multi_tile(M, Nout, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def lora_bwd_workspace_size(M: int, K: int, N: int, r: int) -> int:
    lib = load()
    n = ctypes.c_size_t()
    check(lib.pact_lora_bwd_workspace_size(M, K, N, r, ctypes.byref(n)))
    return n.value


def call(name: str, *args):
    lib = load()
    check(getattr(lib, name)(*args))
