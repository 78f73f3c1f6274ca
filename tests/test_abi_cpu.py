"""CPU-side checks of the C-ABI library: it loads, exports every function the
header declares, and rejects invalid arguments on the host before any HIP
call (so these run without a GPU)."""

import ctypes
import os
import subprocess

import pytest

ROOT_ = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_so = os.path.join(ROOT_, "frozen_weight_gemms_amd", "libpact_nvfp4.so")
if not os.path.exists(_so):       # build once if nothing is built
    subprocess.run(["python", os.path.join(ROOT_, "frozen_weight_gemms_amd", "build.py")], check=True)

from frozen_weight_gemms_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_symbols_exported(lib):
    names = _lib.header_functions()
    assert len(names) == len(set(names)) and len(names) >= 27, names
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n
    # the dynamic symbol table has them unmangled (extern "C")
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in syms, n


def test_library_targets_gfx950_only():
    """The embedded offload bundle holds gfx950 code objects and nothing else."""
    import re
    data = open(_lib.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-[-a-z0-9:+]*", data))
    assert targets == {b"amdgcn-amd-amdhsa--gfx950"}, targets


def test_gemm_tile_query(lib):
    assert _lib.gemm_tile(4096, 8192, 3072) == (256, 256)
    assert _lib.gemm_tile(4096, 3072, 3072) == (256, 192)
    assert _lib.gemm_tile(4096, 1024, 3072) == (128, 128)
    assert lib.pact_gemm_tile(-1, 1, 1, None, None) == -1
    assert _lib.gemm_multi_tile(2048, 12288) == (256, 192)      # 256 x 256 for the plain GEMM
    assert _lib.gemm_multi_tile(4096, 3072) == (256, 192)
    assert _lib.gemm_multi_tile(4096, 2048) == (256, 128)
    assert _lib.gemm_multi_tile(160, 640) == (128, 128)
    assert lib.pact_gemm_multi_tile(-1, 1, None, None) == -1


def test_abi_version(lib):
    assert lib.pact_abi_version() == 15


def test_sizes(lib):
    c, s, r = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.pact_nvfp4_sizes(4096, 3072, ctypes.byref(c), ctypes.byref(s), ctypes.byref(r)) == 0
    assert (c.value, s.value, r.value) == (4096 * 1536, 4096 * 192, 4096 * 4)
    assert (c.value + s.value) * 8 == 4096 * 3072 * 4.5
    assert lib.pact_nvfp4_sizes(4, 24, ctypes.byref(c), ctypes.byref(s), ctypes.byref(r)) == -2
    assert b"multiple of 16" in lib.pact_last_error()
    assert lib.pact_nvfp4_sizes(-1, 16, ctypes.byref(c), ctypes.byref(s), ctypes.byref(r)) == -1


ALIGNED = 1 << 20          # fake, 16-byte aligned addresses: never dereferenced on the error paths
MISALIGNED = ALIGNED + 4


def test_quantize_validation(lib):
    q = lib.nvfp4_quantize
    assert q(ALIGNED, 4, 24, 24, 0, ALIGNED, ALIGNED, ALIGNED, None) == -2          # cols % 16
    assert q(ALIGNED, 4, 32, 32, 2, ALIGNED, ALIGNED, ALIGNED, None) == -1          # bad transpose flag
    assert q(None, 4, 32, 32, 0, ALIGNED, ALIGNED, ALIGNED, None) == -1             # NULL x
    assert q(MISALIGNED, 4, 32, 32, 0, ALIGNED, ALIGNED, ALIGNED, None) == -3       # misaligned x
    assert q(ALIGNED, 4, 32, 16, 0, ALIGNED, ALIGNED, ALIGNED, None) == -2          # ldx < cols
    assert q(ALIGNED, 4, 32, 36, 0, ALIGNED, ALIGNED, ALIGNED, None) == -3          # ldx % 8
    assert q(ALIGNED, 4, 32, 2, 1, ALIGNED, ALIGNED, ALIGNED, None) == -2           # transposed ldx < rows
    assert q(ALIGNED, 0, 32, 32, 0, None, None, None, None) == 0                    # empty: no-op
    assert lib.pact_last_error() == b""



def test_quantize_batch_validation(lib):
    """nvfp4_quantize_batch checks every problem on the host before launching anything."""
    P, I = ctypes.c_void_p * 3, ctypes.c_int64 * 3
    ptrs = P(ALIGNED, ALIGNED, ALIGNED)
    rows, cols, ldx = I(4, 8, 2), I(32, 48, 16), I(32, 48, 16)
    q = lib.nvfp4_quantize_batch
    assert q(0, ptrs, rows, cols, ldx, ptrs, ptrs, ptrs, None) == -1                 # n outside [1, 8]
    assert q(9, ptrs, rows, cols, ldx, ptrs, ptrs, ptrs, None) == -1
    assert q(3, None, rows, cols, ldx, ptrs, ptrs, ptrs, None) == -1                 # NULL problem array
    assert q(3, ptrs, rows, I(32, 40, 16), ldx, ptrs, ptrs, ptrs, None) == -2        # problem 1: cols % 16
    assert b"problem 1" in lib.pact_last_error()
    assert q(3, P(ALIGNED, ALIGNED, MISALIGNED), rows, cols, ldx, ptrs, ptrs, ptrs, None) == -3   # problem 2: x
    assert b"problem 2" in lib.pact_last_error()
    assert q(3, ptrs, rows, cols, I(32, 40, 16), ptrs, ptrs, ptrs, None) == -2       # problem 1: ldx < cols
    assert q(3, ptrs, rows, cols, I(32, 52, 16), ptrs, ptrs, ptrs, None) == -3       # problem 1: ldx % 8
    assert q(3, ptrs, rows, cols, ldx, ptrs, P(ALIGNED, None, ALIGNED), ptrs, None) == -1   # problem 1: scales
    assert q(3, ptrs, I(-1, 8, 2), cols, ldx, ptrs, ptrs, ptrs, None) == -1          # negative rows
    empty = P(None, None, None)
    assert q(3, empty, I(0, 0, 0), cols, ldx, empty, empty, empty, None) == 0          # every problem empty: no-op
    assert lib.pact_last_error() == b""

def test_fused_validation(lib):
    assert lib.rmsnorm_quant(ALIGNED, ALIGNED, 1e-5, 4, 20000, 20000, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                             None) == -5
    assert lib.rmsnorm_quant(ALIGNED, None, 1e-5, 4, 32, 32, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None) == -1
    assert lib.rmsnorm_quant(ALIGNED, ALIGNED, -1.0, 4, 32, 32, ALIGNED, ALIGNED, ALIGNED, ALIGNED, None) == -1
    args9 = [ALIGNED] * 9
    assert lib.silu_mul_quant(ALIGNED, ALIGNED, 4, 40, 40, *args9, None) == -2
    args9[4] = MISALIGNED
    assert lib.silu_mul_quant(ALIGNED, ALIGNED, 4, 32, 32, *args9, None) == -3
    assert lib.silu_mul_quant(ALIGNED, ALIGNED, 0, 32, 32, *([None] * 9), None) == 0


def test_gemm_validation(lib):
    A = [ALIGNED] * 3
    f = lib.nvfp4_gemm_fwd
    assert f(*A, 64, 40, *A, 64, ALIGNED, 64, None, None, 0, 1.0, None) == -2      # K % 16
    assert f(*A, 64, 64, *A, 64, ALIGNED, 32, None, None, 0, 1.0, None) == -2      # ldy < N
    assert f(*A, 64, 64, *A, 64, ALIGNED, 64, ALIGNED, None, 8, 1.0, None) == -1   # T without B
    assert f(*A, 64, 64, *A, 64, ALIGNED, 64, ALIGNED, ALIGNED, 0, 1.0, None) == -2   # rank 0
    assert f(*A, 64, 64, *A, 64, ALIGNED, 64, ALIGNED, ALIGNED, 129, 1.0, None) == -2  # rank > 128
    assert f(None, ALIGNED, ALIGNED, 64, 64, *A, 64, ALIGNED, 64, None, None, 0, 1.0, None) == -1
    assert f(*A, 0, 64, *A, 64, None, 64, None, None, 0, 1.0, None) == 0              # empty: no-op
    d = lib.nvfp4_gemm_dgrad
    assert d(*A, 64, 64, *A, 64, ALIGNED, 64, 2, None, None, 0, None) == -1          # accumulate flag
    assert d(*A, 64, 72, *A, 64, ALIGNED, 64, 0, None, None, 0, None) == -2          # N % 16
    assert d(*A, 64, 64, *A, 64, ALIGNED, 64, 0, ALIGNED, None, 8, None) == -1


def test_lora_and_backward_validation(lib):
    A = [ALIGNED] * 3
    assert lib.lora_down(*A, 64, 64, ALIGNED, 0, ALIGNED, None) == -2
    assert lib.lora_down(*A, 64, 72, ALIGNED, 8, ALIGNED, None) == -2
    assert lib.lora_down(*A, 64, 64, None, 8, ALIGNED, None) == -1
    assert lib.lora_bwd(*A, 64, 64, ALIGNED, ALIGNED, 8, 1.0, ALIGNED, 40, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                        1 << 30, None) == -2
    need = _lib.lora_bwd_workspace_size(4096, 3072, 8192, 16)
    assert need > 4096 * 16 * 2
    assert lib.lora_bwd(*A, 64, 64, ALIGNED, ALIGNED, 8, 1.0, ALIGNED, 64, ALIGNED, ALIGNED, ALIGNED, None,
                        1 << 30, None) == -1                                        # no workspace
    assert lib.lora_bwd(*A, 64, 64, ALIGNED, ALIGNED, 8, 1.0, ALIGNED, 64, ALIGNED, ALIGNED, ALIGNED, ALIGNED,
                        16, None) == -1                                             # too small
    assert lib.lora_bwd(*A, 64, 64, ALIGNED, ALIGNED, 8, 1.0, ALIGNED, 64, ALIGNED, ALIGNED, ALIGNED,
                        ALIGNED + 16, 1 << 30, None) == -3                          # misaligned
    assert lib.silu_mul_bwd(*A, *A, ALIGNED, 4, 40, ALIGNED, ALIGNED, None) == -2
    assert lib.rmsnorm_bwd(*A, ALIGNED, ALIGNED, ALIGNED, 4, 32, None, None) == -1
    assert lib.rmsnorm_bwd(*A, ALIGNED, ALIGNED, ALIGNED, 0, 32, None, None) == 0


def test_package_import_requires_library(tmp_path, monkeypatch):
    """Without the built library the binding refuses to load (no CPU fallback)."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_mxfp4_sizes_and_validation(lib):
    c, s = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.pact_mxfp4_sizes(4096, 3072, ctypes.byref(c), ctypes.byref(s)) == 0
    assert (c.value, s.value) == (4096 * 1536, 4096 * 96)
    assert (c.value + s.value) * 8 == 4096 * 3072 * 4.25
    assert lib.pact_mxfp4_sizes(4, 48, ctypes.byref(c), ctypes.byref(s)) == -2      # cols % 32
    q = lib.mxfp4_quantize
    assert q(ALIGNED, 4, 48, 48, 0, ALIGNED, ALIGNED, None) == -2                  # cols % 32
    assert q(ALIGNED, 4, 64, 64, 3, ALIGNED, ALIGNED, None) == -1                  # bad transpose flag
    assert q(None, 4, 64, 64, 0, ALIGNED, ALIGNED, None) == -1                     # NULL x
    assert q(ALIGNED, 4, 64, 64, 0, MISALIGNED, ALIGNED, None) == -3               # misaligned codes
    assert q(ALIGNED, 4, 64, 32, 0, ALIGNED, ALIGNED, None) == -2                  # ldx < cols
    g = lib.mxfp4_gemm
    assert g(ALIGNED, ALIGNED, 64, 96, ALIGNED, ALIGNED, 64, ALIGNED, 64, 0, None) == -2   # K % 128
    assert g(ALIGNED, ALIGNED, 64, 128, ALIGNED, ALIGNED, 64, ALIGNED, 32, 0, None) == -2  # ldc < N
    assert g(ALIGNED, ALIGNED, 64, 128, None, ALIGNED, 64, ALIGNED, 64, 0, None) == -1     # NULL b
    assert g(ALIGNED, ALIGNED, 64, 128, ALIGNED, ALIGNED, 64, ALIGNED, 64, 2, None) == -1  # accumulate flag
    assert g(ALIGNED, ALIGNED, 0, 128, ALIGNED, ALIGNED, 64, ALIGNED, 64, 0, None) == 0    # empty: no-op


def test_fused_backward_validation(lib):
    A, X = ALIGNED, MISALIGNED
    f = lib.silu_mul_bwd_quant
    assert f(A, A, A, A, A, A, A, 4, 40, A, A, A, A, A, A, A, A, None) == -2        # I % 16
    assert f(A, A, A, A, A, A, A, 4, 32768, A, A, A, A, A, A, A, A, None) == -5     # I > 16384
    assert f(A, A, A, A, A, A, A, 4, 64, A, A, None, A, A, A, A, A, None) == -1     # NULL dgate_q codes
    assert f(A, A, A, A, A, A, A, 4, 64, A, A, A, A, A, A, A, X, None) == -3        # misaligned dup_q rscale
    assert f(A, A, A, A, A, A, A, 0, 64, A, A, A, A, A, A, A, A, None) == 0         # empty
    g = lib.rmsnorm_bwd_residual
    assert g(A, A, A, A, A, A, None, 4, 40, A, None, None, None, None) == -2       # H % 16
    assert g(A, A, A, A, A, A, None, 4, 64, None, None, None, None, None) == -1    # NULL dx
    assert g(A, A, A, A, A, A, X, 4, 64, A, None, None, None, None) == -3          # misaligned resid
    assert g(A, A, A, A, A, A, None, 4, 64, A, A, None, A, None) == -1             # partial NVFP4 output
    assert g(A, A, A, A, A, A, None, 0, 64, A, None, None, None, None) == 0        # empty


def test_dgrad_multi_validation(lib):
    """Argument checks of nvfp4_gemm_dgrad_multi run before any device call."""
    import ctypes
    P = ctypes.c_void_p * 2
    fake = P(ctypes.c_void_p(256), ctypes.c_void_p(512))
    widths = (ctypes.c_int64 * 2)(512, 272)
    st = lib.nvfp4_gemm_dgrad_multi(0, fake, fake, fake, widths, fake, fake, fake, 64, 64, ctypes.c_void_p(256), 64,
                                    0, None, None, None, None)
    assert st == -1                                      # nseg outside [1, 4]
    st = lib.nvfp4_gemm_dgrad_multi(2, fake, fake, fake, widths, fake, fake, fake, 64, 64, ctypes.c_void_p(256), 64,
                                    0, None, None, None, None)
    assert st == -5                                      # 272 is not a multiple of 256
    assert b"multiple of 256" in lib.pact_last_error()



def test_mfma_probe_validation(lib):
    """Argument checks of pact_mfma_probe run before any device call."""
    A = ALIGNED
    assert lib.pact_mfma_probe(2, 10, A, 512 * 256, A, 1024, None) == -1        # kind
    assert lib.pact_mfma_probe(0, 0, A, 512 * 256, A, 1024, None) == -1         # iters
    assert lib.pact_mfma_probe(0, 10, None, 512 * 256, A, 1024, None) == -1     # NULL sink
    assert lib.pact_mfma_probe(1, 10, A, 512 * 256 - 1, A, 1024, None) == -2    # short sink
    assert lib.pact_mfma_probe(1, 10, A, 512 * 256, A, 1023, None) == -2        # short clocks
