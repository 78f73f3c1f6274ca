"""GPU check of lora_bwd_noalloc, the LoRA backward that uses the library's
fixed per-device scratch instead of a caller workspace: called through the C
ABI, its outputs must equal lora_bwd's (the existing entry point, same
kernels) bit for bit, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's contents), and a shape whose scratch need
exceeds the fixed size is refused with PACT_EUNSUPPORTED."""

import numpy as np
import pytest
import torch

import synth
from oracle import lora as olora
from oracle import nvfp4 as onv
from oracle import tolerance as tol

from gpu_util import assert_within, bf16_values, bits_to_torch, nvfp4_to_gpu, torch_bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _case(M, K, N, r, seed):
    x = synth.activations_bf16((M, K), 98, seed)
    A = synth.normal_bf16((r, K), 0.01, 98, seed + 1)
    B = synth.normal_bf16((N, r), 0.01, 98, seed + 2)
    dy = synth.normal_bf16((M, N), 0.01, 98, seed + 3)
    return onv.quantize(bf16_values(x).astype(np.float64)), A, B, dy


def _outs(M, K, N, r):
    e = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda")
    return e(M, r), e(r, K), e(N, r)


def test_noalloc_matches_lora_bwd_twice(fw):
    s = 0.75
    for (M, K, N, r, seed) in ((4096, 3072, 8192, 16, 10), (300, 512, 272, 64, 20)):
        xq, A, B, dy = _case(M, K, N, r, seed)
        gx, gA, gB, gdy = nvfp4_to_gpu(xq), bits_to_torch(A), bits_to_torch(B), bits_to_torch(dy)
        want = fw.lora_bwd(gx, gA, gB, gdy, s)
        got = _outs(M, K, N, r)
        fw.lora_bwd_noalloc(gx, gA, gB, gdy, s, out=got)
        torch.cuda.synchronize()
        for name, g, w in zip(("dT", "dA", "dB"), got, want):
            assert torch.equal(g.view(torch.int16), w.view(torch.int16)), f"{name} differs at {M}x{K}x{N} r={r}"
        # and the oracle's bound, so the shared kernels are checked too
        ref = olora.lora_bwd(xq, bf16_values(A), bf16_values(B), bf16_values(dy), s)
        assert_within(torch_bf16_to_f64(got[0]), ref["dT_exact"], tol.gemm_bound(ref["dT_exact"], ref["dT_abs"]),
                      "dT")
        assert_within(torch_bf16_to_f64(got[2]), ref["dB_exact"],
                      tol.gemm_bound(ref["dB_exact"], ref["dB_abs"], ref["dB_tslack"]), "dB")
        assert_within(torch_bf16_to_f64(got[1]), ref["dA_exact"],
                      tol.gemm_bound(ref["dA_exact"], ref["dA_abs"], ref["dA_tslack"]), "dA")


def test_noalloc_rejects_oversized(fw):
    lib = fw._lib.load()
    M, K, N, r = 65536, 16384, 16384, 128
    need = fw._lib.lora_bwd_workspace_size(M, K, N, r)
    assert need > 32 << 20
    p = torch.empty((64,), dtype=torch.uint8, device="cuda")
    ptr = p.data_ptr()
    st = lib.lora_bwd_noalloc(ptr, ptr, ptr, M, K, ptr, ptr, r, 1.0, ptr, N, ptr, ptr, ptr, None)
    assert st == -5
    assert b"scratch" in lib.pact_last_error()
