"""GPU parity: LoRA branch kernels and the fused RMSNorm / SiLU-multiply kernels.

PACT, Appendix Table 7, row "LoRA branch": BF16 products on the dequantized
input, BF16 adapter gradients; RMSNorm / SiLU-multiply fused with NVFP4 quantization
forward (codes bit-exact) and FP32 reconstruction backward (within
2 ulp_bf16 + 2^-17 * cancelling magnitude).
"""


import numpy as np
import pytest
import torch

import synth
from oracle import backward as obwd
from oracle import fused as ofused
from oracle import lora as olora
from oracle import nvfp4 as onv
from oracle import tolerance as tol

from gpu_util import (assert_nvfp4_equal, assert_within, bf16_values, bits_to_torch, nvfp4_to_gpu,
                      torch_bf16_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _q(bits):
    return onv.quantize(bf16_values(bits).astype(np.float64))


# ---------------------------------------------------------------- LoRA
@pytest.mark.parametrize("M,K,N,r", [(64, 256, 256, 8), (37, 48, 80, 5), (4096, 3072, 1024, 16), (300, 512, 272, 64),
                                     (128, 256, 128, 128),
                                     # the Llama-3B step's gate/up (N = 8192) and down (K = 8192) projections,
                                     # whose token splits and strip counts differ from the k/v shape's
                                     (4096, 3072, 8192, 16), (4096, 8192, 3072, 16), (4096, 3072, 3072, 16)])
def test_lora_down_and_bwd(fw, M, K, N, r):
    s = 2.0
    x = synth.activations_bf16((M, K), 95, M + K)
    A = synth.normal_bf16((r, K), 0.01, 95, M + K + 1)
    B = synth.normal_bf16((N, r), 0.01, 95, M + K + 2)
    dy = synth.normal_bf16((M, N), 0.01, 95, M + K + 3)
    xq = _q(x)
    gx = nvfp4_to_gpu(xq)
    T = fw.lora_down(gx, bits_to_torch(A))
    t_exact, _, t_abs = olora.lora_down(xq, bf16_values(A))
    assert_within(torch_bf16_to_f64(T), t_exact, tol.gemm_bound(t_exact, t_abs), "T")
    dT, dA, dB = fw.lora_bwd(gx, bits_to_torch(A), bits_to_torch(B), bits_to_torch(dy), s)
    ref = olora.lora_bwd(xq, bf16_values(A), bf16_values(B), bf16_values(dy), s)
    assert_within(torch_bf16_to_f64(dT), ref["dT_exact"], tol.gemm_bound(ref["dT_exact"], ref["dT_abs"]), "dT")
    assert_within(torch_bf16_to_f64(dB), ref["dB_exact"],
                  tol.gemm_bound(ref["dB_exact"], ref["dB_abs"], ref["dB_tslack"]), "dB")
    assert_within(torch_bf16_to_f64(dA), ref["dA_exact"],
                  tol.gemm_bound(ref["dA_exact"], ref["dA_abs"], ref["dA_tslack"]), "dA")
    # the same backward in two calls (dT alone, then dA and dB given dT), each
    # with its own buffers: identical bits
    dT2 = fw.lora_bwd_dt(bits_to_torch(dy), bits_to_torch(B), s)
    dA2, dB2 = fw.lora_bwd_ab(gx, bits_to_torch(A), bits_to_torch(dy), dT2, s)
    assert torch.equal(dT2, dT) and torch.equal(dA2, dA) and torch.equal(dB2, dB), "split backward differs"


# ---------------------------------------------------------------- RMSNorm
def _rms_inputs(M, H, wid=3, tid=700):
    x = synth.activations_bf16((M, H), wid, tid)
    g = synth.uniform_bf16((H,), 0.9, 1.1, wid, tid + 1)
    return x, g


@pytest.mark.parametrize("M,H,exact", [(64, 256, "0"), (33, 3072, "0"), (33, 3072, "1"), (8192, 3072, "0"),
                                       (17, 16384, "0"), (5, 48, "1"), (9, 8192, "1"), (9, 6144, "0"),
                                       (6, 12288, "1")])
def test_rmsnorm_quant(fw, M, H, exact):
    x, g = _rms_inputs(M, H, tid=700 + H)
    yq, rstd = fw.rmsnorm_quant(bits_to_torch(x), bits_to_torch(g), 1e-5, exact_sum=exact == "1")
    ref_q, ref_rstd, _ = ofused.rmsnorm_quant(bf16_values(x), bf16_values(g), 1e-5)
    got_rstd = rstd.cpu().numpy()
    bad = np.flatnonzero(got_rstd.view(np.uint32) != ref_rstd.view(np.uint32))
    assert bad.size == 0, f"rstd differs in {bad.size} rows, first {bad[:5]}"
    assert_nvfp4_equal(yq, ref_q, f"rmsnorm {M}x{H}")


def test_rmsnorm_bwd(fw):
    M, H = 257, 3072
    x, g = _rms_inputs(M, H, tid=710)
    dy = synth.normal_bf16((M, H), 0.01, 3, 712)
    yq, rstd, _ = ofused.rmsnorm_quant(bf16_values(x), bf16_values(g), 1e-5)
    dx = fw.rmsnorm_bwd(nvfp4_to_gpu(yq), torch.from_numpy(rstd).cuda(), bits_to_torch(g), bits_to_torch(dy))
    ref, cancel = obwd.rmsnorm_bwd(yq, rstd, bf16_values(g), bf16_values(dy))
    assert_within(torch_bf16_to_f64(dx), ref, tol.grad_bound(ref, cancel), "rmsnorm_bwd")


# ---------------------------------------------------------------- SiLU-multiply
@pytest.mark.parametrize("M,I", [(64, 256), (19, 8192), (7, 14336), (3, 48)])
def test_silu_mul_quant(fw, M, I):
    a = synth.normal_bf16((M, I), 2.0, 96, I + 1)
    b = synth.normal_bf16((M, I), 1.0, 96, I + 2)
    if M >= 3:
        av = bf16_values(a).copy()
        av[0, :16] = [0, -0.0, 100, -100, 88, -88, 89.5, -89.5, 80.25, -80.25, 1e-30, -1e-30, 3, -3, 1e-3, -1e-3]
        a = synth.bf16_bits(av)
    hq, gq, uq = fw.silu_mul_quant(bits_to_torch(a), bits_to_torch(b))
    rh, ra, rb, _ = ofused.silu_mul_quant(bf16_values(a), bf16_values(b))
    assert_nvfp4_equal(gq, ra, "gate copy")
    assert_nvfp4_equal(uq, rb, "up copy")
    assert_nvfp4_equal(hq, rh, "h")


def test_silu_mul_quant_full_size_sampled(fw):
    """MLP-block shape [8192 x 8192]; rows are independent, 256 sampled rows checked."""
    M, I = 8192, 8192
    a = synth.normal_bf16((M, I), 2.0, 3, 720)
    b = synth.normal_bf16((M, I), 1.0, 3, 721)
    hq, gq, uq = fw.silu_mul_quant(bits_to_torch(a), bits_to_torch(b))
    rows = np.sort(np.random.default_rng(5).choice(M, size=256, replace=False))
    rh, ra, rb, _ = ofused.silu_mul_quant(bf16_values(a[rows]), bf16_values(b[rows]))
    assert_nvfp4_equal(hq, rh, "h", rows=rows)
    assert_nvfp4_equal(gq, ra, "gate", rows=rows)
    assert_nvfp4_equal(uq, rb, "up", rows=rows)


@pytest.mark.parametrize("M,I", [(64, 256), (33, 8192)])
def test_silu_mul_bwd(fw, M, I):
    a = synth.normal_bf16((M, I), 2.0, 97, I + 1)
    b = synth.normal_bf16((M, I), 1.0, 97, I + 2)
    dh = synth.normal_bf16((M, I), 0.01, 97, I + 3)
    aq, bq = _q(a), _q(b)
    dg, du = fw.silu_mul_bwd(nvfp4_to_gpu(aq), nvfp4_to_gpu(bq), bits_to_torch(dh))
    da, db, cda, cdb = obwd.silu_mul_bwd(aq, bq, bf16_values(dh))
    assert_within(torch_bf16_to_f64(dg), da, tol.grad_bound(da, cda), "dgate")
    assert_within(torch_bf16_to_f64(du), db, tol.grad_bound(db, cdb), "dup")


def test_lora_bwd_ab_batch_equals_single_calls(fw):
    """The batched adapter gradients of several projections (different K, N
    and ranks of one class, ragged M), each given T from lora_down (also a
    column slice of a stacked lora_down), equal each projection's
    lora_bwd bit for bit, and ranks of different classes are refused."""
    from frozen_weight_gemms_amd import _lib
    M, s = 300, 0.75
    shapes = [(256, 272, 16), (512, 128, 5), (272, 1024, 9), (1024, 256, 16), (128, 128, 1)]
    probs, refs = [], []
    for k, (K, N, r) in enumerate(shapes):
        x = synth.activations_bf16((M, K), 94, 10 * k)
        A = bits_to_torch(synth.normal_bf16((r, K), 0.01, 94, 10 * k + 1))
        B = bits_to_torch(synth.normal_bf16((N, r), 0.01, 94, 10 * k + 2))
        dy = bits_to_torch(synth.normal_bf16((M, N), 0.01, 94, 10 * k + 3))
        gx = nvfp4_to_gpu(_q(x))
        refs.append(fw.lora_bwd(gx, A, B, dy, s))
        dT = fw.lora_bwd_dt(dy, B, s)
        out = (torch.full((r, K), 7.0, dtype=torch.bfloat16, device="cuda"),
               torch.full((N, r), 7.0, dtype=torch.bfloat16, device="cuda"))
        probs.append((gx, fw.lora_down(gx, A), dy, dT, out, fw.lora_bwd_workspace(M, K, N, r), A, B))
    # two projections over one input with their adapters stacked in one lora_down
    gx0, A0, A1 = probs[0][0], probs[0][6], probs[3][6][:, :256]
    Ts = fw.lora_down(gx0, torch.cat([A0, A1]).contiguous())
    B1 = probs[3][7]
    ref_st = fw.lora_bwd(gx0, A1.contiguous(), B1, probs[3][2], s)
    out_st = (torch.empty((16, 256), dtype=torch.bfloat16, device="cuda"), torch.empty_like(ref_st[2]))
    dT_st = fw.lora_bwd_dt(probs[3][2], B1, s)
    fw.lora_bwd_ab_batch([p[:6] for p in probs] + [(gx0, Ts[:, 16:32], probs[3][2], dT_st, out_st,
                                                   fw.lora_bwd_workspace(M, 256, 256, 16))], s)
    for (dT_ref, dA_ref, dB_ref), p in zip(refs, probs):
        assert torch.equal(p[3], dT_ref)
        assert torch.equal(p[4][0], dA_ref) and torch.equal(p[4][1], dB_ref), "batched dA / dB differ"
    assert torch.equal(Ts[:, :16], probs[0][1]), "stacked lora_down T differs from the single one"
    assert torch.equal(out_st[0], ref_st[1]) and torch.equal(out_st[1], ref_st[2]), "stacked-T problem differs"
    # one problem, and the Llama-3B gate shape (token splits of the big shapes)
    fw.lora_bwd_ab_batch([probs[0][:6]], s)
    assert torch.equal(probs[0][4][0], refs[0][1])
    M2, K2, N2, r2 = 4096, 3072, 8192, 16
    x = synth.activations_bf16((M2, K2), 94, 99)
    A = bits_to_torch(synth.normal_bf16((r2, K2), 0.01, 94, 100))
    B = bits_to_torch(synth.normal_bf16((N2, r2), 0.01, 94, 101))
    dy = bits_to_torch(synth.normal_bf16((M2, N2), 0.01, 94, 102))
    gx = nvfp4_to_gpu(_q(x))
    dT, dA, dB = fw.lora_bwd(gx, A, B, dy, s)
    out = (torch.empty_like(dA), torch.empty_like(dB))
    fw.lora_bwd_ab_batch([(gx, fw.lora_down(gx, A), dy, dT, out, fw.lora_bwd_workspace(M2, K2, N2, r2))], s)
    assert torch.equal(out[0], dA) and torch.equal(out[1], dB)
    # ranks of different classes in one batch
    bad = [probs[0][:6]]
    gx, T, dy, dT, _, ws = probs[0][:6]
    T32 = torch.zeros((M, 32), dtype=torch.bfloat16, device="cuda")
    dT32 = torch.zeros((M, 32), dtype=torch.bfloat16, device="cuda")
    bad.append((gx, T32, dy, dT32, (torch.empty((32, gx.cols), dtype=torch.bfloat16, device="cuda"),
                                    torch.empty((dy.shape[1], 32), dtype=torch.bfloat16, device="cuda")),
                fw.lora_bwd_workspace(M, gx.cols, dy.shape[1], 32)))
    with pytest.raises(_lib.PactError):
        fw.lora_bwd_ab_batch(bad, s)


def test_lora_bwd_ab_batch_edges(fw):
    """Empty token axis (every gradient an empty sum: zeros), the maximum of 8
    problems in one call, and problem counts outside 1..8 refused."""
    from frozen_weight_gemms_amd import _lib
    s = 0.5
    # M = 0: dA and dB are zero-filled
    K, N, r = 256, 128, 16
    gx = fw.empty_nvfp4(0, K, "cuda")
    out = (torch.full((r, K), 3.0, dtype=torch.bfloat16, device="cuda"),
           torch.full((N, r), 3.0, dtype=torch.bfloat16, device="cuda"))
    z = lambda *sh: torch.zeros(sh, dtype=torch.bfloat16, device="cuda")
    fw.lora_bwd_ab_batch([(gx, z(0, r), z(0, N), z(0, r), out, fw.lora_bwd_workspace(0, K, N, r))], s)
    assert not out[0].any() and not out[1].any()
    # 8 problems at once, each equal to its own lora_bwd
    M = 96
    probs, refs = [], []
    for k in range(8):
        K, N, r = 128 + 16 * k, 256 - 16 * k, 9 + k
        x = synth.activations_bf16((M, K), 95, 10 * k)
        A = bits_to_torch(synth.normal_bf16((r, K), 0.01, 95, 10 * k + 1))
        B = bits_to_torch(synth.normal_bf16((N, r), 0.01, 95, 10 * k + 2))
        dy = bits_to_torch(synth.normal_bf16((M, N), 0.01, 95, 10 * k + 3))
        g = nvfp4_to_gpu(_q(x))
        refs.append(fw.lora_bwd(g, A, B, dy, s))
        out = (torch.empty((r, K), dtype=torch.bfloat16, device="cuda"),
               torch.empty((N, r), dtype=torch.bfloat16, device="cuda"))
        probs.append((g, fw.lora_down(g, A), dy, fw.lora_bwd_dt(dy, B, s), out, fw.lora_bwd_workspace(M, K, N, r)))
    fw.lora_bwd_ab_batch(probs, s)
    for (_, dA_ref, dB_ref), p in zip(refs, probs):
        assert torch.equal(p[4][0], dA_ref) and torch.equal(p[4][1], dB_ref)
    with pytest.raises(_lib.PactError):
        fw.lora_bwd_ab_batch(probs + probs[:1], s)
    with pytest.raises(_lib.PactError):
        fw.lora_bwd_ab_batch([], s)
