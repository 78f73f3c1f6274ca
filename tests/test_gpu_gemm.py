"""GPU parity: nvfp4_gemm_fwd / nvfp4_gemm_dgrad against the oracle's float64 GEMM.

Frozen projections: NVFP4 GEMMs, FP32 accumulation, BF16 output, forward over
W_fwd = Q(W) and input gradient over W_bwd = Q(W^T) (PACT, Appendix Table 7).
Bound: |y - y_ref| <= ulp_bf16(y_ref) + 1e-5 * sum_k |a_k b_k| (+ the LoRA
term's share).  Operands are quantized by the oracle and uploaded, so these
tests do not depend on the GPU quantizer.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import lora as olora
from oracle import nvfp4 as onv
from oracle import tolerance as tol

from gpu_util import assert_within, bf16_values, bits_to_torch, nvfp4_to_gpu, torch_bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _q(bits):
    return onv.quantize(bf16_values(bits).astype(np.float64))


def _qt(bits):
    return onv.quantize(bf16_values(bits).astype(np.float64), transpose=True)


def test_tiny_fwd_dgrad(fw):
    x = synth.workload_activation(synth.WORKLOADS[0], 64, 256, 1)
    w = synth.normal_bf16((256, 256), 0.02, 0, 2)
    dy = synth.normal_bf16((64, 256), 0.01, 0, 3)
    xq, wf, wb, dyq = _q(x), _q(w), _qt(w), _q(dy)
    y = fw.gemm_fwd(nvfp4_to_gpu(xq), nvfp4_to_gpu(wf))
    yref, yabs = ogemm.gemm_fwd(xq, wf)
    assert_within(torch_bf16_to_f64(y), yref, tol.gemm_bound(yref, yabs), "fwd")
    dx = fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb))
    dref, dabs = ogemm.gemm_dgrad(dyq, wb)
    assert_within(torch_bf16_to_f64(dx), dref, tol.gemm_bound(dref, dabs), "dgrad")


def _direct(codes, scale_byte, rows):
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = np.asarray(scale_byte, dtype=np.uint8)
    if sc.ndim == 0:
        sc = np.full((rows, codes.shape[1] // 16), int(sc), np.uint8)
    return onv.NVFP4(packed, sc, np.ones(rows, np.float32))


@pytest.mark.parametrize("M,N,K", [(64, 64, 512), (300, 200, 512), (256, 512, 256)])
def test_exact_special_case_bit_identical(fw, M, N, K):
    """Scales in [1, 1.875] and row scale 1: FP32 accumulation is exact, so the
    BF16 output must equal RNE of the exact result bit for bit."""
    rng = np.random.default_rng(M * 7 + N)
    ca, cb = rng.integers(0, 16, size=(M, K)), rng.integers(0, 16, size=(N, K))
    sa = rng.integers(0x38, 0x40, size=(M, K // 16))       # 1.0 .. 1.875
    sb = rng.integers(0x38, 0x40, size=(N, K // 16))
    a, b = _direct(ca, sa, M), _direct(cb, sb, N)
    y = fw.gemm_fwd(nvfp4_to_gpu(a), nvfp4_to_gpu(b))
    yref, _ = ogemm.gemm_nt(a, b)
    got = torch_bf16_to_f64(y)
    want = tol.bf16_rne(yref)
    assert np.array_equal(got, want), f"{np.sum(got != want)} outputs differ"


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (7, 33, 48), (130, 257, 272), (300, 100, 1040),
                                   (513, 640, 4096), (64, 2048, 128), (2, 300, 768), (1000, 130, 1280)])
def test_ragged_shapes(fw, M, N, K):
    a = synth.activations_bf16((M, K), 92, M + 3 * N + 7 * K)
    b = synth.normal_bf16((N, K), 0.02, 92, M + 3 * N + 7 * K + 1)
    aq, bq = _q(a), _q(b)
    y = fw.gemm_fwd(nvfp4_to_gpu(aq), nvfp4_to_gpu(bq))
    yref, yabs = ogemm.gemm_nt(aq, bq)
    assert_within(torch_bf16_to_f64(y), yref, tol.gemm_bound(yref, yabs), f"{M}x{N}x{K}")


def test_lora_epilogue_fwd(fw):
    M, K, N, r, s = 96, 256, 320, 8, 2.0
    x = synth.activations_bf16((M, K), 93, 1)
    w = synth.normal_bf16((N, K), 0.02, 93, 2)
    t = synth.normal_bf16((M, r), 0.3, 93, 3)
    b = synth.normal_bf16((N, r), 0.01, 93, 4)
    xq, wf = _q(x), _q(w)
    gx, gw = nvfp4_to_gpu(xq), nvfp4_to_gpu(wf)
    base = fw.gemm_fwd(gx, gw)
    zero = fw.gemm_fwd(gx, gw, lora_t=bits_to_torch(t), lora_b=torch.zeros((N, r), dtype=torch.bfloat16,
                                                                          device="cuda"), lora_scale=s)
    assert torch.equal(base.view(torch.int16), zero.view(torch.int16)), "B = 0 must not change Y"
    y = fw.gemm_fwd(gx, gw, lora_t=bits_to_torch(t), lora_b=bits_to_torch(b), lora_scale=s)
    yref, yabs = ogemm.gemm_fwd(xq, wf)
    term, tabs, _ = olora.lora_term(bf16_values(t), bf16_values(b).T, s)
    assert_within(torch_bf16_to_f64(y), yref + term, tol.gemm_bound(yref + term, yabs + tabs), "fwd+lora")



@pytest.mark.parametrize("M,N,K", [(96, 320, 256), (200, 1536, 512), (4096, 2048, 256), (1024, 12288, 256),
                                   (2048, 12288, 256)])
@pytest.mark.parametrize("s", [2.0, 0.75, -1.0 / 3.0])
def test_lora_term_scale_under_cancellation(fw, M, N, K, s):
    """lora_scale * T B^T alone (W = 0), with rank pairs that nearly cancel:
    T = [T1, T2] with T2 = bf16(T1 (1 + 2^-6)) and B = [B1, -B1], so the term is
    about 2^-6 of sum |T||B| and the bound (1e-5 of that sum plus one BF16 ulp)
    exposes any rounding of s T before the products.  Fast-path tiles:
    128 x 128 (the first two, one with a ragged row tile), 256 x 128,
    256 x 192 and 256 x 256.  A power-of-two s scales T exactly; any other s
    must keep FP32 accuracy of s T (a single BF16 rounding of s T / r_A is
    shown below to violate the bound)."""
    x = synth.activations_bf16((M, K), 95, 1)
    w = np.zeros((N, K), dtype=np.uint16)
    t1 = synth.normal_bf16((M, 16), 0.3, 95, 3)
    t2 = synth.bf16_bits(synth.bf16_from_bits(t1) * np.float32(1 + 2.0 ** -6))
    b1 = synth.normal_bf16((N, 16), 0.01, 95, 4)
    t = np.ascontiguousarray(np.hstack([t1, t2]))
    b = np.ascontiguousarray(np.hstack([b1, b1 ^ np.uint16(0x8000)]))
    xq, wf = _q(x), _q(w)
    y = fw.gemm_fwd(nvfp4_to_gpu(xq), nvfp4_to_gpu(wf), lora_t=bits_to_torch(t), lora_b=bits_to_torch(b),
                    lora_scale=s)
    rows = np.arange(M) if M <= 256 else np.sort(np.random.default_rng(M + N).choice(M, size=64, replace=False))
    rows[-1] = M - 1
    tv, bv = bf16_values(t)[rows], bf16_values(b)
    term, tabs, _ = olora.lora_term(tv, bv.T, s)
    bound = tol.gemm_bound(term, tabs)
    assert_within(torch_bf16_to_f64(y)[rows], term, bound, f"lora s={s} {M}x{N}x{K}")
    if s != 2.0:
        # the planted mistake: s T / r_A rounded once to BF16, then exact products
        f = (np.float32(s) * (np.float32(1.0) / xq.rscale[rows])).astype(np.float32)
        hi = synth.bf16_round((tv * f[:, None]).astype(np.float32)).astype(np.float64)
        wrong = synth.bf16_round(((hi * xq.rscale[rows].astype(np.float64)[:, None]) @ bv.T.astype(np.float64))
                                 .astype(np.float32)).astype(np.float64)
        assert tol.violations(wrong, term, bound)[0] > 0, "the case does not separate FP32 from BF16 scaling"

@pytest.mark.parametrize("M,N,K,r", [(80, 192, 272, 16), (200, 512, 320, 16), (64, 768, 1100, 5)])
def test_dgrad_accumulate_and_lora(fw, M, N, K, r):
    """N is the contraction length of the input gradient: 192 and 1100 take the
    generic kernel, 512 and 768 the direct-to-LDS one (ragged output tiles)."""
    dy = synth.normal_bf16((M, N), 0.01, 94, 1)
    w = synth.normal_bf16((N, K), 0.02, 94, 2)
    dt = synth.normal_bf16((M, r), 0.01, 94, 3)
    A = synth.normal_bf16((r, K), 0.01, 94, 4)
    prev = synth.normal_bf16((M, K), 0.001, 94, 5)
    dyq, wb = _q(dy), _qt(w)
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb), out=out, accumulate=True,
                  lora_dt=bits_to_torch(dt), lora_a=bits_to_torch(A))
    dref, dabs = ogemm.gemm_dgrad(dyq, wb)
    term, tabs, _ = olora.lora_term(bf16_values(dt), bf16_values(A), 1.0)
    want = bf16_values(prev).astype(np.float64) + dref + term
    # accumulate rounds once: the previous value enters exactly, so the bound is the same
    assert_within(torch_bf16_to_f64(out), want, tol.gemm_bound(want, dabs + tabs), "dgrad acc+lora")


LLAMA3B = [("q/o", 3072, 3072), ("k/v", 3072, 1024), ("gate/up", 3072, 8192), ("down", 8192, 3072)]


@pytest.mark.parametrize("name,d_in,d_out", LLAMA3B)
def test_llama3b_full_size_sampled(fw, name, d_in, d_out):
    """Full Llama-3B projection shapes at M = 4096 (the benchmark's launches);
    64 sampled rows of Y and dX against the oracle."""
    M = 4096
    wl = synth.WORKLOADS[2]
    x = synth.workload_activation(wl, M, d_in, 601)
    w = synth.normal_bf16((d_out, d_in), 0.02, 2, 602)
    dy = synth.normal_bf16((M, d_out), 0.01, 2, 603)
    xq, wf, wb, dyq = _q(x), _q(w), _qt(w), _q(dy)
    y = fw.gemm_fwd(nvfp4_to_gpu(xq), nvfp4_to_gpu(wf))
    dx = fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb))
    rows = np.sort(np.random.default_rng(d_in + d_out).choice(M, size=64, replace=False))
    rows[-1] = M - 1
    ysub = torch_bf16_to_f64(y)[rows]
    dxsub = torch_bf16_to_f64(dx)[rows]
    sel = lambda q: onv.NVFP4(q.codes[rows], q.scales[rows], q.rscale[rows])
    yref, yabs = ogemm.gemm_nt(sel(xq), wf)
    assert_within(ysub, yref, tol.gemm_bound(yref, yabs), f"{name} fwd")
    dref, dabs = ogemm.gemm_nt(sel(dyq), wb)
    assert_within(dxsub, dref, tol.gemm_bound(dref, dabs), f"{name} dgrad")


@pytest.mark.parametrize("r", [64, 128])
@pytest.mark.parametrize("s", [2.0, 0.75])
@pytest.mark.parametrize("M,N,K", [(320, 640, 512), (200, 384, 272), (4096, 3072, 3072)])
def test_lora_epilogue_high_rank(fw, M, N, K, r, s):
    """The fused LoRA term at rank 64 (the 8B-scale workload's rank) and 128
    (the largest the library accepts), forward (s T B^T) and input gradient
    (dT A, accumulating), with a power-of-two and another scale.  K = 512 and
    3072 take the direct-to-LDS kernel (the 3072 case is a step shape, rows
    sampled), K = 272 the generic one (contraction not a multiple of 256)."""
    x = synth.activations_bf16((M, K), 97, M + K + r)
    w = synth.normal_bf16((N, K), 0.02, 97, M + K + r + 1)
    t = synth.normal_bf16((M, r), 0.3, 97, M + K + r + 2)
    b = synth.normal_bf16((N, r), 0.01, 97, M + K + r + 3)
    dy = synth.normal_bf16((M, N), 0.01, 97, M + K + r + 4)
    dt = synth.normal_bf16((M, r), 0.01, 97, M + K + r + 5)
    A = synth.normal_bf16((r, K), 0.01, 97, M + K + r + 6)
    prev = synth.normal_bf16((M, K), 0.001, 97, M + K + r + 7)
    xq, wf, wb, dyq = _q(x), _q(w), _qt(w), _q(dy)
    rows = np.arange(M) if M <= 512 else np.sort(np.random.default_rng(M + r).choice(M, size=48, replace=False))
    rows[-1] = M - 1
    sel = lambda q: onv.NVFP4(q.codes[rows], q.scales[rows], q.rscale[rows])
    y = fw.gemm_fwd(nvfp4_to_gpu(xq), nvfp4_to_gpu(wf), lora_t=bits_to_torch(t), lora_b=bits_to_torch(b),
                    lora_scale=s)
    yref, yabs = ogemm.gemm_nt(sel(xq), wf)
    term, tabs, _ = olora.lora_term(bf16_values(t)[rows], bf16_values(b).T, s)
    assert np.abs(term).max() > 0
    assert_within(torch_bf16_to_f64(y)[rows], yref + term, tol.gemm_bound(yref + term, yabs + tabs),
                  f"fwd r={r} s={s}")
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb), out=out, accumulate=True,
                  lora_dt=bits_to_torch(dt), lora_a=bits_to_torch(A))
    dref, dabs = ogemm.gemm_nt(sel(dyq), wb)
    dterm, dtabs, _ = olora.lora_term(bf16_values(dt)[rows], bf16_values(A), 1.0)
    want = bf16_values(prev)[rows].astype(np.float64) + dref + dterm
    assert_within(torch_bf16_to_f64(out)[rows], want, tol.gemm_bound(want, dabs + dtabs), f"dgrad r={r}")
