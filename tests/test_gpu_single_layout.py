"""GPU parity: single-layout input gradient dX = deq(dY_q) deq(W_fwd) over the
forward weight layout only (nvfp4_gemm_dgrad_fwd_layout).

Bound as for the frozen GEMMs: |dx - ref| <= ulp_bf16(ref) + 1e-5 * sum |a b|
(+ the LoRA term's share).  Operands are quantized by the oracle and uploaded
for the small cases; the Llama-3B cases quantize on the GPU and check sampled
rows x columns against an exact sub-problem (quantization is per row of W_fwd:
the blocks holding the sampled columns plus the block holding each row's
maximum reproduce every row's scales).
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


@pytest.mark.parametrize("M,N,K", [(64, 256, 128), (1, 256, 64), (200, 512, 320), (300, 768, 1088),
                                   (513, 1024, 3072), (130, 2048, 192)])
def test_shapes(fw, M, N, K):
    dy = synth.normal_bf16((M, N), 0.01, 88, M + N)
    w = synth.normal_bf16((N, K), 0.02, 88, M + N + 1)
    dyq, wf = _q(dy), _q(w)
    sw = fw.SingleLayoutWeight(nvfp4_to_gpu(wf))
    nz = wf.scales.any(axis=1)
    emax = int(np.max(np.frexp(wf.rscale.astype(np.float64))[1][nz] - 1))
    assert int(sw.exp_max.item()) == emax, "largest row exponent over nonzero rows"
    dx = fw.gemm_dgrad_fwd_layout(nvfp4_to_gpu(dyq), sw)
    ref, rabs = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    assert_within(torch_bf16_to_f64(dx), ref, tol.gemm_bound(ref, rabs), f"{M}x{N}x{K}")


def test_row_scale_spread_and_zero_rows(fw):
    """Rows of W at scales 2^-14 .. 2^0 of each other (every B element exact in
    FP16), all-zero rows, and zero dY rows."""
    M, N, K = 96, 512, 256
    rng = np.random.default_rng(89)
    w = bf16_values(synth.normal_bf16((N, K), 0.02, 88, 3)).astype(np.float64)
    w *= np.exp2(-rng.integers(0, 15, size=(N, 1)))
    w[5] = 0.0
    w[300] = 0.0
    dyv = bf16_values(synth.normal_bf16((M, N), 0.01, 88, 4)).astype(np.float64)
    dyv[7] = 0.0
    wf, dyq = onv.quantize(w), onv.quantize(dyv)
    sw = fw.SingleLayoutWeight(nvfp4_to_gpu(wf))
    nz = wf.scales.any(axis=1)
    assert int(sw.exp_max.item()) == int(np.max(np.frexp(wf.rscale.astype(np.float64))[1][nz] - 1))
    dx = fw.gemm_dgrad_fwd_layout(nvfp4_to_gpu(dyq), sw)
    ref, rabs = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    assert_within(torch_bf16_to_f64(dx), ref, tol.gemm_bound(ref, rabs), "spread rows")
    assert torch.count_nonzero(dx[7]).item() == 0


def test_exponent_window_is_enforced(fw):
    """Nonzero rows 2^20 apart in row scale (beyond the 2^14 window in which
    the FP16 weight operand is exact): the set-up call refuses the weight,
    and the kernel, launched anyway with that weight's largest exponent,
    writes NaN rather than a rounded gradient.  The oracle's exact product is
    finite and nonzero there."""
    M, N, K = 64, 512, 128
    w = bf16_values(synth.normal_bf16((N, K), 0.02, 88, 21)).astype(np.float64)
    w[N // 2:] *= 2.0 ** -20
    dyv = bf16_values(synth.normal_bf16((M, N), 0.01, 88, 22)).astype(np.float64)
    wf, dyq = onv.quantize(w), onv.quantize(dyv)
    gw = nvfp4_to_gpu(wf)
    with pytest.raises(fw._lib.PactError) as ei:
        fw.SingleLayoutWeight(gw)
    assert ei.value.status == -5
    sw = fw.SingleLayoutWeight.__new__(fw.SingleLayoutWeight)
    sw.w_fwd = gw
    sw.exp_range = torch.empty((2,), dtype=torch.int32, device="cuda")
    sw.exp_max = sw.exp_range[:1]
    lib = fw._lib.load()
    st = lib.pact_nvfp4_row_exp_max(*gw.ptrs(), N, K, sw.exp_range.data_ptr(), None)
    assert st == -5
    lo, hi = np.frexp(wf.rscale.astype(np.float64))[1].min() - 1, np.frexp(wf.rscale.astype(np.float64))[1].max() - 1
    assert sw.exp_range.cpu().tolist() == [hi, lo] and hi - lo >= 20
    dx = fw.gemm_dgrad_fwd_layout(nvfp4_to_gpu(dyq), sw)
    assert torch.isnan(dx.float()).all(), "an inexact launch must not return numbers"
    ref, _ = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    assert np.all(np.isfinite(ref)) and np.abs(ref).max() > 0


def test_accumulate_and_lora(fw):
    M, N, K, r = 160, 512, 384, 16
    dy = synth.normal_bf16((M, N), 0.01, 88, 10)
    w = synth.normal_bf16((N, K), 0.02, 88, 11)
    dt = synth.normal_bf16((M, r), 0.01, 88, 12)
    A = synth.normal_bf16((r, K), 0.01, 88, 13)
    prev = synth.normal_bf16((M, K), 0.001, 88, 14)
    dyq, wf = _q(dy), _q(w)
    sw = fw.SingleLayoutWeight(nvfp4_to_gpu(wf))
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad_fwd_layout(nvfp4_to_gpu(dyq), sw, out=out, accumulate=True, lora_dt=bits_to_torch(dt),
                             lora_a=bits_to_torch(A))
    ref, rabs = ogemm.gemm_dgrad_fwd_layout(dyq, wf)
    term, tabs, _ = olora.lora_term(bf16_values(dt), bf16_values(A), 1.0)
    want = bf16_values(prev).astype(np.float64) + ref + term
    assert_within(torch_bf16_to_f64(out), want, tol.gemm_bound(want, rabs + tabs), "accumulate + LoRA")


def _wfwd_columns(wv, kcols):
    """deq(Q(W))[:, kcols] from an exact sub-problem: the 16-column blocks holding
    kcols plus, per row, the block holding the row's maximum (same row scale)."""
    N, K = wv.shape
    blocks = np.unique(kcols // 16)
    blk = wv.reshape(N, K // 16, 16)
    amax_blk = np.abs(wv).argmax(axis=1) // 16
    sub = np.concatenate([blk[:, blocks, :].reshape(N, -1), blk[np.arange(N), amax_blk, :]], axis=1)
    d = onv.dequantize(onv.quantize(sub))[:, :blocks.size * 16]
    pos = {b: i for i, b in enumerate(blocks)}
    idx = np.array([pos[k // 16] * 16 + k % 16 for k in kcols])
    return d[:, idx]


@pytest.mark.parametrize("name,N,K", [("q/o", 3072, 3072), ("k/v", 1024, 3072), ("gate/up", 8192, 3072),
                                      ("down", 3072, 8192)])
def test_llama3b_sampled(fw, name, N, K):
    """Llama-3B input gradients at M = 4096 (N = the projection's output width,
    K its input width): GPU-quantized dY and W_fwd, 48 rows x 256 columns."""
    M, seed = 4096, 77 + N + K
    wl = synth.WORKLOADS[2]
    dy = synth.normal_bf16((M, N), wl.dy_std, wl.wid, seed)
    w = synth.normal_bf16((N, K), wl.w_std, wl.wid, seed + 1)
    gdyq = fw.quantize(bits_to_torch(dy))
    sw = fw.SingleLayoutWeight(fw.quantize(bits_to_torch(w)))
    dx = fw.gemm_dgrad_fwd_layout(gdyq, sw)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=48, replace=False))
    rows[-1] = M - 1
    kcols = np.sort(rng.choice(K, size=256, replace=False))
    kcols[-1] = K - 1
    wsub = _wfwd_columns(bf16_values(w).astype(np.float64), kcols)
    a = onv.dequantize(onv.quantize(bf16_values(dy[rows]).astype(np.float64)))
    ref, rabs = a @ wsub, np.abs(a) @ np.abs(wsub)
    assert_within(torch_bf16_to_f64(dx)[np.ix_(rows, kcols)], ref, tol.gemm_bound(ref, rabs), name)
