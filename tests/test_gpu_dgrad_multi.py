"""GPU parity: input gradient summed over projection segments in one launch
(nvfp4_gemm_dgrad_multi), e.g. q, k and v or gate and up, which all add into
the dX of one input.

Bound as for the frozen GEMMs: |dx - ref| <= ulp_bf16(ref) + 1e-5 * sum |a b|
(+ the LoRA terms' share), against the oracle's float64 sum over segments.
With one segment the kernel must reproduce nvfp4_gemm_dgrad bit for bit.
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


def _seg(M, n, K, seed, dy_scale=1.0):
    dy = bf16_values(synth.normal_bf16((M, n), 0.01, 96, seed)).astype(np.float64) * dy_scale
    w = bf16_values(synth.normal_bf16((n, K), 0.02, 96, seed + 1)).astype(np.float64)
    return onv.quantize(dy), onv.quantize(w, transpose=True)


@pytest.mark.parametrize("M,N,K", [(200, 512, 384), (64, 256, 3072), (300, 1024, 1024)])
def test_one_segment_equals_dgrad(fw, M, N, K):
    dyq, wb = _seg(M, N, K, 10 + M)
    gd, gw = nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb)
    r = 16
    dT = bits_to_torch(synth.normal_bf16((M, r), 0.01, 96, 3))
    A = bits_to_torch(synth.normal_bf16((r, K), 0.01, 96, 4))
    prev = bits_to_torch(synth.normal_bf16((M, K), 0.001, 96, 5))
    for lora in (None, (dT, A)):
        for acc in (False, True):
            o1, o2 = prev.clone(), prev.clone()
            fw.gemm_dgrad(gd, gw, out=o1, accumulate=acc, lora_dt=lora[0] if lora else None,
                          lora_a=lora[1] if lora else None)
            fw.gemm_dgrad_multi([(gd, gw)], out=o2, accumulate=acc, lora=[lora])
            assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"lora={lora is not None} acc={acc}"


# Segments of one, two, three and four stages (256 to 1024 wide) in several
# orders, with row scales spread across the segments.
@pytest.mark.parametrize("widths,scales", [((512, 256, 256), (1.0, 2.0 ** -12, 2.0 ** 8)),
                                           ((256, 768), (1.0, 1.0)),
                                           ((256, 256, 512, 256), (2.0 ** 20, 1.0, 2.0 ** -20, 4.0)),
                                           ((512, 512, 768), (2.0 ** -6, 1.0, 2.0 ** 10)),
                                           ((768, 512), (4.0, 2.0 ** -16)),
                                           ((768, 256, 1024), (1.0, 2.0 ** 12, 0.5))])
def test_segments_against_oracle(fw, widths, scales):
    M, K, r = 160, 640, 16
    segs = [_seg(M, n, K, 40 + 3 * i, sc) for i, (n, sc) in enumerate(zip(widths, scales))]
    lora, terms = [], []
    for i in range(len(widths)):
        if i == 1:
            lora.append(None)
            continue
        dT = synth.normal_bf16((M, r), 0.01, 96, 70 + i)
        A = synth.normal_bf16((r, K), 0.01, 96, 80 + i)
        lora.append((bits_to_torch(dT), bits_to_torch(A)))
        terms.append(olora.lora_term(bf16_values(dT), bf16_values(A), 1.0))
    prev = synth.normal_bf16((M, K), 0.001, 96, 90)
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad_multi([(nvfp4_to_gpu(d), nvfp4_to_gpu(w)) for d, w in segs], out=out, accumulate=True, lora=lora)
    ref, rabs = ogemm.gemm_dgrad_multi(segs)
    want = bf16_values(prev).astype(np.float64) + ref + sum(t for t, _, _ in terms)
    bound_abs = rabs + sum(a for _, a, _ in terms)
    assert_within(torch_bf16_to_f64(out), want, tol.gemm_bound(want, bound_abs), f"widths {widths}")


def _wbwd_rows(wv, kcols):
    """Rows kcols of Q(W^T): quantization runs along each row of W^T, so the
    sampled rows quantize exactly on their own."""
    return onv.dequantize(onv.quantize(wv.T[kcols]))


@pytest.mark.parametrize("name,widths,K", [("q/k/v", (3072, 1024, 1024), 3072), ("gate/up", (8192, 8192), 3072)])
def test_llama3b_sampled(fw, name, widths, K):
    """Llama-3B input gradients at M = 4096: GPU-quantized dY_i and W_bwd,i,
    48 rows x 192 columns checked against an exact sub-problem."""
    M = 4096
    wl = synth.WORKLOADS[2]
    rng = np.random.default_rng(sum(widths))
    rows = np.sort(rng.choice(M, size=48, replace=False))
    rows[-1] = M - 1
    kcols = np.sort(rng.choice(K, size=192, replace=False))
    kcols[-1] = K - 1
    segs, ref, rabs = [], 0.0, 0.0
    for i, n in enumerate(widths):
        dy = synth.normal_bf16((M, n), wl.dy_std, wl.wid, 500 + i)
        w = synth.normal_bf16((n, K), wl.w_std, wl.wid, 510 + i)
        segs.append((fw.quantize(bits_to_torch(dy)), fw.quantize(bits_to_torch(w), transpose=True)))
        a = onv.dequantize(onv.quantize(bf16_values(dy[rows]).astype(np.float64)))
        b = _wbwd_rows(bf16_values(w).astype(np.float64), kcols)
        ref = ref + a @ b.T
        rabs = rabs + np.abs(a) @ np.abs(b).T
    dx = fw.gemm_dgrad_multi(segs)
    assert_within(torch_bf16_to_f64(dx)[np.ix_(rows, kcols)], ref, tol.gemm_bound(ref, rabs), name)



@pytest.mark.parametrize("M,K,widths", [(2048, 12288, (512, 256, 256)), (4096, 2048, (256, 768)),
                                        (1024, 12288, (256, 256, 256, 256)), (4096, 3072, (256, 512))])
def test_segmented_tiles_sampled(fw, M, K, widths):
    """Every tile of the segmented kernel (256 x 192 in place of 256 x 256,
    256 x 128, 256 x 192), with row scales spread over 2^20 between segments,
    LoRA terms on some segments and accumulate; 48 rows x 160 columns against
    an exact sub-problem (quantization is per row of dY_i and of W_bwd,i)."""
    assert fw._lib.gemm_multi_tile(M, K) in ((256, 192), (256, 128))
    r = 16
    rng = np.random.default_rng(M + K + len(widths))
    rows = np.sort(rng.choice(M, size=48, replace=False))
    rows[-1] = M - 1
    kcols = np.sort(rng.choice(K, size=160, replace=False))
    kcols[-1] = K - 1
    spread = (1.0, 2.0 ** -12, 2.0 ** 8, 2.0 ** -4)
    segs, lora, ref, rabs = [], [], 0.0, 0.0
    for i, n in enumerate(widths):
        dyv = bf16_values(synth.normal_bf16((M, n), 0.01, 97, 10 * i + 1)).astype(np.float64) * spread[i]
        dy = synth.bf16_bits(dyv.astype(np.float32))
        w = synth.normal_bf16((n, K), 0.02, 97, 10 * i + 2)
        segs.append((fw.quantize(bits_to_torch(dy)), fw.quantize(bits_to_torch(w), transpose=True)))
        a = onv.dequantize(onv.quantize(bf16_values(dy[rows]).astype(np.float64)))
        b = _wbwd_rows(bf16_values(w).astype(np.float64), kcols)
        ref = ref + a @ b.T
        rabs = rabs + np.abs(a) @ np.abs(b).T
        if i % 2 == 0:
            dT = synth.normal_bf16((M, r), 0.01, 97, 10 * i + 3)
            A = synth.normal_bf16((r, K), 0.01, 97, 10 * i + 4)
            lora.append((bits_to_torch(dT), bits_to_torch(A)))
            t, tabs, _ = olora.lora_term(bf16_values(dT)[rows], bf16_values(A)[:, kcols], 1.0)
            ref, rabs = ref + t, rabs + tabs
        else:
            lora.append(None)
    prev = synth.normal_bf16((M, K), 0.001, 97, 99)
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad_multi(segs, out=out, accumulate=True, lora=lora)
    want = bf16_values(prev[np.ix_(rows, kcols)]).astype(np.float64) + ref
    assert_within(torch_bf16_to_f64(out)[np.ix_(rows, kcols)], want, tol.gemm_bound(want, rabs),
                  f"{M}x{K} widths {widths}")

def test_unsupported_width_is_rejected(fw):
    dyq, wb = _seg(64, 272, 256, 7)
    with pytest.raises(fw.PactError, match="multiple of 256"):
        fw.gemm_dgrad_multi([(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb))])


@pytest.mark.parametrize("r", [64, 128])
def test_segments_high_rank_lora(fw, r):
    """Segmented input gradient with rank-64 and rank-128 LoRA terms on every
    segment (and one segment without), against the oracle's sum."""
    M, K, widths = 192, 768, (512, 256, 256)
    segs = [_seg(M, n, K, 70 + 3 * i + r) for i, n in enumerate(widths)]
    lora, terms = [], []
    for i in range(len(widths)):
        if i == 1:
            lora.append(None)
            continue
        dT = synth.normal_bf16((M, r), 0.01, 96, 80 + i + r)
        A = synth.normal_bf16((r, K), 0.01, 96, 90 + i + r)
        lora.append((bits_to_torch(dT), bits_to_torch(A)))
        terms.append(olora.lora_term(bf16_values(dT), bf16_values(A), 1.0))
    out = fw.gemm_dgrad_multi([(nvfp4_to_gpu(a), nvfp4_to_gpu(b)) for a, b in segs], lora=lora)
    ref, rabs = ogemm.gemm_dgrad_multi(segs)
    for term, tabs, _ in terms:
        ref, rabs = ref + term, rabs + tabs
    assert_within(torch_bf16_to_f64(out), ref, tol.gemm_bound(ref, rabs), f"segments r={r}")
