"""GPU parity: pinned-FP32 backward kernels and their quantize-on-emit variants.

PACT, Appendix Table 7: RMSNorm / SiLU-multiply backward reconstruct in FP32
from the NVFP4 state and emit BF16 gradients; residual gradients accumulate in
BF16.  The kernels evaluate a pinned FP32 sequence (the oracle's ``*_f32``), so
their BF16 outputs are compared bit for bit, and so are the NVFP4 copies that
silu_mul_bwd_quant and rmsnorm_bwd_residual emit of them.  The float64
derivatives bound the pinned values as before (2 ulp_bf16 + cancellation).
"""

import numpy as np
import pytest
import torch

import synth
from oracle import backward as obwd
from oracle import fused as ofused
from oracle import nvfp4 as onv
from oracle import tolerance as tol

from gpu_util import (assert_nvfp4_equal, assert_within, bf16_values, bits_to_torch, nvfp4_to_gpu, torch_to_bits,
                      torch_bf16_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _q(bits):
    return onv.quantize(bf16_values(bits).astype(np.float64))


def _assert_bits(got_t, want_f32, what):
    got = torch_to_bits(got_t)
    want = synth.bf16_bits(np.asarray(want_f32, dtype=np.float32))
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, f"{what}: {bad.shape[0]} BF16 values differ, first {bad[:5].tolist()}"


def _silu_inputs(M, I, seed):
    a = synth.normal_bf16((M, I), 2.0, 98, seed)
    b = synth.normal_bf16((M, I), 1.0, 98, seed + 1)
    dh = synth.normal_bf16((M, I), 0.01, 98, seed + 2)
    if M >= 3:
        av = bf16_values(a).copy()
        av[0, :16] = [0, -0.0, 100, -100, 88, -88, 89.5, -89.5, 80.25, -80.25, 1e-30, -1e-30, 3, -3, 1e-3, -1e-3]
        a = synth.bf16_bits(av)
        dv = bf16_values(dh).copy()
        dv[1, :] = 0.0                                        # an all-zero gradient row
        dh = synth.bf16_bits(dv)
    return _q(a), _q(b), dh


@pytest.mark.parametrize("M,I", [(64, 256), (33, 8192), (5, 14336), (3, 16384), (7, 48)])
def test_silu_mul_bwd_bit_exact_and_fused_copies(fw, M, I):
    aq, bq, dh = _silu_inputs(M, I, I + 7)
    ga, gb, gdh = nvfp4_to_gpu(aq), nvfp4_to_gpu(bq), bits_to_torch(dh)
    dg, du = fw.silu_mul_bwd(ga, gb, gdh)
    rda, rdb = obwd.silu_mul_bwd_f32(aq, bq, bf16_values(dh))
    _assert_bits(dg, rda, "dgate (elementwise kernel)")
    _assert_bits(du, rdb, "dup (elementwise kernel)")
    ea, eb, ca, cb = obwd.silu_mul_bwd(aq, bq, bf16_values(dh))
    assert_within(torch_bf16_to_f64(dg), ea, tol.grad_bound(ea, ca), "dgate vs exact")
    assert_within(torch_bf16_to_f64(du), eb, tol.grad_bound(eb, cb), "dup vs exact")
    fg, fu, fgq, fuq = fw.silu_mul_bwd_quant(ga, gb, gdh)
    _, _, qa, qb = obwd.silu_mul_bwd_quant(aq, bq, bf16_values(dh))
    _assert_bits(fg, rda, "dgate (fused)")
    _assert_bits(fu, rdb, "dup (fused)")
    assert_nvfp4_equal(fgq, qa, "Q(dgate)")
    assert_nvfp4_equal(fuq, qb, "Q(dup)")


def _rms_state(M, H, seed):
    x = synth.workload_activation(synth.WORKLOADS[2], M, H, seed)
    g = synth.uniform_bf16((H,), 0.9, 1.1, 98, seed + 1)
    yq, rstd, _ = ofused.rmsnorm_quant(bf16_values(x), bf16_values(g), 1e-5)
    dy = synth.normal_bf16((M, H), 0.01, 98, seed + 2)
    resid = synth.normal_bf16((M, H), 0.01, 98, seed + 3)
    return yq, rstd, g, dy, resid


@pytest.mark.parametrize("M,H", [(257, 3072), (64, 2048), (9, 16384), (4, 48), (5, 8192), (7, 5120)])
def test_rmsnorm_bwd_bit_exact_and_residual(fw, M, H):
    yq, rstd, g, dy, resid = _rms_state(M, H, H + 11)
    gy, grs, gg, gdy, gres = (nvfp4_to_gpu(yq), torch.from_numpy(rstd).cuda(), bits_to_torch(g),
                              bits_to_torch(dy), bits_to_torch(resid))
    dx = fw.rmsnorm_bwd(gy, grs, gg, gdy)
    want = obwd.rmsnorm_bwd_f32(yq, rstd, bf16_values(g), bf16_values(dy))
    _assert_bits(dx, want, "rmsnorm_bwd")
    ref, cancel = obwd.rmsnorm_bwd(yq, rstd, bf16_values(g), bf16_values(dy))
    assert_within(torch_bf16_to_f64(dx), ref, tol.grad_bound(ref, cancel), "rmsnorm_bwd vs exact")
    # residual + NVFP4 copy
    out, q = fw.rmsnorm_bwd_residual(gy, grs, gg, gdy, resid=gres)
    rout, rq = obwd.rmsnorm_bwd_residual(yq, rstd, bf16_values(g), bf16_values(dy), bf16_values(resid))
    _assert_bits(out, rout, "rmsnorm_bwd + residual")
    assert_nvfp4_equal(q, rq, "Q(rmsnorm_bwd + residual)")
    # no residual, NVFP4 copy only
    out0, q0 = fw.rmsnorm_bwd_residual(gy, grs, gg, gdy)
    _assert_bits(out0, want, "rmsnorm_bwd_residual without residual")
    assert_nvfp4_equal(q0, _q(synth.bf16_bits(want)), "Q(rmsnorm_bwd)")
    # residual, no NVFP4 copy
    out1, q1 = fw.rmsnorm_bwd_residual(gy, grs, gg, gdy, resid=gres, quantize_out=False)
    assert q1 is None
    _assert_bits(out1, rout, "rmsnorm_bwd + residual (no copy)")


def test_residual_chain_full_size_sampled(fw):
    """Llama-3B MLP-block backward at M = 4096: silu_mul_bwd_quant on [4096 x 8192],
    then rmsnorm_bwd_residual on [4096 x 3072]; rows are independent, 64 sampled
    rows checked bit for bit (BF16 outputs and NVFP4 copies)."""
    M, I, H = 4096, 8192, 3072
    aq, bq, dh = _silu_inputs(M, I, 900)
    ga, gb = nvfp4_to_gpu(aq), nvfp4_to_gpu(bq)
    fg, fu, fgq, fuq = fw.silu_mul_bwd_quant(ga, gb, bits_to_torch(dh))
    yq, rstd, g, dy, resid = _rms_state(M, H, 910)
    out, q = fw.rmsnorm_bwd_residual(nvfp4_to_gpu(yq), torch.from_numpy(rstd).cuda(), bits_to_torch(g),
                                     bits_to_torch(dy), resid=bits_to_torch(resid))
    rows = np.sort(np.random.default_rng(912).choice(M, size=64, replace=False))
    rows[-1] = M - 1
    sel = lambda t: onv.NVFP4(t.codes[rows], t.scales[rows], t.rscale[rows])
    rda, rdb, qa, qb = obwd.silu_mul_bwd_quant(sel(aq), sel(bq), bf16_values(dh[rows]))
    _assert_bits(fg[rows.tolist()], rda, "dgate rows")
    _assert_bits(fu[rows.tolist()], rdb, "dup rows")
    assert_nvfp4_equal(fgq, qa, "Q(dgate) rows", rows=rows)
    assert_nvfp4_equal(fuq, qb, "Q(dup) rows", rows=rows)
    rout, rq = obwd.rmsnorm_bwd_residual(sel(yq), rstd[rows], bf16_values(g), bf16_values(dy[rows]),
                                         bf16_values(resid[rows]))
    _assert_bits(out[rows.tolist()], rout, "residual rows")
    assert_nvfp4_equal(q, rq, "Q(residual) rows", rows=rows)
