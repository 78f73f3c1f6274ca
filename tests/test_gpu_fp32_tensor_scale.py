"""GPU parity: the NVFP4 recipe with a conventional FP32 tensor scale.

* nvfp4_quantize_ex with PACT_QUANT_TENSOR_SCALE_FP32: stored scale
  S = RN32(amax / 2688), multiplier R = RN32(1 / S), scaled magnitudes
  u = RN32(|x| R), then the block rules on u; bit-exact against the oracle's
  quantizer with the same options, row-wise (every row kernel) and
  transposed, computed and supplied maxima, round-up scales, and the edge
  cases (zero tensor, tiny maximum where S is raised to 2^-126, huge values).
* The GEMMs on such operands (row scales that are not powers of two):
  forward and input gradient within the GEMM bound against the oracle's
  float64 product, without LoRA on both kernels, with the fused LoRA term
  (power-of-two and other scale) through PACT_GEMM_ANY_ROW_SCALES; without
  that flag the direct-to-LDS kernel writes NaN rather than a rounded term.
* Entry points that need power-of-two row scales say so: the segmented input
  gradient writes NaN with two or more segments (and equals the single GEMM
  with one), and pact_nvfp4_row_exp_max refuses such a weight.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
from oracle import lora as olora
from oracle import nvfp4 as onv
from oracle import tolerance as tol

from gpu_util import assert_nvfp4_equal, assert_within, bf16_values, bits_to_torch, nvfp4_to_gpu, torch_bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _vals(bits):
    return bf16_values(bits).astype(np.float64)


def _q32(bits, transpose=False, amax="auto", round_up=False):
    return onv.quantize(_vals(bits), transpose=transpose, round_up=round_up, tensor_amax=amax,
                        fp32_tensor_scale=True)


@pytest.mark.parametrize("round_up", [False, True])
@pytest.mark.parametrize("rows,cols", [(33, 272), (300, 1024), (5, 8192), (3, 20480), (64, 96)])
def test_quantize_rows(fw, rows, cols, round_up):
    bits = synth.activations_bf16((rows, cols), 98, rows * 5 + cols)
    x = bits_to_torch(bits)
    amax = torch.empty((), dtype=torch.float32, device="cuda")
    q = fw.quantize_ex(x, round_up=round_up, tensor_scale=True, fp32_scale=True, amax=amax)
    assert amax.item() == float(np.abs(bf16_values(bits)).max())
    ref = _q32(bits, round_up=round_up)
    assert float(ref.rscale[0]) != 2.0 ** np.round(np.log2(float(ref.rscale[0]))), "scale is a power of two"
    assert_nvfp4_equal(q, ref, f"fp32 tensor scale round_up={round_up}")
    # a supplied maximum that is not a BF16 value
    sup = torch.tensor(float(np.float32(amax.item() * 1.3371)), dtype=torch.float32, device="cuda")
    qs = fw.quantize_ex(x, round_up=round_up, tensor_scale=True, fp32_scale=True, amax=sup, compute_amax=False)
    assert_nvfp4_equal(qs, _q32(bits, amax=sup.item(), round_up=round_up), "supplied amax")


@pytest.mark.parametrize("round_up", [False, True])
def test_quantize_transposed(fw, round_up):
    w = synth.normal_bf16((272, 200), 0.02, 98, 7)          # W [N x K]; Q(W^T) is [200 x 272]
    q = fw.quantize_ex(bits_to_torch(w), transpose=True, round_up=round_up, tensor_scale=True, fp32_scale=True)
    assert_nvfp4_equal(q, _q32(w, transpose=True, round_up=round_up), "transposed fp32 tensor scale")


def test_quantize_edge_cases(fw):
    rng = np.random.default_rng(98)
    cases = {
        "zero": np.zeros((4, 64), np.float32),
        "tiny": (rng.standard_normal((4, 64)) * 2.0 ** -120).astype(np.float32),   # S raised to 2^-126
        "huge": (rng.standard_normal((4, 64)) * 2.0 ** 120).astype(np.float32),
        # amax 2688: S = R = 1, u = |x|; blocks with maximum 6 (s = 1) hold every E2M1 midpoint
        "ties": np.tile(np.array([2688.0] + [1.0] * 15 + [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75,
                                                           -1.25, -1.75, -2.5, -3.5, -5.0, -0.0] * 3, np.float32),
                        (4, 1)),
    }
    for name, v in cases.items():
        bits = synth.bf16_bits(v)
        q = fw.quantize_ex(bits_to_torch(bits), tensor_scale=True, fp32_scale=True)
        assert_nvfp4_equal(q, _q32(bits), name)


def test_flag_validation(fw):
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fw.quantize_ex(x, fp32_scale=True)                   # needs the tensor-scale flag
    from frozen_weight_gemms_amd import _lib
    q = fw.empty_nvfp4(4, 64)
    with pytest.raises(_lib.PactError):
        _lib.call("nvfp4_quantize_ex", x.data_ptr(), 4, 64, 64, 0, 8, 0, *q.ptrs(), 0)


@pytest.mark.parametrize("K", [512, 272])
@pytest.mark.parametrize("r,s", [(16, 2.0), (64, 0.75)])
def test_gemms_on_fp32_scaled_operands(fw, K, r, s):
    """Forward (s T B^T) and input gradient (dT A, accumulating) with every
    operand carrying a non-power-of-two row scale; K = 512 takes the
    direct-to-LDS kernel, 272 the generic one.  The activations keep the
    power-of-two row rule in one case (mixed recipes)."""
    M, N = 300, 320
    x = synth.activations_bf16((M, K), 96, K + r)
    w = synth.normal_bf16((N, K), 0.02, 96, K + r + 1)
    t = synth.normal_bf16((M, r), 0.3, 96, K + r + 2)
    b = synth.normal_bf16((N, r), 0.01, 96, K + r + 3)
    dy = synth.normal_bf16((M, N), 0.01, 96, K + r + 4)
    dt = synth.normal_bf16((M, r), 0.01, 96, K + r + 5)
    A = synth.normal_bf16((r, K), 0.01, 96, K + r + 6)
    prev = synth.normal_bf16((M, K), 0.001, 96, K + r + 7)
    wf, wb, dyq = _q32(w), _q32(w, transpose=True), _q32(dy)
    lt, lb = bits_to_torch(t), bits_to_torch(b)
    for xq in (_q32(x), onv.quantize(_vals(x))):
        gx, gw = nvfp4_to_gpu(xq), nvfp4_to_gpu(wf)
        y = fw.gemm_fwd(gx, gw, lora_t=lt, lora_b=lb, lora_scale=s, any_row_scales=True)
        yref, yabs = ogemm.gemm_nt(xq, wf)
        term, tabs, _ = olora.lora_term(bf16_values(t), bf16_values(b).T, s)
        assert_within(torch_bf16_to_f64(y), yref + term, tol.gemm_bound(yref + term, yabs + tabs),
                      f"fwd K={K} r={r} s={s}")
        y0 = fw.gemm_fwd(gx, gw)
        assert_within(torch_bf16_to_f64(y0), yref, tol.gemm_bound(yref, yabs), "fwd without LoRA")
        yf = fw.gemm_fwd(gx, gw, lora_t=lt, lora_b=lb, lora_scale=s)          # no flag
        if K % 256 == 0:
            assert torch.isnan(yf.float()).all().item(), "fused term on non-power-of-two scales must give NaN"
        else:                                                                   # register-staged kernel anyway
            assert torch.equal(yf, y)
    out = bits_to_torch(prev).clone()
    fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb), out=out, accumulate=True,
                  lora_dt=bits_to_torch(dt), lora_a=bits_to_torch(A), any_row_scales=True)
    dref, dabs = ogemm.gemm_nt(dyq, wb)
    dterm, dtabs, _ = olora.lora_term(bf16_values(dt), bf16_values(A), 1.0)
    want = bf16_values(prev).astype(np.float64) + dref + dterm
    assert_within(torch_bf16_to_f64(out), want, tol.gemm_bound(want, dabs + dtabs), f"dgrad K={K} r={r}")
    d0 = fw.gemm_dgrad(nvfp4_to_gpu(dyq), nvfp4_to_gpu(wb))
    assert_within(torch_bf16_to_f64(d0), dref, tol.gemm_bound(dref, dabs), "dgrad without LoRA")


def test_entry_points_that_need_power_of_two_scales(fw):
    M, K = 256, 512
    ns = (256, 512)
    segs = []
    for i, n in enumerate(ns):
        dy = synth.normal_bf16((M, n), 0.01, 95, 10 + i)
        w = synth.normal_bf16((n, K), 0.02, 95, 20 + i)
        segs.append((_q32(dy), _q32(w, transpose=True), w))
    # one segment: the same kernel path as the plain input gradient, any row scale
    one = fw.gemm_dgrad_multi([(nvfp4_to_gpu(segs[0][0]), nvfp4_to_gpu(segs[0][1]))])
    ref, rabs = ogemm.gemm_nt(segs[0][0], segs[0][1])
    assert_within(torch_bf16_to_f64(one), ref, tol.gemm_bound(ref, rabs), "one segment")
    # two segments: NaN (the carried partial sum needs power-of-two scales)
    two = fw.gemm_dgrad_multi([(nvfp4_to_gpu(a), nvfp4_to_gpu(b)) for a, b, _ in segs])
    assert torch.isnan(two.float()).all().item(), "segmented dgrad must refuse non-power-of-two row scales"
    # the single-layout weight set-up refuses a W_fwd with such row scales
    from frozen_weight_gemms_amd import _lib
    wf = nvfp4_to_gpu(_q32(segs[0][2]))
    with pytest.raises(_lib.PactError) as e:
        fw.SingleLayoutWeight(wf)
    assert e.value.status == -5                    # PACT_EUNSUPPORTED
