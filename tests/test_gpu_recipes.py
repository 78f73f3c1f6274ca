"""GPU parity: NVFP4 recipe variants.

* nvfp4_quantize_ex: round-up block scales and one power-of-two scale per
  tensor (from a computed or supplied maximum), row-wise and transposed,
  bit-exact against the oracle's quantizer with the same options.
* Concatenated projection weights (Q/K/V and gate/up stacked along N): one
  forward GEMM serves the stacked projections (bit-identical to the separate
  GEMMs, LoRA terms included through a block-diagonal B) and one
  input-gradient GEMM sums every consumer's contribution before its single
  BF16 rounding (checked against the oracle's float64 product).
"""

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm
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


@pytest.mark.parametrize("round_up", [False, True])
@pytest.mark.parametrize("rows,cols", [(33, 272), (300, 1024), (3, 20480), (64, 96)])
def test_quantize_ex_rows(fw, rows, cols, round_up):
    bits = synth.activations_bf16((rows, cols), 99, rows * 7 + cols)
    x = bits_to_torch(bits)
    q = fw.quantize_ex(x, round_up=round_up)
    assert_nvfp4_equal(q, onv.quantize(_vals(bits), round_up=round_up), f"round_up={round_up}")
    amax = torch.empty((), dtype=torch.float32, device="cuda")
    qt = fw.quantize_ex(x, round_up=round_up, tensor_scale=True, amax=amax)
    assert amax.item() == float(np.abs(bf16_values(bits)).max()), "computed tensor maximum"
    assert_nvfp4_equal(qt, onv.quantize(_vals(bits), round_up=round_up, tensor_amax="auto"), "tensor scale")
    # a supplied maximum (4x the true one, e.g. from an upstream epilogue)
    sup = torch.tensor(4.0 * amax.item(), dtype=torch.float32, device="cuda")
    qs = fw.quantize_ex(x, round_up=round_up, tensor_scale=True, amax=sup, compute_amax=False)
    assert sup.item() == 4.0 * amax.item(), "supplied maximum left untouched"
    assert_nvfp4_equal(qs, onv.quantize(_vals(bits), round_up=round_up, tensor_amax=sup.item()), "supplied amax")


@pytest.mark.parametrize("round_up", [False, True])
def test_quantize_ex_transposed(fw, round_up):
    w = synth.normal_bf16((272, 200), 0.02, 99, 3)        # W [N x K]; W_bwd = Q(W^T) is [200 x 272]
    amax = torch.empty((), dtype=torch.float32, device="cuda")
    qt = fw.quantize_ex(bits_to_torch(w), transpose=True, round_up=round_up, tensor_scale=True, amax=amax)
    assert amax.item() == float(np.abs(bf16_values(w)).max())
    assert_nvfp4_equal(qt, onv.quantize(_vals(w), transpose=True, round_up=round_up, tensor_amax="auto"),
                       "transposed tensor scale")
    q = fw.quantize_ex(bits_to_torch(w), transpose=True, round_up=round_up)
    assert_nvfp4_equal(q, onv.quantize(_vals(w), transpose=True, round_up=round_up), "transposed")


def test_gemm_on_recipe_variants(fw):
    """The GEMM consumes any recipe's operands (row scales are per row either way)."""
    M, N, K = 200, 320, 512
    x = synth.activations_bf16((M, K), 99, 11)
    w = synth.normal_bf16((N, K), 0.02, 99, 12)
    gx = fw.quantize_ex(bits_to_torch(x), round_up=True, tensor_scale=True)
    gw = fw.quantize_ex(bits_to_torch(w), tensor_scale=True)
    y = fw.gemm_fwd(gx, gw)
    ox = onv.quantize(_vals(x), round_up=True, tensor_amax="auto")
    ow = onv.quantize(_vals(w), tensor_amax="auto")
    yref, yabs = ogemm.gemm_nt(ox, ow)
    assert_within(torch_bf16_to_f64(y), yref, tol.gemm_bound(yref, yabs), "fwd on variant operands")


def test_concatenated_qkv_forward_and_dgrad(fw):
    M, K, r, s = 256, 512, 16, 2.0
    widths = [512, 128, 128]                             # q, k, v output widths (kv heads narrower)
    ws = [synth.normal_bf16((n, K), 0.02, 99, 20 + i) for i, n in enumerate(widths)]
    As = [synth.normal_bf16((r, K), 0.01, 99, 30 + i) for i in range(3)]
    Bs = [synth.normal_bf16((n, r), 0.01, 99, 40 + i) for i, n in enumerate(widths)]
    x = bits_to_torch(synth.activations_bf16((M, K), 99, 50))
    xq = fw.quantize(x)
    # separate projections
    Ts = [fw.lora_down(xq, bits_to_torch(A)) for A in As]
    sep = [fw.gemm_fwd(xq, fw.quantize(bits_to_torch(w)), lora_t=T, lora_b=bits_to_torch(B), lora_scale=s)
           for w, T, B in zip(ws, Ts, Bs)]
    # stacked: W_cat [sum N x K], T_cat [M x 3r], B_cat block-diagonal [sum N x 3r]
    wcat = np.concatenate(ws, axis=0)
    gw_cat = fw.quantize(bits_to_torch(wcat))
    T_cat = torch.cat(Ts, dim=1).contiguous()
    Bcat = np.zeros((sum(widths), 3 * r), np.uint16)
    o = 0
    for i, (n, B) in enumerate(zip(widths, Bs)):
        Bcat[o:o + n, i * r:(i + 1) * r] = B
        o += n
    y_cat = fw.gemm_fwd(xq, gw_cat, lora_t=T_cat, lora_b=bits_to_torch(Bcat), lora_scale=s)
    assert torch.equal(y_cat.view(torch.int16), torch.cat(sep, dim=1).view(torch.int16)), \
        "stacked forward must equal the separate GEMMs bit for bit"
    # the stack launched as q plus k/v (row blocks of the stacked layout, the
    # matching rows of B_cat, column blocks of one output, the stacked T)
    y_two = torch.empty_like(y_cat)
    Bg = bits_to_torch(Bcat)
    for a, b in ((0, widths[0]), (widths[0], sum(widths))):
        part = fw.NVFP4Tensor(gw_cat.codes[a:b], gw_cat.scales[a:b], gw_cat.rscale[a:b])
        fw.gemm_fwd(xq, part, lora_t=T_cat, lora_b=Bg[a:b], lora_scale=s, out=y_two[:, a:b])
    assert torch.equal(y_two.view(torch.int16), y_cat.view(torch.int16)), \
        "the stack in two launches must equal one launch bit for bit"
    # input gradient: one GEMM over the stacked contraction sum(N)
    dys = [synth.normal_bf16((M, n), 0.01, 99, 60 + i) for i, n in enumerate(widths)]
    dy_cat = np.concatenate(dys, axis=1)
    dyq = onv.quantize(_vals(dy_cat))
    wb = onv.quantize(_vals(wcat), transpose=True)
    dx = fw.gemm_dgrad(nvfp4_to_gpu(dyq), fw.quantize(bits_to_torch(wcat), transpose=True))
    assert_nvfp4_equal(fw.quantize(bits_to_torch(wcat), transpose=True), wb, "stacked W_bwd")
    ref, rabs = ogemm.gemm_dgrad(dyq, wb)
    assert_within(torch_bf16_to_f64(dx), ref, tol.gemm_bound(ref, rabs), "stacked dgrad")
