"""GPU parity: the decoder-MLP chain stage by stage, the 8B-scale and Llama-1B
shapes, and HIP-graph replays of the path.

Chain (PACT, Appendix Table 7, rows RMSNorm / Frozen projections /
SiLU-multiply / LoRA branch; abstract: NVFP4 RMSNorm outputs reused as the
projection input, gate/up saved in NVFP4): every GPU stage receives the
oracle's output of the previous stage (uploaded), so each comparison is at that
stage's own bound and no oracle input comes from the GPU.  Token rows are
independent in every stage, so a row sample of the full-size workload is an
exact sub-problem.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import backward as obwd
from oracle import fused as ofused
from oracle import gemm as ogemm
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


def _q(vals):
    return onv.quantize(np.asarray(vals, dtype=np.float64))


def _bits(vals64):
    """float64 values that are BF16-exact -> BF16 bits."""
    return synth.bf16_bits(np.asarray(vals64, dtype=np.float32))


def test_mlp_block_chain_stagewise(fw):
    """Llama-3B MLP block dims (hidden 3072, intermediate 8192), 192 token rows."""
    wl = synth.WORKLOADS[3]
    H, I, rows = 3072, 8192, 192
    x = synth.workload_activation(wl, rows, H, 800)
    g = synth.uniform_bf16((H,), 0.9, 1.1, wl.wid, 801)
    Wg = synth.normal_bf16((I, H), 0.02, wl.wid, 802)
    Wu = synth.normal_bf16((I, H), 0.02, wl.wid, 803)
    Wd = synth.normal_bf16((H, I), 0.02, wl.wid, 804)
    dOut = synth.normal_bf16((rows, H), 0.01, wl.wid, 805)
    gWg, gWu, gWd = (fw.weight_layouts(bits_to_torch(w)) for w in (Wg, Wu, Wd))
    oWg, oWu, oWd = (ogemm.weight_layouts(bf16_values(w).astype(np.float64)) for w in (Wg, Wu, Wd))
    for gl, ol, nm in ((gWg, oWg, "Wg"), (gWu, oWu, "Wu"), (gWd, oWd, "Wd")):
        assert_nvfp4_equal(gl[0], ol[0], nm + " fwd layout")
        assert_nvfp4_equal(gl[1], ol[1], nm + " bwd layout")

    # 1. RMSNorm -> NVFP4 (bit-exact codes and rstd)
    yq, rstd = fw.rmsnorm_quant(bits_to_torch(x), bits_to_torch(g), 1e-5)
    oyq, orstd, _ = ofused.rmsnorm_quant(bf16_values(x), bf16_values(g), 1e-5)
    assert_nvfp4_equal(yq, oyq, "rmsnorm y_q")
    assert np.array_equal(rstd.cpu().numpy().view(np.uint32), orstd.view(np.uint32))
    # 2. gate / up GEMMs from the oracle's y_q
    a = fw.gemm_fwd(nvfp4_to_gpu(oyq), nvfp4_to_gpu(oWg[0]))
    b = fw.gemm_fwd(nvfp4_to_gpu(oyq), nvfp4_to_gpu(oWu[0]))
    aref, aabs = ogemm.gemm_fwd(oyq, oWg[0])
    bref, babs = ogemm.gemm_fwd(oyq, oWu[0])
    assert_within(torch_bf16_to_f64(a), aref, tol.gemm_bound(aref, aabs), "gate out")
    assert_within(torch_bf16_to_f64(b), bref, tol.gemm_bound(bref, babs), "up out")
    # 3. SiLU-multiply -> NVFP4 from the oracle's BF16-rounded a, b
    a_bits, b_bits = _bits(tol.bf16_rne(aref)), _bits(tol.bf16_rne(bref))
    hq, gq, uq = fw.silu_mul_quant(bits_to_torch(a_bits), bits_to_torch(b_bits))
    ohq, ogq, ouq, _ = ofused.silu_mul_quant(bf16_values(a_bits), bf16_values(b_bits))
    assert_nvfp4_equal(hq, ohq, "h_q")
    assert_nvfp4_equal(gq, ogq, "gate_q")
    assert_nvfp4_equal(uq, ouq, "up_q")
    # 4. down GEMM
    out = fw.gemm_fwd(nvfp4_to_gpu(ohq), nvfp4_to_gpu(oWd[0]))
    oref, oabs = ogemm.gemm_fwd(ohq, oWd[0])
    assert_within(torch_bf16_to_f64(out), oref, tol.gemm_bound(oref, oabs), "down out")
    # 5. backward: dOut -> NVFP4 -> down dgrad
    dOq = fw.quantize(bits_to_torch(dOut))
    odOq = _q(bf16_values(dOut))
    assert_nvfp4_equal(dOq, odOq, "dOut_q")
    dh = fw.gemm_dgrad(nvfp4_to_gpu(odOq), nvfp4_to_gpu(oWd[1]))
    dhref, dhabs = ogemm.gemm_dgrad(odOq, oWd[1])
    assert_within(torch_bf16_to_f64(dh), dhref, tol.gemm_bound(dhref, dhabs), "dh")
    # 6. SiLU-multiply backward from the saved NVFP4 gate/up
    dh_bits = _bits(tol.bf16_rne(dhref))
    da, db = fw.silu_mul_bwd(nvfp4_to_gpu(ogq), nvfp4_to_gpu(ouq), bits_to_torch(dh_bits))
    daref, dbref, cda, cdb = obwd.silu_mul_bwd(ogq, ouq, bf16_values(dh_bits))
    assert_within(torch_bf16_to_f64(da), daref, tol.grad_bound(daref, cda), "dgate")
    assert_within(torch_bf16_to_f64(db), dbref, tol.grad_bound(dbref, cdb), "dup")
    # 7. quantize da, db; gate dgrad + up dgrad accumulated into one dy
    da_bits, db_bits = _bits(tol.bf16_rne(daref)), _bits(tol.bf16_rne(dbref))
    daq, dbq = fw.quantize(bits_to_torch(da_bits)), fw.quantize(bits_to_torch(db_bits))
    odaq, odbq = _q(bf16_values(da_bits)), _q(bf16_values(db_bits))
    assert_nvfp4_equal(daq, odaq, "da_q")
    assert_nvfp4_equal(dbq, odbq, "db_q")
    dy1 = fw.gemm_dgrad(nvfp4_to_gpu(odaq), nvfp4_to_gpu(oWg[1]))
    y1, y1abs = ogemm.gemm_dgrad(odaq, oWg[1])
    assert_within(torch_bf16_to_f64(dy1), y1, tol.gemm_bound(y1, y1abs), "dy (gate)")
    y1_bits = _bits(tol.bf16_rne(y1))
    dy = bits_to_torch(y1_bits).clone()
    fw.gemm_dgrad(nvfp4_to_gpu(odbq), nvfp4_to_gpu(oWu[1]), out=dy, accumulate=True)
    y2, y2abs = ogemm.gemm_dgrad(odbq, oWu[1])
    want = bf16_values(y1_bits).astype(np.float64) + y2
    assert_within(torch_bf16_to_f64(dy), want, tol.gemm_bound(want, y2abs), "dy (gate + up)")
    # 8. RMSNorm backward from y_q and rstd
    dy_bits = _bits(tol.bf16_rne(want))
    dx = fw.rmsnorm_bwd(nvfp4_to_gpu(oyq), torch.from_numpy(orstd).cuda(), bits_to_torch(g), bits_to_torch(dy_bits))
    dxref, cancel = obwd.rmsnorm_bwd(oyq, orstd, bf16_values(g), bf16_values(dy_bits))
    assert_within(torch_bf16_to_f64(dx), dxref, tol.grad_bound(dxref, cancel), "dx")


def _sampled_fwd_dgrad(fw, wl, M, d_in, d_out, seed, what):
    """Full-size fwd and dgrad launches; 48 sampled token rows x 384 sampled output
    columns checked against the oracle.  Quantization is per row of X, dY, W
    (W_fwd) and of W^T (W_bwd), so the oracle needs only the sampled rows of
    each operand: an exact sub-problem of the full-size product."""
    x = synth.workload_activation(wl, M, d_in, seed)
    w = synth.normal_bf16((d_out, d_in), 0.02, wl.wid, seed + 1)
    dy = synth.normal_bf16((M, d_out), 0.01, wl.wid, seed + 2)
    gx, gdy = fw.quantize(bits_to_torch(x)), fw.quantize(bits_to_torch(dy))
    gwf, gwb = fw.weight_layouts(bits_to_torch(w))
    y, dx = fw.gemm_fwd(gx, gwf), fw.gemm_dgrad(gdy, gwb)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=48, replace=False))
    ncols = np.sort(rng.choice(d_out, size=384, replace=False))
    kcols = np.sort(rng.choice(d_in, size=384, replace=False))
    wv = bf16_values(w).astype(np.float64)
    oxq, odyq = _q(bf16_values(x[rows])), _q(bf16_values(dy[rows]))
    owf = _q(wv[ncols])                        # rows ncols of W_fwd = Q(W)
    owb = _q(np.ascontiguousarray(wv[:, kcols].T))   # rows kcols of W_bwd = Q(W^T)
    assert_nvfp4_equal(gx, oxq, what + " x_q", rows=rows)
    assert_nvfp4_equal(gdy, odyq, what + " dy_q", rows=rows)
    assert_nvfp4_equal(gwf, owf, what + " W_fwd", rows=ncols)
    assert_nvfp4_equal(gwb, owb, what + " W_bwd", rows=kcols)
    yref, yabs = ogemm.gemm_fwd(oxq, owf)
    assert_within(torch_bf16_to_f64(y)[np.ix_(rows, ncols)], yref, tol.gemm_bound(yref, yabs), what + " fwd")
    dref, dabs = ogemm.gemm_dgrad(odyq, owb)
    assert_within(torch_bf16_to_f64(dx)[np.ix_(rows, kcols)], dref, tol.gemm_bound(dref, dabs), what + " dgrad")


@pytest.mark.parametrize("name,d_in,d_out", [("gate/up", 4096, 14336), ("down", 14336, 4096), ("k/v", 4096, 1024)])
def test_8b_scale_gemms_sampled(fw, name, d_in, d_out):
    """8B-scale projections at M = 16384 with Student-t (nu = 3) activations."""
    _sampled_fwd_dgrad(fw, synth.WORKLOADS[4], 16384, d_in, d_out, 820, "8B " + name)


def test_8b_scale_lora_rank64(fw):
    """LoRA rank 64 branch at 8B widths (K = 4096, N = 14336), 512 token rows."""
    M, K, N, r, s = 512, 4096, 14336, 64, 0.5
    wl = synth.WORKLOADS[4]
    x = synth.workload_activation(wl, M, K, 830)
    A = synth.normal_bf16((r, K), 0.01, wl.wid, 831)
    B = synth.normal_bf16((N, r), 0.01, wl.wid, 832)
    dy = synth.normal_bf16((M, N), 0.01, wl.wid, 833)
    xq = _q(bf16_values(x))
    gx = nvfp4_to_gpu(xq)
    T = fw.lora_down(gx, bits_to_torch(A))
    t_exact, _, t_abs = olora.lora_down(xq, bf16_values(A))
    assert_within(torch_bf16_to_f64(T), t_exact, tol.gemm_bound(t_exact, t_abs), "T r64")
    dT, dA, dB = fw.lora_bwd(gx, bits_to_torch(A), bits_to_torch(B), bits_to_torch(dy), s)
    ref = olora.lora_bwd(xq, bf16_values(A), bf16_values(B), bf16_values(dy), s)
    assert_within(torch_bf16_to_f64(dT), ref["dT_exact"], tol.gemm_bound(ref["dT_exact"], ref["dT_abs"]), "dT")
    assert_within(torch_bf16_to_f64(dB), ref["dB_exact"],
                  tol.gemm_bound(ref["dB_exact"], ref["dB_abs"], ref["dB_tslack"]), "dB")
    assert_within(torch_bf16_to_f64(dA), ref["dA_exact"],
                  tol.gemm_bound(ref["dA_exact"], ref["dA_abs"], ref["dA_tslack"]), "dA")


@pytest.mark.parametrize("name,d_in,d_out", [("k/v", 2048, 512), ("gate/up", 2048, 8192), ("down", 8192, 2048)])
def test_llama1b_gemms_sampled(fw, name, d_in, d_out):
    """Llama-1B projection shapes at M = 4096."""
    _sampled_fwd_dgrad(fw, synth.WORKLOADS[1], 4096, d_in, d_out, 840, "1B " + name)


def test_graph_replays_match_eager(fw):
    """A captured HIP graph of the LoRA linear layer (quantize, lora_down, fwd GEMM
    with LoRA term, dY quantize, lora_bwd, dgrad with LoRA term) replayed several
    times, with eager work and synchronizations between replays: every replay
    must reproduce the eager results bit for bit."""
    M, K, N, r = 512, 3072, 1024, 16
    x = bits_to_torch(synth.activations_bf16((M, K), 97, 1))
    w = bits_to_torch(synth.normal_bf16((N, K), 0.02, 97, 2))
    dy = bits_to_torch(synth.normal_bf16((M, N), 0.01, 97, 3))
    A = bits_to_torch(synth.normal_bf16((r, K), 0.01, 97, 4))
    B = bits_to_torch(synth.normal_bf16((N, r), 0.01, 97, 5))
    wf, wb = fw.weight_layouts(w)
    xq, dyq = fw.empty_nvfp4(M, K), fw.empty_nvfp4(M, N)
    T = torch.empty((M, r), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    outs = (torch.empty((M, r), dtype=torch.bfloat16, device="cuda"),
            torch.empty((r, K), dtype=torch.bfloat16, device="cuda"),
            torch.empty((N, r), dtype=torch.bfloat16, device="cuda"))
    ws = fw.lora_bwd_workspace(M, K, N, r)

    def step():
        fw.quantize(x, out=xq)
        fw.lora_down(xq, A, out=T)
        fw.gemm_fwd(xq, wf, lora_t=T, lora_b=B, lora_scale=2.0, out=Y)
        fw.quantize(dy, out=dyq)
        fw.lora_bwd(xq, A, B, dy, 2.0, out=outs, workspace=ws)
        fw.gemm_dgrad(dyq, wb, out=dX, lora_dt=outs[0], lora_a=A)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (xq.codes, xq.scales, T, Y, dX, *outs)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (T, Y, dX, *outs):
            t.fill_(0)
        _ = (x.float() * 2).sum()            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (xq.codes, xq.scales, T, Y, dX, *outs)
        for i, (a, b) in enumerate(zip(got, ref)):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager result"
