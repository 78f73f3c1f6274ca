"""GPU parity for the MXFP4 variant: mxfp4_quantize and mxfp4_gemm against the oracle.

Format (PACT, Appendix Table 6, MXFP4 column): 32-element blocks, E2M1
elements, E8M0 block scales chosen by the OCP shared-exponent rule.  Codes and
scales must be bit-exact; GEMM outputs (FP32 accumulation, BF16 output) lie
within ulp_bf16(y_ref) + 1e-5 * sum_k |a_k b_k| of the oracle's float64 product.
Contraction lengths 128 .. 640 take every prologue / pipeline-depth case of
the kernel (1 .. 5 stages of 128).
"""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4 as omx
from oracle import tolerance as tol

from gpu_util import assert_within, bf16_values, bits_to_torch, dev, torch_bf16_to_f64

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_vectors.txt")


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _ox(bits):
    return omx.quantize(bf16_values(bits).astype(np.float64))


def _oxt(bits):
    return omx.quantize(bf16_values(bits).astype(np.float64), transpose=True)


def _to_gpu(q: omx.MXFP4):
    from frozen_weight_gemms_amd import MXFP4Tensor
    return MXFP4Tensor(torch.from_numpy(np.ascontiguousarray(q.codes)).to(dev()),
                       torch.from_numpy(np.ascontiguousarray(q.scales)).to(dev()))


def _assert_equal(gq, ref: omx.MXFP4, what="", rows=None):
    gc, gs = gq.codes.cpu().numpy(), gq.scales.cpu().numpy()
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert gc.shape == ref.codes.shape and gs.shape == ref.scales.shape, what
    bad_s = np.argwhere(gs != ref.scales)
    assert bad_s.shape[0] == 0, f"{what}: {bad_s.shape[0]} scales differ, first {bad_s[:5].tolist()}"
    bad_c = np.argwhere(gc != ref.codes)
    assert bad_c.shape[0] == 0, f"{what}: {bad_c.shape[0]} code bytes differ, first {bad_c[:5].tolist()}"


def _check_quant(fw, bits, transpose=False, what=""):
    g = fw.mx_quantize(bits_to_torch(bits), transpose=transpose)
    _assert_equal(g, _oxt(bits) if transpose else _ox(bits), what)
    return g


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 64), (33, 288), (300, 1024), (65, 4128), (3, 16384)])
def test_quantize_rows_and_transposed(fw, rows, cols):
    bits = synth.activations_bf16((rows, cols), 95, rows * 1009 + cols)
    _check_quant(fw, bits, what=f"rows {rows}x{cols}")
    # transposed: input [cols' x rows'] with rows' = cols, cols' = rows rounded to 32
    tb = synth.activations_bf16((((rows + 31) // 32) * 32, cols), 95, rows * 1009 + cols + 1)
    _check_quant(fw, tb, transpose=True, what=f"transposed {tb.shape}")


def test_quantize_strided_input(fw):
    bits = synth.activations_bf16((64, 512), 95, 77)
    x = bits_to_torch(bits)[:, 128:384]                     # row stride 512 elements
    g = fw.mx_quantize(x)
    _assert_equal(g, _ox(np.ascontiguousarray(bits[:, 128:384])), "strided rows")
    gt = fw.mx_quantize(bits_to_torch(bits)[:, :96], transpose=True)   # W^T of a column slice
    _assert_equal(gt, _oxt(np.ascontiguousarray(bits[:, :96])), "strided transposed")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("input "):
            vals = [float(v) for v in line.split()[1:]]
            rows.append(vals + [0.0] * (32 - len(vals)))
    return np.array(rows, dtype=np.float64)


def test_golden_and_edge_values(fw):
    """Hand-worked vectors (those exactly representable in BF16) plus all-zero,
    signed-zero, subnormal-range, near-BF16-max and midpoint blocks."""
    g = _golden_rows()
    keep = np.array([np.array_equal(bf16_values(synth.bf16_bits(r.astype(np.float32))), r.astype(np.float32))
                     and np.array_equal(r.astype(np.float32).astype(np.float64), r) for r in g])
    assert keep.sum() >= 4, "most hand-worked vectors are BF16 values"
    rng = np.random.default_rng(96)
    edge = [np.zeros(32), -np.zeros(32),
            rng.uniform(-1, 1, 32) * 2.0 ** -125, rng.uniform(-1, 1, 32) * 2.0 ** -131,
            rng.uniform(-1, 1, 32) * 3.0e38,
            rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0], 32) * rng.choice([-1, 1], 32) * 2.0 ** 9,
            np.concatenate([[6.0 * 2.0 ** 100], rng.standard_normal(31)])]
    rows = np.concatenate([g[keep], np.array(edge)])
    bits = synth.bf16_bits(rows.astype(np.float32))
    bits = np.tile(bits, (1, 3))                             # 96 columns: three blocks per row
    _check_quant(fw, bits, what="golden+edge rows")
    _check_quant(fw, np.ascontiguousarray(bits[:, :64].T), transpose=True, what="golden+edge transposed")


def test_weight_layouts(fw):
    w = synth.normal_bf16((320, 256), 0.02, 95, 5)
    wf, wb = fw.mx_weight_layouts(bits_to_torch(w))
    of, ob = omx.weight_layouts(bf16_values(w).astype(np.float64))
    _assert_equal(wf, of, "W_fwd")
    _assert_equal(wb, ob, "W_bwd")


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def _gemm_check(fw, M, N, K, seed, what):
    a = synth.activations_bf16((M, K), 95, seed)
    b = synth.normal_bf16((N, K), 0.02, 95, seed + 1)
    aq, bq = _ox(a), _ox(b)
    y = fw.mx_gemm(_to_gpu(aq), _to_gpu(bq))
    yref, yabs = omx.gemm_nt(aq, bq)
    assert_within(torch_bf16_to_f64(y), yref, tol.gemm_bound(yref, yabs), what)


@pytest.mark.parametrize("K", [128, 256, 384, 512, 640, 1280])
def test_gemm_pipeline_depths(fw, K):
    _gemm_check(fw, 96, 160, K, K, f"96x160x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (7, 33, 256), (130, 257, 384), (300, 200, 512),
                                   (2, 300, 768), (1000, 130, 1280), (513, 640, 4096)])
def test_gemm_ragged_shapes(fw, M, N, K):
    _gemm_check(fw, M, N, K, M + 3 * N + 7 * K, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (300, 200, 512), (256, 512, 256)])
def test_gemm_exact_special_case_bit_identical(fw, M, N, K):
    """Scales within 2^-3 .. 2^3 for A and 1 for B keep every partial sum exact
    in FP32, so the BF16 output must equal RNE of the exact product bit for bit."""
    rng = np.random.default_rng(M * 11 + N)
    ca, cb = rng.integers(0, 16, size=(M, K)), rng.integers(0, 16, size=(N, K))
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    a = omx.MXFP4(pack(ca), rng.integers(124, 131, size=(M, K // 32)).astype(np.uint8))
    b = omx.MXFP4(pack(cb), np.full((N, K // 32), 127, np.uint8))
    y = fw.mx_gemm(_to_gpu(a), _to_gpu(b))
    yref, _ = omx.gemm_nt(a, b)
    got, want = torch_bf16_to_f64(y), tol.bf16_rne(yref)
    assert np.array_equal(got, want), f"{np.sum(got != want)} outputs differ"


def test_gemm_accumulate_and_empty(fw):
    M, N, K = 200, 300, 512
    a = _ox(synth.activations_bf16((M, K), 95, 901))
    b = _ox(synth.normal_bf16((N, K), 0.02, 95, 902))
    prev = synth.normal_bf16((M, N), 0.05, 95, 903)
    out = bits_to_torch(prev).clone()
    fw.mx_gemm(_to_gpu(a), _to_gpu(b), out=out, accumulate=True)
    yref, yabs = omx.gemm_nt(a, b)
    want = bf16_values(prev).astype(np.float64) + yref
    assert_within(torch_bf16_to_f64(out), want, tol.gemm_bound(want, yabs), "accumulate")
    # padded output (ldc > N, unaligned rows take the scalar store path)
    big = torch.zeros((M, N + 5), dtype=torch.bfloat16, device=dev())
    fw.mx_gemm(_to_gpu(a), _to_gpu(b), out=big[:, :N])
    assert_within(torch_bf16_to_f64(big[:, :N]), yref, tol.gemm_bound(yref, yabs), "ldc = N + 5")
    assert torch.count_nonzero(big[:, N:]).item() == 0, "columns beyond N written"
    # M = 0: nothing to do
    e = fw.mx_gemm(_to_gpu(omx.MXFP4(np.zeros((0, K // 2), np.uint8), np.zeros((0, K // 32), np.uint8))),
                   _to_gpu(b))
    assert e.shape == (0, N)


LLAMA3B = [("q/o", 3072, 3072), ("k/v", 3072, 1024), ("gate/up", 3072, 8192), ("down", 8192, 3072)]


@pytest.mark.parametrize("name,d_in,d_out", LLAMA3B)
def test_llama3b_full_size_sampled(fw, name, d_in, d_out):
    """Llama-3B projections at M = 4096 (every tile shape of the kernel): the GPU
    quantizes X, dY, W and W^T and runs the forward and input-gradient GEMMs at
    full size; 48 sampled rows x 384 sampled columns are checked.  Quantization
    is per row of each operand, so the oracle needs only the sampled rows: an
    exact sub-problem of the full product."""
    M, seed = 4096, 910 + d_in // 1024 + d_out
    wl = synth.WORKLOADS[2]
    x = synth.workload_activation(wl, M, d_in, seed)
    w = synth.normal_bf16((d_out, d_in), 0.02, wl.wid, seed + 1)
    dy = synth.normal_bf16((M, d_out), 0.01, wl.wid, seed + 2)
    gx, gdy = fw.mx_quantize(bits_to_torch(x)), fw.mx_quantize(bits_to_torch(dy))
    gwf, gwb = fw.mx_weight_layouts(bits_to_torch(w))
    y, dx = fw.mx_gemm(gx, gwf), fw.mx_gemm(gdy, gwb)
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=48, replace=False))
    rows[-1] = M - 1
    ncols = np.sort(rng.choice(d_out, size=384, replace=False))
    kcols = np.sort(rng.choice(d_in, size=384, replace=False))
    wv = bf16_values(w).astype(np.float64)
    oxq, odyq = _ox(x[rows]), _ox(dy[rows])
    owf = omx.quantize(wv[ncols])
    owb = omx.quantize(np.ascontiguousarray(wv[:, kcols].T))
    _assert_equal(gx, oxq, name + " x_q", rows=rows)
    _assert_equal(gdy, odyq, name + " dy_q", rows=rows)
    _assert_equal(gwf, owf, name + " W_fwd", rows=ncols)
    _assert_equal(gwb, owb, name + " W_bwd", rows=kcols)
    yref, yabs = omx.gemm_nt(oxq, owf)
    assert_within(torch_bf16_to_f64(y)[np.ix_(rows, ncols)], yref, tol.gemm_bound(yref, yabs), name + " fwd")
    dref, dabs = omx.gemm_nt(odyq, owb)
    assert_within(torch_bf16_to_f64(dx)[np.ix_(rows, kcols)], dref, tol.gemm_bound(dref, dabs), name + " dgrad")


# ---------------------------------------------------------------- fused forward operators, MXFP4 outputs
@pytest.mark.parametrize("M,H", [(64, 256), (33, 3072), (9, 8192), (17, 16384), (5, 96), (8192, 3072), (3, 12288)])
def test_mx_rmsnorm_quant(fw, M, H):
    """RMSNorm -> MXFP4: rstd, codes and E8M0 scales bit-exact (every row layout:
    one, two and four waves per row, ragged blocks per lane); the MLP-block
    shape [8192 x 3072] checked on sampled rows."""
    x = synth.activations_bf16((M, H), 3, 760 + H)
    g = synth.uniform_bf16((H,), 0.9, 1.1, 3, 761 + H)
    yq, rstd = fw.mx_rmsnorm_quant(bits_to_torch(x), bits_to_torch(g), 1e-5)
    rows = np.arange(M) if M <= 64 else np.sort(np.random.default_rng(M).choice(M, size=128, replace=False))
    ref_q, ref_rstd, _ = omx.rmsnorm_quant(bf16_values(x[rows]), bf16_values(g), 1e-5)
    got = rstd.cpu().numpy()[rows]
    assert np.array_equal(got.view(np.uint32), ref_rstd.view(np.uint32)), "rstd"
    _assert_equal(yq, ref_q, f"mx rmsnorm {M}x{H}", rows=rows)


@pytest.mark.parametrize("M,I", [(64, 256), (19, 8192), (7, 14336), (3, 96), (4096, 8192)])
def test_mx_silu_mul_quant(fw, M, I):
    """SiLU-multiply -> MXFP4 h, gate and up copies bit-exact, including
    sigmoid edge values (0, -0, saturating and overflowing exponent inputs)."""
    a = synth.normal_bf16((M, I), 2.0, 98, I + 1)
    b = synth.normal_bf16((M, I), 1.0, 98, I + 2)
    av = bf16_values(a).copy()
    av[0, :16] = [0, -0.0, 100, -100, 88, -88, 89.5, -89.5, 80.25, -80.25, 1e-30, -1e-30, 3, -3, 1e-3, -1e-3]
    av[-1, :32] = 0.0                                       # a zero block of h and of the gate copy
    a = synth.bf16_bits(av)
    hq, gq, uq = fw.mx_silu_mul_quant(bits_to_torch(a), bits_to_torch(b))
    rows = np.arange(M) if M <= 64 else np.sort(np.append(
        np.random.default_rng(I).choice(M - 1, size=127, replace=False), M - 1))
    rows[0] = 0
    rows = np.unique(rows)
    rh, ra, rb, _ = omx.silu_mul_quant(bf16_values(a[rows]), bf16_values(b[rows]))
    _assert_equal(gq, ra, "gate copy", rows=rows)
    _assert_equal(uq, rb, "up copy", rows=rows)
    _assert_equal(hq, rh, "h", rows=rows)


def test_mx_fused_strided_and_validation(fw):
    """Gate and up as column halves of one [M x 2I] buffer (the stacked
    gate/up GEMM output), and host-side rejection of widths not a multiple of 32."""
    M, I = 16, 512
    y = synth.normal_bf16((M, 2 * I), 1.5, 98, 901)
    t = bits_to_torch(y)
    hq, gq, uq = fw.mx_silu_mul_quant(t[:, :I], t[:, I:])
    rh, ra, rb, _ = omx.silu_mul_quant(bf16_values(y[:, :I]), bf16_values(y[:, I:]))
    _assert_equal(hq, rh, "h (strided)")
    _assert_equal(gq, ra, "gate (strided)")
    _assert_equal(uq, rb, "up (strided)")
    lib = fw._lib.load()
    p = t.data_ptr()
    assert lib.mxfp4_silu_mul_quant(p, p, 4, 48, 48, p, p, p, p, p, p, None) == -2
    assert lib.mxfp4_rmsnorm_quant(p, p, 1e-5, 4, 48, 48, p, p, p, None) == -2


# ---------------------------------------------------------------- backward from an MXFP4 state
def _as_values_f32(bits):
    return bf16_values(bits).astype(np.float32)


@pytest.mark.parametrize("M,I", [(64, 256), (33, 8192), (5, 14336), (2, 96), (2048, 8192)])
def test_mx_silu_mul_bwd_quant(fw, M, I):
    """BF16 gradients and their MXFP4 copies bit-exact against the oracle's
    pinned sequence on the dequantized MXFP4 gate/up state (sampled rows at
    the MLP-block width)."""
    a = synth.normal_bf16((M, I), 2.0, 99, I + 11)
    b = synth.normal_bf16((M, I), 1.0, 99, I + 12)
    dh = synth.normal_bf16((M, I), 0.01, 99, I + 13)
    aq, bq = _ox(a), _ox(b)
    dg, du, dgq, duq = fw.mx_silu_mul_bwd_quant(_to_gpu(aq), _to_gpu(bq), bits_to_torch(dh))
    rows = np.arange(M) if M <= 64 else np.sort(np.random.default_rng(I).choice(M, size=64, replace=False))
    sel = lambda q: omx.MXFP4(q.codes[rows], q.scales[rows])
    da, db, daq, dbq = omx.silu_mul_bwd_quant(sel(aq), sel(bq), _as_values_f32(dh[rows]))
    got_a = dg.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    got_b = du.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    assert np.array_equal(bf16_values(got_a).view(np.uint32), da.view(np.uint32)), "dgate"
    assert np.array_equal(bf16_values(got_b).view(np.uint32), db.view(np.uint32)), "dup"
    _assert_equal(dgq, daq, "dgate copy", rows=rows)
    _assert_equal(duq, dbq, "dup copy", rows=rows)


@pytest.mark.parametrize("M,H,resid,copy", [(64, 256, True, True), (33, 3072, True, True), (9, 8192, False, True),
                                             (17, 16384, True, False), (3, 96, True, True), (4096, 3072, True, True)])
def test_mx_rmsnorm_bwd_residual(fw, M, H, resid, copy):
    x = synth.activations_bf16((M, H), 99, 900 + H)
    g = synth.uniform_bf16((H,), 0.9, 1.1, 99, 901 + H)
    yq, rstd = omx.rmsnorm_quant(bf16_values(x), bf16_values(g), 1e-5)[:2]
    dy = synth.normal_bf16((M, H), 0.01, 99, 902 + H)
    rs = synth.normal_bf16((M, H), 0.01, 99, 903 + H) if resid else None
    out, q = fw.mx_rmsnorm_bwd_residual(_to_gpu(yq), torch.from_numpy(rstd).to(dev()), bits_to_torch(g),
                                        bits_to_torch(dy), resid=bits_to_torch(rs) if resid else None,
                                        quantize_out=copy)
    rows = np.arange(M) if M <= 64 else np.sort(np.random.default_rng(H).choice(M, size=64, replace=False))
    ref, refq = omx.rmsnorm_bwd_residual(omx.MXFP4(yq.codes[rows], yq.scales[rows]), rstd[rows], bf16_values(g),
                                         _as_values_f32(dy[rows]), _as_values_f32(rs[rows]) if resid else None)
    got = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    assert np.array_equal(bf16_values(got).view(np.uint32), ref.view(np.uint32)), "out"
    if copy:
        _assert_equal(q, refq, "out copy", rows=rows)
    else:
        assert q is None
