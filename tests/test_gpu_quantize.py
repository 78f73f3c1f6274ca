"""GPU parity: nvfp4_quantize (row-wise and transposed) against the oracle.

NVFP4 format per PACT Appendix Table 6; codes, block scales and row scales
must be bit-exact (integer/byte results).
"""

import os

import numpy as np
import pytest

import synth
from oracle import nvfp4 as onv

from gpu_util import assert_nvfp4_equal, bf16_values, bits_to_torch

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_vectors.txt")


@pytest.fixture(scope="module")
def fw():
    import frozen_weight_gemms_amd as fw
    return fw


def _check(fw, bits, transpose=False, what=""):
    x = bits_to_torch(bits)
    q = fw.quantize(x, transpose=transpose)
    ref = onv.quantize(bf16_values(bits).astype(np.float64), transpose=transpose)
    assert_nvfp4_equal(q, ref, what)
    return q, ref


def test_tiny_workload_tensors(fw):
    wl = synth.WORKLOADS[0]
    x = synth.workload_activation(wl, 64, 256, 1)
    w = synth.normal_bf16((256, 256), 0.02, 0, 2)
    dy = synth.normal_bf16((64, 256), 0.01, 0, 3)
    _check(fw, x, what="X")
    _check(fw, w, what="W_fwd")
    _check(fw, w, transpose=True, what="W_bwd")
    _check(fw, dy, what="dY")


def test_golden_vectors_on_gpu(fw):
    rows = []
    for line in open(GOLDEN):
        if line.startswith("input "):
            rows.append([float(v) for v in line.split()[1:]])
    x = synth.bf16_bits(np.array(rows, dtype=np.float32))
    assert np.array_equal(bf16_values(x), np.array(rows, dtype=np.float32))
    _check(fw, x, what="golden")


@pytest.mark.parametrize("rows,cols", [(1, 16), (7, 48), (33, 272), (5, 2048), (3, 4096 + 16), (2, 16384),
                                       (3, 20480), (300, 1024),
                                       # 513..768 blocks per row: four waves per row, three blocks per lane
                                       (3, 8208), (5, 10240), (4, 12288), (2, 12304)])
def test_ragged_and_long_shapes(fw, rows, cols):
    bits = synth.activations_bf16((rows, cols), 90, rows * 100003 + cols)
    _check(fw, bits, what=f"{rows}x{cols}")
    tcols = min(cols, 4096)
    tbits = synth.normal_bf16((tcols, rows), 0.02, 90, rows * 100003 + cols + 1)   # W [N x K] with N % 16 == 0
    _check(fw, tbits, transpose=True, what=f"T {rows}x{tcols}")


def test_edge_values(fw):
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.zeros(64, np.float32))                           # all-zero row
    r = np.zeros(64, np.float32); r[:] = -0.0; rows.append(r)       # all -0
    r = rng.standard_normal(64).astype(np.float32); r[:16] = 0; r[16:20] = -0.0; rows.append(r)
    rows.append(np.full(64, 3.3895314e38, np.float32))              # BF16 max
    rows.append((rng.standard_normal(64) * 1e-38).astype(np.float32))   # subnormal range
    r = (rng.standard_normal(64) * 1e-3).astype(np.float32); r[3] = 3e4; rows.append(r)  # zero-scale blocks
    rows.append(np.full(64, 1.0, np.float32))
    rows.append(np.tile(np.float32([6, -6, 5, 3.5, 2.5, 1.75, 1.25, 0.75]), 8))
    # exact E2M1 and E4M3 midpoints at many scales
    for k in range(-12, 4):
        s = onv.E4M3_POS[rng.integers(1, 127, size=4)]
        blk = np.concatenate([onv.E2M1_MID, onv.E2M1_MAG, [0.0]])[:16]
        rows.append(np.concatenate([blk * si for si in s]).astype(np.float32) * np.float32(2.0 ** k))
    while len(rows) % 16:
        rows.append(rng.standard_normal(64).astype(np.float32))
    bits = synth.bf16_bits(np.array(rows, dtype=np.float32))
    _check(fw, bits, what="edges")
    _check(fw, bits, transpose=True, what="edges T")


def test_row_exponents_across_the_range(fw):
    """Rows whose power-of-two scales 2^e span -75 .. 110, each with exact
    E2M1 midpoints times E4M3 scales, random values, values far below the
    block scale, and -0: codes, scales and row scales are bit-exact against
    the oracle at every exponent."""
    rng = np.random.default_rng(78)
    rows = []
    for e in (-75, -61, -60, -59, -33, -1, 0, 1, 64, 99, 100, 101, 110):
        p2 = np.float32(2.0 ** e)
        s = onv.E4M3_POS[rng.integers(1, 127, size=2)]
        mids = np.concatenate([onv.E2M1_MID, onv.E2M1_MAG, [0.0]])[:16]
        r = np.concatenate([
            np.concatenate([[2688.0], rng.standard_normal(15) * 300]),        # row maximum: scale exponent e
            mids * s[0], mids * s[1],
            np.concatenate([rng.standard_normal(8) * 2.0 ** -30, [-0.0, 0.0], rng.standard_normal(6)]),
        ]).astype(np.float32) * p2
        rows.append(r)
    while len(rows) % 16:
        rows.append(rng.standard_normal(64).astype(np.float32))
    x = np.array(rows, dtype=np.float32)
    bits = synth.bf16_bits(x)
    q, ref = _check(fw, bits, what="row exponents")
    got_e = np.log2(np.asarray(ref.rscale[:13], dtype=np.float64))
    assert np.array_equal(got_e, [-75, -61, -60, -59, -33, -1, 0, 1, 64, 99, 100, 101, 110])
    _check(fw, bits, transpose=True, what="row exponents T")


def test_strided_input(fw):
    bits = synth.activations_bf16((40, 512), 91, 1)
    x = bits_to_torch(bits)[:, 128:384]
    q = fw.quantize(x)
    ref = onv.quantize(bf16_values(bits[:, 128:384]).astype(np.float64))
    assert_nvfp4_equal(q, ref, "strided")


def test_empty(fw):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q = fw.quantize(x)
    assert q.codes.shape == (0, 32)


@pytest.mark.parametrize("name,rows,cols,kind", [
    ("llama3b dY gate/up [4096x8192]", 4096, 8192, "dy"),
    ("llama3b X [4096x3072]", 4096, 3072, "act"),
    ("llama3b W_fwd down [3072x8192]", 3072, 8192, "w"),
    ("8b-scale X student-t [2048x4096]", 2048, 4096, "t3"),
])
def test_full_size(fw, name, rows, cols, kind):
    if kind == "dy":
        bits = synth.normal_bf16((rows, cols), 0.01, 2, 501)
    elif kind == "act":
        bits = synth.activations_bf16((rows, cols), 2, 502)
    elif kind == "w":
        bits = synth.normal_bf16((rows, cols), 0.02, 2, 503)
    else:
        bits = synth.student_t_bf16((rows, cols), 3.0, 4, 504)
    _check(fw, bits, what=name)


def test_full_size_transposed_weight(fw):
    bits = synth.normal_bf16((3072, 8192), 0.02, 2, 505)    # W_down [N=3072 x K=8192]
    _check(fw, bits, transpose=True, what="W_bwd down [8192 x 3072]")


def _bits_equal(a, b):
    import torch
    return (torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
            and torch.equal(a.rscale.view(torch.int32), b.rscale.view(torch.int32)))


def test_quantize_batch_equals_single_calls(fw):
    """nvfp4_quantize_batch: every problem bit-identical to its own nvfp4_quantize
    call: the attention-gradient shapes of the Llama-3B step (one launch),
    ragged rows, one 16-column row, a padded leading dimension, an empty
    problem, and problems wider than 3072 columns (launches of their own)."""
    import torch
    wl = synth.WORKLOADS[2]
    cases = [
        [(4096, 3072), (4096, 1024), (4096, 1024)],
        [(333, 3072), (1, 16), (77, 1024), (0, 512), (129, 2048)],
        [(64, 4096), (40, 3072), (96, 8192), (33, 16384), (8, 20480)],
    ]
    for k, shapes in enumerate(cases):
        xs = []
        for i, (rows, cols) in enumerate(shapes):
            if rows and cols:
                x = synth.activation_torch(wl, rows, cols, 300 + 10 * k + i) * (2.0 ** (3 * i - 4))
            else:
                x = torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda")
            xs.append(x)
        if k == 1:                          # one padded leading dimension
            big = synth.activation_torch(wl, 129, 2048 + 64, 399)
            xs[4] = big[:, :2048]
        got = fw.quantize_batch(xs)
        torch.cuda.synchronize()
        for i, (x, q) in enumerate(zip(xs, got)):
            want = fw.quantize(x)
            assert _bits_equal(q, want), f"case {k} problem {i} {tuple(x.shape)}"


def test_quantize_batch_plan_reruns(fw):
    """A QuantizeBatch plan run twice reads its inputs' current contents."""
    import torch
    xs = [synth.normal_torch((256, 3072), 0.02, 2, 410), synth.normal_torch((256, 1024), 0.02, 2, 411)]
    plan = fw.QuantizeBatch(xs)
    plan.run()
    first = [fw.quantize(x) for x in xs]
    assert all(_bits_equal(a, b) for a, b in zip(plan.outputs, first))
    for x in xs:
        x.mul_(-3.0)
    plan.run()
    torch.cuda.synchronize()
    second = [fw.quantize(x) for x in xs]
    assert all(_bits_equal(a, b) for a, b in zip(plan.outputs, second))
