"""Helpers shared by the GPU parity tests: tensor transfer and comparisons.

Inputs come from ``synth`` (seeded BF16 bit patterns); expected values come
from ``oracle`` only.  The GPU path is called through the C ABI via the
package's thin wrappers.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import nvfp4 as onv
from oracle import tolerance as tol


def dev():
    return torch.device("cuda:0")


def bits_to_torch(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns -> bfloat16 device tensor (bit-identical)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def torch_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """BF16 bits -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def torch_bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return bf16_values(torch_to_bits(t)).astype(np.float64)


def to_oracle(q) -> onv.NVFP4:
    """Copy a GPU NVFP4Tensor to the oracle's representation (for comparisons only)."""
    return onv.NVFP4(q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.rscale.cpu().numpy())


def nvfp4_to_gpu(q: onv.NVFP4):
    from frozen_weight_gemms_amd import NVFP4Tensor
    return NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(q.codes)).to(dev()),
                       torch.from_numpy(np.ascontiguousarray(q.scales)).to(dev()),
                       torch.from_numpy(np.ascontiguousarray(q.rscale)).to(dev()))


def assert_nvfp4_equal(gpu_q, ref: onv.NVFP4, what: str = "", rows=None):
    g = to_oracle(gpu_q)
    gc, gs, gr = g.codes, g.scales, g.rscale
    if rows is not None:
        gc, gs, gr = gc[rows], gs[rows], gr[rows]
    assert gc.shape == ref.codes.shape, what
    bad_r = np.flatnonzero(gr.view(np.uint32) != np.asarray(ref.rscale, np.float32).view(np.uint32))
    assert bad_r.size == 0, f"{what}: {bad_r.size} row scales differ, first row {bad_r[:5]}"
    bad_s = np.argwhere(gs != ref.scales)
    assert bad_s.shape[0] == 0, f"{what}: {bad_s.shape[0]} block scales differ, first {bad_s[:5].tolist()}"
    bad_c = np.argwhere(gc != ref.codes)
    assert bad_c.shape[0] == 0, f"{what}: {bad_c.shape[0]} code bytes differ, first {bad_c[:5].tolist()}"


def assert_within(got, ref, bound, what: str = ""):
    n, worst = tol.violations(got, ref, bound)
    assert n == 0, f"{what}: {n} of {np.size(ref)} elements outside the bound (worst err/bound {worst:.3g})"
    return worst
