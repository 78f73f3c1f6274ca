"""Seeded synthetic inputs for the NVFP4 frozen-projection path.

This module holds no arithmetic of the method: it only draws random numbers
and rounds them to BF16, the precision the LoRA linear layer receives its
activations, gradients and adapters in (PACT, Appendix Table 7).  Both the
CPU oracle's tests and the GPU path's tests and benchmark take their inputs
from here, so each side sees the same tensors.

Test tensors are drawn from ``numpy.random.default_rng([workload_id, tensor_id])``
in float32 and rounded to BF16 with round-to-nearest-even.  The benchmark's
large inputs come from the ``*_torch`` functions below: the same
distributions drawn on the device by torch's generator seeded with
``(workload_id << 40) + tensor_id``, so multi-GB workloads need no host
sampling.  ``N(0, s)`` means standard deviation ``s``.

The workloads are the synthetic Llama-shaped projection sets: the pages use
Llama-1B/3B models and quote Llama-3B projection dimensions in Table 1 (query
3072x3072, gate/up 3072x8192, down 8192x3072); the other dimensions are the
public Llama-3.2-1B/3B and Llama-3-8B shapes.
"""

from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "bf16_from_bits",
    "normal_bf16",
    "uniform_bf16",
    "student_t_bf16",
    "activations_bf16",
    "Projection",
    "Workload",
    "WORKLOADS",
]


# ---------------------------------------------------------------------------
# BF16 storage helpers (storage conversion of random samples, not method math)
# ---------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """float32 -> uint16 BF16 bit patterns, round-to-nearest-even (NaN not expected)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    """uint16 BF16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round float32 samples to the nearest BF16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


def _rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(tensor_id)])


def normal_bf16(shape, std: float, workload_id: int, tensor_id: int) -> np.ndarray:
    """BF16 bit patterns of N(0, std) samples."""
    g = _rng(workload_id, tensor_id)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x)


def uniform_bf16(shape, lo: float, hi: float, workload_id: int, tensor_id: int) -> np.ndarray:
    g = _rng(workload_id, tensor_id)
    x = g.uniform(lo, hi, size=shape).astype(np.float32)
    return bf16_bits(x)


def student_t_bf16(shape, nu: float, workload_id: int, tensor_id: int) -> np.ndarray:
    """BF16 bit patterns of standard Student-t(nu) samples (heavy-tailed activations)."""
    g = _rng(workload_id, tensor_id)
    x = g.standard_t(nu, size=shape).astype(np.float32)
    return bf16_bits(x)


def activations_bf16(shape, workload_id: int, tensor_id: int, outlier_frac: float = 0.01,
                     outlier_gain: float = 20.0) -> np.ndarray:
    """N(0,1) activations [tokens x channels] with ceil(frac*channels) channels scaled by gain.

    The outlier channels are columns (the contraction axis of the forward GEMM),
    chosen without replacement from the same generator.
    """
    g = _rng(workload_id, tensor_id)
    x = g.standard_normal(size=shape, dtype=np.float32)
    ch = shape[-1]
    n_out = int(np.ceil(outlier_frac * ch))
    if n_out > 0 and outlier_gain != 1.0:
        idx = g.choice(ch, size=n_out, replace=False)
        x[..., idx] *= np.float32(outlier_gain)
    return bf16_bits(x)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Projection:
    """One frozen projection W [d_out x d_in]; forward Y = X W^T, dgrad dX = dY W."""
    name: str
    d_in: int
    d_out: int


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    tokens: int
    projections: tuple
    lora_rank: int
    act: str           # "normal", "normal_outliers", "student_t3"
    w_std: float = 0.02
    dy_std: float = 0.01
    a_std: float = 0.01

    def flops_fwd_dgrad(self) -> int:
        return sum(4 * self.tokens * p.d_in * p.d_out for p in self.projections)


def _llama(h, kv, inter):
    return (
        Projection("q", h, h),
        Projection("k", h, kv),
        Projection("v", h, kv),
        Projection("o", h, h),
        Projection("gate", h, inter),
        Projection("up", h, inter),
        Projection("down", inter, h),
    )


WORKLOADS = {
    0: Workload(0, "tiny-lora-linear-64x256x256-r8", 64, (Projection("w", 256, 256),), 8, "normal"),
    1: Workload(1, "llama1b-proj-M4096", 4096, _llama(2048, 512, 8192), 16, "normal_outliers"),
    2: Workload(2, "llama3b-proj-M4096", 4096, _llama(3072, 1024, 8192), 16, "normal_outliers"),
    3: Workload(3, "llama3b-mlp-block-M8192", 8192,
                (Projection("gate", 3072, 8192), Projection("up", 3072, 8192),
                 Projection("down", 8192, 3072)), 16, "normal_outliers"),
    4: Workload(4, "llama8b-proj-M16384", 16384, _llama(4096, 1024, 14336), 64, "student_t3"),
}


def workload_activation(wl: Workload, rows: int, cols: int, tensor_id: int) -> np.ndarray:
    """BF16 activation bits [rows x cols] with the workload's distribution."""
    if wl.act == "normal":
        return normal_bf16((rows, cols), 1.0, wl.wid, tensor_id)
    if wl.act == "normal_outliers":
        return activations_bf16((rows, cols), wl.wid, tensor_id)
    if wl.act == "student_t3":
        return student_t_bf16((rows, cols), 3.0, wl.wid, tensor_id)
    raise ValueError(wl.act)


# ---------------------------------------------------------------------------
# Device-side draws (benchmark inputs): the same distributions drawn by torch's
# seeded generator on the GPU, so multi-GB workloads need no host sampling.
# Parity checks of benchmark outputs read these tensors back from the device.
# ---------------------------------------------------------------------------

def torch_generator(workload_id: int, tensor_id: int, device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((int(workload_id) << 40) + int(tensor_id))
    return g


def normal_torch(shape, std: float, workload_id: int, tensor_id: int, device="cuda"):
    """bfloat16 device tensor of N(0, std) samples (float32 draws, RNE to BF16)."""
    import torch
    g = torch_generator(workload_id, tensor_id, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def uniform_torch(shape, lo: float, hi: float, workload_id: int, tensor_id: int, device="cuda"):
    import torch
    g = torch_generator(workload_id, tensor_id, device)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return (x * (hi - lo) + lo).to(torch.bfloat16)


def activation_torch(wl: Workload, rows: int, cols: int, tensor_id: int, device="cuda"):
    """bfloat16 device activations [rows x cols] with the workload's distribution:
    N(0,1); N(0,1) with ceil(1%) of the columns x20; or standard Student-t(3),
    drawn as Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from independent normals."""
    import torch
    g = torch_generator(wl.wid, tensor_id, device)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    if wl.act == "normal_outliers":
        n_out = int(np.ceil(0.01 * cols))
        idx = torch.randperm(cols, generator=g, device=device)[:n_out]
        x[:, idx] *= 20.0
    elif wl.act == "student_t3":
        chi = torch.zeros_like(x)
        for _ in range(3):
            z = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
            chi.addcmul_(z, z)
        x.div_(torch.sqrt(chi / 3.0))
    elif wl.act != "normal":
        raise ValueError(wl.act)
    return x.to(torch.bfloat16)
