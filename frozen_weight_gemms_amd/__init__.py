"""NVFP4 frozen-projection path of PACT's LoRA fine-tuning, native on MI355X.

Thin torch-facing wrappers over the C ABI in include/pact_nvfp4.h.  torch
provides device memory and the current HIP stream; every operation runs in
the hand-written gfx950 kernels of libpact_nvfp4.so.  The wrappers allocate
outputs with torch and pass raw pointers; they compute nothing themselves.
"""

from __future__ import annotations

import dataclasses

import torch

from . import _lib
from ._lib import PactError, load  # noqa: F401

__all__ = [
    "NVFP4Tensor", "empty_nvfp4", "quantize", "rmsnorm_quant", "silu_mul_quant", "gemm_fwd", "gemm_dgrad",
    "lora_down", "lora_bwd", "lora_bwd_workspace", "silu_mul_bwd", "rmsnorm_bwd", "weight_layouts", "PactError",
]


@dataclasses.dataclass
class NVFP4Tensor:
    """Canonical NVFP4 tensor [rows x cols]: codes u8 [rows, cols/2], scales u8 [rows, cols/16], rscale f32 [rows]."""
    codes: torch.Tensor
    scales: torch.Tensor
    rscale: torch.Tensor

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2

    def ptrs(self):
        return self.codes.data_ptr(), self.scales.data_ptr(), self.rscale.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    return t


def _dense(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense rows)")
    return t


def empty_nvfp4(rows: int, cols: int, device="cuda") -> NVFP4Tensor:
    if cols % 16:
        raise ValueError("cols must be a multiple of 16")
    return NVFP4Tensor(
        torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
        torch.empty((rows, cols // 16), dtype=torch.uint8, device=device),
        torch.empty((rows,), dtype=torch.float32, device=device),
    )


def quantize(x: torch.Tensor, transpose: bool = False, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """nvfp4_quantize: Q(x) (blocks along the last axis) or, with transpose, Q(x^T)."""
    _bf16(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    if transpose:
        rows, cols = x.shape[1], x.shape[0]
    else:
        rows, cols = x.shape
    out = out or empty_nvfp4(rows, cols, x.device)
    _lib.call("nvfp4_quantize", x.data_ptr(), rows, cols, x.stride(0), int(transpose), *out.ptrs(), _stream())
    return out


class QuantizeBatch:
    """nvfp4_quantize_batch: Q(x_i) of several BF16 [rows_i x cols_i] tensors in
    one launch (each bit-identical to quantize(x_i)), with the call's argument
    arrays built once; every run() reads the inputs' current contents and
    writes ``outputs`` (allocated here unless given) on the current stream."""

    def __init__(self, xs, outs=None):
        import ctypes
        n = len(xs)
        if outs is None:
            outs = [empty_nvfp4(x.shape[0], x.shape[1], x.device) for x in xs]
        if len(outs) != n:
            raise ValueError("one output per input")
        for x, o in zip(xs, outs):
            _bf16(x, "x")
            if x.dim() != 2 or x.stride(1) != 1:
                raise ValueError("x must be a 2-D tensor with unit column stride")
            if (o.rows, o.cols) != tuple(x.shape):
                raise ValueError("output shape differs from its input's")
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        arr = lambda t, vals: (t * max(n, 1))(*vals) if n else None
        self.inputs, self.outputs = list(xs), list(outs)   # keeps the tensors alive while the plan exists
        self._args = (n, arr(vp, [x.data_ptr() for x in xs]), arr(i64, [x.shape[0] for x in xs]),
                      arr(i64, [x.shape[1] for x in xs]), arr(i64, [x.stride(0) for x in xs]),
                      arr(vp, [o.codes.data_ptr() for o in outs]), arr(vp, [o.scales.data_ptr() for o in outs]),
                      arr(vp, [o.rscale.data_ptr() for o in outs]))

    def run(self):
        _lib.call("nvfp4_quantize_batch", *self._args, _stream())
        return self.outputs


def quantize_batch(xs, outs=None):
    """One run of QuantizeBatch(xs, outs): the NVFP4 outputs, in input order."""
    return QuantizeBatch(xs, outs).run()


QUANT_ROUND_UP_SCALES = 1
QUANT_TENSOR_SCALE = 2
QUANT_COMPUTE_AMAX = 4
QUANT_TENSOR_SCALE_FP32 = 8


def quantize_ex(x: torch.Tensor, transpose: bool = False, round_up: bool = False, tensor_scale: bool = False,
                amax: torch.Tensor | None = None, compute_amax: bool = True, out: NVFP4Tensor | None = None,
                fp32_scale: bool = False):
    """NVFP4 of x (or x^T) with the recipe variants: round-up block scales and/or one
    scale for the whole tensor from amax (a float32 device scalar, computed here
    by a first pass when compute_amax, else supplied): a power of two, or with
    fp32_scale the conventional FP32 scale RN32(amax / 2688)."""
    if fp32_scale and not tensor_scale:
        raise ValueError("fp32_scale needs tensor_scale")
    _bf16(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    rows, cols = (x.shape[1], x.shape[0]) if transpose else (x.shape[0], x.shape[1])
    out = out if out is not None else empty_nvfp4(rows, cols, x.device)
    flags = (QUANT_ROUND_UP_SCALES if round_up else 0)
    if tensor_scale:
        flags |= QUANT_TENSOR_SCALE | (QUANT_COMPUTE_AMAX if compute_amax else 0)
        flags |= QUANT_TENSOR_SCALE_FP32 if fp32_scale else 0
        if amax is None:
            if not compute_amax:
                raise ValueError("a supplied amax is needed when compute_amax is False")
            amax = torch.empty((), dtype=torch.float32, device=x.device)
        if amax.dtype != torch.float32 or amax.numel() != 1:
            raise TypeError("amax must be a float32 device scalar")
    _lib.call("nvfp4_quantize_ex", x.data_ptr(), rows, cols, x.stride(0), int(transpose), flags,
              amax.data_ptr() if tensor_scale else 0, *out.ptrs(), _stream())
    return out


def selftest_arith(device="cuda") -> list:
    """Disagreement counts of the device's arithmetic shortcuts against IEEE
    operations over their whole input ranges (pact_selftest_arith); all 0 on a
    conforming device."""
    counts = torch.zeros((5,), dtype=torch.int64, device=device)
    _lib.call("pact_selftest_arith", counts.data_ptr(), _stream())
    return [int(v) for v in counts.cpu().tolist()]


def mfma_probe(kind: int, iters: int = 4000, device="cuda"):
    """Measured MFMA-loop peak (pact_mfma_probe): kind 0 FP16 32x32x16, kind 1
    scaled FP4 32x32x64.  Returns (TFLOP/s from events around one launch on the
    current stream, mean shader clock in GHz over the workgroups)."""
    groups = 512
    sink = torch.empty((groups * 256,), dtype=torch.float32, device=device)
    clocks = torch.zeros((2 * groups,), dtype=torch.int64, device=device)
    args = lambda: (kind, iters, sink.data_ptr(), sink.numel(), clocks.data_ptr(), clocks.numel(), _stream())
    _lib.call("pact_mfma_probe", *args())                  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    _lib.call("pact_mfma_probe", *args())
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = groups * 4 * iters * 16 * (32768 if kind == 0 else 131072)
    c = clocks.view(groups, 2).cpu().double()
    ghz = float((c[:, 0] / (c[:, 1] / 100e6)).mean() / 1e9)
    return flops / (ms * 1e-3) / 1e12, ghz


def weight_layouts(w: torch.Tensor):
    """The two cached NVFP4 layouts Q(W) (forward) and Q(W^T) (input gradient) of a frozen BF16 weight W [N x K]."""
    return quantize(w), quantize(w, transpose=True)


def rmsnorm_quant(x: torch.Tensor, gain: torch.Tensor, eps: float = 1e-5, out=None, exact_sum: bool = False):
    """(Q(y), rstd) with y = (x * rstd) * gain; ``out`` = (NVFP4Tensor, rstd) to reuse buffers.
    ``exact_sum``: every row's sum of squares on the double-double path (same results)."""
    _bf16(x, "x"); _bf16(gain, "gain")
    M, H = x.shape
    if out is not None:
        y, rstd = out
    else:
        y = empty_nvfp4(M, H, x.device)
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device)
    if exact_sum:
        _lib.call("rmsnorm_quant_ex", x.data_ptr(), gain.data_ptr(), float(eps), M, H, x.stride(0), 1, *y.ptrs(),
                  rstd.data_ptr(), _stream())
    else:
        _lib.call("rmsnorm_quant", x.data_ptr(), gain.data_ptr(), float(eps), M, H, x.stride(0), *y.ptrs(),
                  rstd.data_ptr(), _stream())
    return y, rstd


def silu_mul_quant(gate: torch.Tensor, up: torch.Tensor, out=None):
    """(Q(h), Q(gate), Q(up)) with h = silu(gate) * up; ``out`` = three NVFP4Tensors to reuse."""
    _bf16(gate, "gate"); _bf16(up, "up")
    if gate.shape != up.shape or gate.stride() != up.stride():
        raise ValueError("gate and up must have the same shape and strides")
    M, I = gate.shape
    h, gq, uq = out if out is not None else (empty_nvfp4(M, I, gate.device) for _ in range(3))
    _lib.call("silu_mul_quant", gate.data_ptr(), up.data_ptr(), M, I, gate.stride(0), *h.ptrs(), *gq.ptrs(),
              *uq.ptrs(), _stream())
    return h, gq, uq


GEMM_ANY_ROW_SCALES = 1


def gemm_fwd(xq: NVFP4Tensor, w_fwd: NVFP4Tensor, lora_t: torch.Tensor | None = None,
             lora_b: torch.Tensor | None = None, lora_scale: float = 1.0, out: torch.Tensor | None = None,
             any_row_scales: bool = False):
    """Y = bf16(deq(X_q) deq(W_fwd)^T [+ lora_scale * T B^T]).  ``any_row_scales``:
    operands may carry non-power-of-two row scales (FP32 tensor-scale recipe)."""
    M, K = xq.rows, xq.cols
    N = w_fwd.rows
    if w_fwd.cols != K:
        raise ValueError(f"K mismatch: {K} vs {w_fwd.cols}")
    out = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.codes.device)
    r = 0
    if lora_t is not None:
        r = lora_t.shape[1]
        if lora_b is None or lora_b.shape != (N, r) or lora_t.shape[0] != M:
            raise ValueError("LoRA shapes: T [M x r], B [N x r]")
    _lib.call("nvfp4_gemm_fwd_ex", *xq.ptrs(), M, K, *w_fwd.ptrs(), N, out.data_ptr(), out.stride(0),
              _ptr(lora_t), _ptr(lora_b), r, float(lora_scale), GEMM_ANY_ROW_SCALES if any_row_scales else 0,
              _stream())
    return out


def gemm_dgrad(dyq: NVFP4Tensor, w_bwd: NVFP4Tensor, out: torch.Tensor | None = None, accumulate: bool = False,
               lora_dt: torch.Tensor | None = None, lora_a: torch.Tensor | None = None,
               any_row_scales: bool = False):
    """dX = bf16([f32(dX) +] deq(dY_q) deq(W_bwd)^T [+ dT A]); ``any_row_scales`` as for gemm_fwd."""
    M, N = dyq.rows, dyq.cols
    K = w_bwd.rows
    if w_bwd.cols != N:
        raise ValueError(f"N mismatch: {N} vs {w_bwd.cols}")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing output")
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dyq.codes.device)
    r = 0
    if lora_dt is not None:
        r = lora_dt.shape[1]
        if lora_a is None or lora_a.shape != (r, K) or lora_dt.shape[0] != M:
            raise ValueError("LoRA shapes: dT [M x r], A [r x K]")
    _lib.call("nvfp4_gemm_dgrad_ex", *dyq.ptrs(), M, N, *w_bwd.ptrs(), K, out.data_ptr(), out.stride(0),
              int(accumulate), _ptr(lora_dt), _ptr(lora_a), r, GEMM_ANY_ROW_SCALES if any_row_scales else 0,
              _stream())
    return out


def gemm_dgrad_multi(segments, out: torch.Tensor | None = None, accumulate: bool = False, lora=None):
    """dX = bf16([f32(dX) +] sum_i (deq(dY_i) deq(W_bwd,i)^T [+ dT_i A_i])) in one launch.

    ``segments``: list of (dY_i NVFP4 [M x N_i], W_bwd,i NVFP4 [K x N_i]), 1..4 of them,
    N_i multiples of 256; ``lora``: None or a list of (dT_i, A_i) or None per segment."""
    import ctypes
    n = len(segments)
    M = segments[0][0].rows
    K = segments[0][1].rows
    for dyq, wb in segments:
        if dyq.rows != M or wb.rows != K or wb.cols != dyq.cols:
            raise ValueError("segments: dY_i [M x N_i] and W_bwd,i [K x N_i] with one M and one K")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing output")
        out = torch.empty((M, K), dtype=torch.bfloat16, device=segments[0][0].codes.device)
    P = ctypes.c_void_p * n
    arr = lambda vals: P(*[ctypes.c_void_p(v) for v in vals])
    i64 = ctypes.c_int64 * n
    dts = as_ = rs = None
    if lora is not None:
        if len(lora) != n:
            raise ValueError("one LoRA entry (or None) per segment")
        dtp, ap, rv = [], [], []
        for entry in lora:
            if entry is None:
                dtp.append(0); ap.append(0); rv.append(0)
                continue
            dT, A = entry
            r = dT.shape[1]
            if dT.shape[0] != M or A.shape != (r, K):
                raise ValueError("LoRA shapes: dT [M x r], A [r x K]")
            dtp.append(dT.data_ptr()); ap.append(A.data_ptr()); rv.append(r)
        dts, as_, rs = arr(dtp), arr(ap), i64(*rv)
    _lib.call("nvfp4_gemm_dgrad_multi", n, arr([d.codes.data_ptr() for d, _ in segments]),
              arr([d.scales.data_ptr() for d, _ in segments]), arr([d.rscale.data_ptr() for d, _ in segments]),
              i64(*[d.cols for d, _ in segments]), arr([w.codes.data_ptr() for _, w in segments]),
              arr([w.scales.data_ptr() for _, w in segments]), arr([w.rscale.data_ptr() for _, w in segments]),
              M, K, out.data_ptr(), out.stride(0), int(accumulate), dts, as_, rs, _stream())
    return out


class SingleLayoutWeight:
    """A frozen weight kept only as W_fwd = Q(W) [N x K], plus the largest and
    smallest row-scale exponents over its nonzero rows (device int32 [2]), for
    the single-layout dgrad.  Raises PactError (PACT_EUNSUPPORTED) for a weight
    whose nonzero rows span more than 2^14 in row scale (the dgrad would not
    be exact); the set-up synchronizes the current stream."""

    def __init__(self, w_fwd: NVFP4Tensor):
        self.w_fwd = w_fwd
        self.exp_range = torch.empty((2,), dtype=torch.int32, device=w_fwd.codes.device)
        self.exp_max = self.exp_range[:1]
        _lib.call("pact_nvfp4_row_exp_max", *w_fwd.ptrs(), w_fwd.rows, w_fwd.cols, self.exp_range.data_ptr(),
                  _stream())


def gemm_dgrad_fwd_layout(dyq: NVFP4Tensor, w: SingleLayoutWeight, out: torch.Tensor | None = None,
                          accumulate: bool = False, lora_dt: torch.Tensor | None = None,
                          lora_a: torch.Tensor | None = None):
    """dX = bf16([dX +] deq(dY_q) deq(W_fwd) [+ dT A]) over the forward layout only."""
    M, N = dyq.rows, dyq.cols
    K = w.w_fwd.cols
    if w.w_fwd.rows != N:
        raise ValueError(f"contraction mismatch: dY has {N} columns, W_fwd {w.w_fwd.rows} rows")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing output")
        out = torch.empty((M, K), dtype=torch.bfloat16, device=dyq.codes.device)
    r = 0
    if lora_dt is not None:
        r = lora_dt.shape[1]
        if lora_a is None or lora_a.shape != (r, K) or lora_dt.shape[0] != M:
            raise ValueError("LoRA shapes: dT [M x r], A [r x K]")
    _lib.call("nvfp4_gemm_dgrad_fwd_layout", *dyq.ptrs(), M, N, *w.w_fwd.ptrs(), w.exp_max.data_ptr(), K,
              out.data_ptr(), out.stride(0), int(accumulate), _ptr(lora_dt), _ptr(lora_a), r, _stream())
    return out


def lora_down(xq: NVFP4Tensor, A: torch.Tensor, out: torch.Tensor | None = None):
    _bf16(A, "A")
    r, K = A.shape
    if K != xq.cols:
        raise ValueError("A must be [r x K]")
    out = out if out is not None else torch.empty((xq.rows, r), dtype=torch.bfloat16, device=A.device)
    _lib.call("lora_down", *xq.ptrs(), xq.rows, K, A.data_ptr(), r, out.data_ptr(), _stream())
    return out


def lora_bwd_workspace(M: int, K: int, N: int, r: int, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size lora_bwd needs for these shapes (caller-owned, reusable)."""
    n = _lib.lora_bwd_workspace_size(M, K, N, r)
    return torch.empty((max(n, 1),), dtype=torch.uint8, device=device)


def lora_bwd(xq: NVFP4Tensor, A: torch.Tensor, B: torch.Tensor, dy: torch.Tensor, scale: float, out=None,
             workspace: torch.Tensor | None = None):
    """(dT, dA, dB); ``out`` = (dT, dA, dB) tensors to reuse; ``workspace`` from lora_bwd_workspace()."""
    _bf16(A, "A"); _bf16(B, "B"); _bf16(dy, "dy")
    r, K = A.shape
    N = B.shape[0]
    M = xq.rows
    if B.shape != (N, r) or dy.shape != (M, N) or K != xq.cols:
        raise ValueError("shapes: A [r x K], B [N x r], dy [M x N]")
    dev = A.device
    if out is not None:
        dT, dA, dB = out
    else:
        dT = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((r, K), dtype=torch.bfloat16, device=dev)
        dB = torch.empty((N, r), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = lora_bwd_workspace(M, K, N, r, dev)
    _lib.call("lora_bwd", *xq.ptrs(), M, K, A.data_ptr(), B.data_ptr(), r, float(scale), dy.data_ptr(), N,
              dT.data_ptr(), dA.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    return dT, dA, dB


def lora_bwd_dt(dy: torch.Tensor, B: torch.Tensor, scale: float, out: torch.Tensor | None = None):
    """dT = bf16(scale dY B) alone (lora_bwd's dT, bit for bit)."""
    _bf16(B, "B"); _dense(_bf16(dy, "dy"), "dy")
    M, N = dy.shape
    r = B.shape[1]
    if B.shape != (N, r):
        raise ValueError("shapes: dy [M x N], B [N x r]")
    dT = out if out is not None else torch.empty((M, r), dtype=torch.bfloat16, device=dy.device)
    _lib.call("lora_bwd_dt", dy.data_ptr(), M, N, B.data_ptr(), r, float(scale), dT.data_ptr(), _stream())
    return dT


def lora_bwd_ab(xq: NVFP4Tensor, A: torch.Tensor, dy: torch.Tensor, dT: torch.Tensor, scale: float, out=None,
                workspace: torch.Tensor | None = None):
    """(dA, dB) given lora_bwd_dt's dT (lora_bwd's dA and dB, bit for bit)."""
    _bf16(A, "A"); _bf16(dy, "dy"); _bf16(dT, "dT")
    r, K = A.shape
    M, N = dy.shape
    if K != xq.cols or xq.rows != M or dT.shape != (M, r):
        raise ValueError("shapes: xq [M x K], A [r x K], dy [M x N], dT [M x r]")
    dev = A.device
    dA, dB = out if out is not None else (torch.empty((r, K), dtype=torch.bfloat16, device=dev),
                                          torch.empty((N, r), dtype=torch.bfloat16, device=dev))
    if workspace is None:
        workspace = lora_bwd_workspace(M, K, N, r, dev)
    _lib.call("lora_bwd_ab", *xq.ptrs(), M, K, A.data_ptr(), r, float(scale), dy.data_ptr(), N, dT.data_ptr(),
              dA.data_ptr(), dB.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream())
    return dA, dB


class LoraAbBatch:
    """dA and dB of several projections in three launches, given T = X_q A^T
    (lora_down's output), with the call's argument arrays built once (every
    run() reads the tensors' current contents and launches on the current
    stream).
    ``problems``: list of (xq, T, dy, dT, (dA, dB), workspace) with one token
    count; T [M x r] is the projection's lora_down output (a column slice of a
    stacked lora_down output is accepted: rows may be strided, columns must be
    contiguous).  run() writes each problem's dA and dB in place (lora_bwd's
    values, bit for bit, when T = lora_down(xq, A))."""

    def __init__(self, problems, scale: float):
        import ctypes
        n = len(problems)
        if n == 0:                               # the library refuses it (PACT_EINVAL) when run
            self.problems, self.outputs = [], []
            self._args = (0,) + (None,) * 3 + (0, None, None, None, None, float(scale)) + (None,) * 7
            return
        M = problems[0][2].shape[0]
        for xq, T, dy, dT, (dA, dB), ws in problems:
            _bf16(T, "T"); _dense(_bf16(dy, "dy"), "dy"); _dense(_bf16(dT, "dT"), "dT")
            _dense(_bf16(dA, "dA"), "dA"); _dense(_bf16(dB, "dB"), "dB")
            if T.dim() != 2 or T.stride(1) != 1 or T.stride(0) < T.shape[1]:
                raise ValueError("T must be [M x r] with contiguous columns")
            r, K = T.shape[1], xq.cols
            if dy.shape[0] != M or xq.rows != M or T.shape[0] != M or dT.shape != (M, r) or dA.shape != (r, K) \
                    or dB.shape != (dy.shape[1], r):
                raise ValueError("shapes: xq [M x K], T [M x r], dy [M x N], dT [M x r], dA [r x K], dB [N x r]")
        arr = lambda t, f: (t * n)(*[f(p) for p in problems])
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        self.problems = list(problems)          # keeps the tensors alive while the plan exists
        self.outputs = [p[4] for p in problems]
        self._args = (n,
                      arr(vp, lambda p: p[0].codes.data_ptr()), arr(vp, lambda p: p[0].scales.data_ptr()),
                      arr(vp, lambda p: p[0].rscale.data_ptr()), M, arr(i64, lambda p: p[0].cols),
                      arr(vp, lambda p: p[1].data_ptr()), arr(i64, lambda p: p[1].stride(0)),
                      arr(i64, lambda p: p[1].shape[1]), float(scale),
                      arr(vp, lambda p: p[2].data_ptr()), arr(i64, lambda p: p[2].shape[1]),
                      arr(vp, lambda p: p[3].data_ptr()), arr(vp, lambda p: p[4][0].data_ptr()),
                      arr(vp, lambda p: p[4][1].data_ptr()), arr(vp, lambda p: p[5].data_ptr()),
                      arr(ctypes.c_size_t, lambda p: p[5].numel()))

    def run(self):
        _lib.call("lora_bwd_ab_batch", *self._args, _stream())
        return self.outputs


def lora_bwd_ab_batch(problems, scale: float):
    """One run of LoraAbBatch(problems, scale): dA and dB of every problem, in place."""
    return LoraAbBatch(problems, scale).run()


def lora_bwd_noalloc(xq: NVFP4Tensor, A: torch.Tensor, B: torch.Tensor, dy: torch.Tensor, scale: float, out):
    """lora_bwd into caller tensors ``out`` = (dT, dA, dB) with the library's fixed
    per-device scratch instead of a workspace (allocates nothing)."""
    _bf16(A, "A"); _bf16(B, "B"); _bf16(dy, "dy")
    r, K = A.shape
    N = B.shape[0]
    M = xq.rows
    if B.shape != (N, r) or dy.shape != (M, N) or K != xq.cols:
        raise ValueError("shapes: A [r x K], B [N x r], dy [M x N]")
    dT, dA, dB = out
    _lib.call("lora_bwd_noalloc", *xq.ptrs(), M, K, A.data_ptr(), B.data_ptr(), r, float(scale), dy.data_ptr(), N,
              dT.data_ptr(), dA.data_ptr(), dB.data_ptr(), _stream())
    return dT, dA, dB


def silu_mul_bwd(gq: NVFP4Tensor, uq: NVFP4Tensor, dh: torch.Tensor, out=None):
    _dense(_bf16(dh, "dh"), "dh")
    M, I = dh.shape
    dg, du = out if out is not None else (torch.empty_like(dh), torch.empty_like(dh))
    _lib.call("silu_mul_bwd", *gq.ptrs(), *uq.ptrs(), dh.data_ptr(), M, I, dg.data_ptr(), du.data_ptr(), _stream())
    return dg, du


def rmsnorm_bwd(yq: NVFP4Tensor, rstd: torch.Tensor, gain: torch.Tensor, dy: torch.Tensor, out=None):
    _bf16(gain, "gain"); _dense(_bf16(dy, "dy"), "dy")
    M, H = dy.shape
    dx = out if out is not None else torch.empty_like(dy)
    _lib.call("rmsnorm_bwd", *yq.ptrs(), rstd.data_ptr(), gain.data_ptr(), dy.data_ptr(), M, H, dx.data_ptr(),
              _stream())
    return dx


def silu_mul_bwd_quant(gq: NVFP4Tensor, uq: NVFP4Tensor, dh: torch.Tensor, out=None):
    """(dgate, dup, Q(dgate), Q(dup)): silu_mul_bwd plus the NVFP4 copies of its outputs."""
    _dense(_bf16(dh, "dh"), "dh")
    M, I = dh.shape
    if out is None:
        out = (torch.empty_like(dh), torch.empty_like(dh), empty_nvfp4(M, I, dh.device), empty_nvfp4(M, I, dh.device))
    dg, du, dgq, duq = out
    _lib.call("silu_mul_bwd_quant", *gq.ptrs(), *uq.ptrs(), dh.data_ptr(), M, I, dg.data_ptr(), du.data_ptr(),
              *dgq.ptrs(), *duq.ptrs(), _stream())
    return dg, du, dgq, duq


def rmsnorm_bwd_residual(yq: NVFP4Tensor, rstd: torch.Tensor, gain: torch.Tensor, dy: torch.Tensor,
                         resid: torch.Tensor | None = None, quantize_out: bool = True, out=None):
    """(out, Q(out) or None) with out = bf16(bf16(rmsnorm_bwd) + resid)."""
    _bf16(gain, "gain"); _dense(_bf16(dy, "dy"), "dy")
    if resid is not None:
        _dense(_bf16(resid, "resid"), "resid")
        if resid.shape != dy.shape:
            raise ValueError("resid must have dy's shape")
    M, H = dy.shape
    if out is None:
        out = (torch.empty_like(dy), empty_nvfp4(M, H, dy.device) if quantize_out else None)
    dx, q = out
    qp = q.ptrs() if q is not None else (0, 0, 0)
    _lib.call("rmsnorm_bwd_residual", *yq.ptrs(), rstd.data_ptr(), gain.data_ptr(), dy.data_ptr(),
              resid.data_ptr() if resid is not None else 0, M, H, dx.data_ptr(), *qp, _stream())
    return dx, q


# ---------------------------------------------------------------------------
# MXFP4 variant (32-element blocks, E8M0 scales)
# ---------------------------------------------------------------------------
class MXFP4Tensor:
    """MXFP4 tensor [rows x cols]: codes uint8 [rows, cols/2], E8M0 scales uint8 [rows, cols/32]."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        self.codes, self.scales = codes, scales

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def cols(self) -> int:
        return self.codes.shape[1] * 2

    def ptrs(self):
        return self.codes.data_ptr(), self.scales.data_ptr()


def empty_mxfp4(rows: int, cols: int, device="cuda") -> MXFP4Tensor:
    if cols % 32:
        raise ValueError("MXFP4 needs cols % 32 == 0")
    return MXFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                       torch.empty((rows, cols // 32), dtype=torch.uint8, device=device))


def mx_quantize(x: torch.Tensor, transpose: bool = False, out: MXFP4Tensor | None = None) -> MXFP4Tensor:
    """MXFP4 of x [rows x cols] (or of x^T with ``transpose``)."""
    _bf16(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    rows, cols = (x.shape[1], x.shape[0]) if transpose else (x.shape[0], x.shape[1])
    out = out if out is not None else empty_mxfp4(rows, cols, x.device)
    _lib.call("mxfp4_quantize", x.data_ptr(), rows, cols, x.stride(0), int(transpose), *out.ptrs(), _stream())
    return out


def mx_weight_layouts(w: torch.Tensor):
    """(W_fwd, W_bwd) = (Q(W), Q(W^T)) in MXFP4 for a BF16 weight W [N x K]."""
    return mx_quantize(w), mx_quantize(w, transpose=True)


def mx_rmsnorm_quant(x: torch.Tensor, gain: torch.Tensor, eps: float = 1e-5, out=None):
    """(MXFP4(y), rstd) with y = (x * rstd) * gain; ``out`` = (MXFP4Tensor, rstd) to reuse buffers."""
    _bf16(x, "x"); _bf16(gain, "gain")
    M, H = x.shape
    if out is not None:
        y, rstd = out
    else:
        y = empty_mxfp4(M, H, x.device)
        rstd = torch.empty((M,), dtype=torch.float32, device=x.device)
    _lib.call("mxfp4_rmsnorm_quant", x.data_ptr(), gain.data_ptr(), float(eps), M, H, x.stride(0), *y.ptrs(),
              rstd.data_ptr(), _stream())
    return y, rstd


def mx_silu_mul_quant(gate: torch.Tensor, up: torch.Tensor, out=None):
    """(MXFP4(h), MXFP4(gate), MXFP4(up)) with h = silu(gate) * up; ``out`` = three MXFP4Tensors."""
    _bf16(gate, "gate"); _bf16(up, "up")
    if gate.shape != up.shape or gate.stride() != up.stride():
        raise ValueError("gate and up must have the same shape and strides")
    M, I = gate.shape
    h, gq, uq = out if out is not None else (empty_mxfp4(M, I, gate.device) for _ in range(3))
    _lib.call("mxfp4_silu_mul_quant", gate.data_ptr(), up.data_ptr(), M, I, gate.stride(0), *h.ptrs(), *gq.ptrs(),
              *uq.ptrs(), _stream())
    return h, gq, uq


def mx_silu_mul_bwd_quant(gq: MXFP4Tensor, uq: MXFP4Tensor, dh: torch.Tensor, out=None):
    """(dgate, dup, MXFP4(dgate), MXFP4(dup)) from the MXFP4 state of silu_mul."""
    _dense(_bf16(dh, "dh"), "dh")
    M, I = dh.shape
    if out is None:
        out = (torch.empty_like(dh), torch.empty_like(dh), empty_mxfp4(M, I, dh.device), empty_mxfp4(M, I, dh.device))
    dg, du, dgq, duq = out
    _lib.call("mxfp4_silu_mul_bwd_quant", *gq.ptrs(), *uq.ptrs(), dh.data_ptr(), M, I, dg.data_ptr(), du.data_ptr(),
              *dgq.ptrs(), *duq.ptrs(), _stream())
    return dg, du, dgq, duq


def mx_rmsnorm_bwd_residual(yq: MXFP4Tensor, rstd: torch.Tensor, gain: torch.Tensor, dy: torch.Tensor,
                            resid: torch.Tensor | None = None, quantize_out: bool = True, out=None):
    """(out, MXFP4(out) or None) with out = bf16(bf16(rmsnorm_bwd) + resid) from an MXFP4 state."""
    _bf16(gain, "gain"); _dense(_bf16(dy, "dy"), "dy")
    if resid is not None:
        _dense(_bf16(resid, "resid"), "resid")
        if resid.shape != dy.shape:
            raise ValueError("resid must have dy's shape")
    M, H = dy.shape
    if out is None:
        out = (torch.empty_like(dy), empty_mxfp4(M, H, dy.device) if quantize_out else None)
    dx, q = out
    qp = q.ptrs() if q is not None else (0, 0)
    _lib.call("mxfp4_rmsnorm_bwd_residual", *yq.ptrs(), rstd.data_ptr(), gain.data_ptr(), dy.data_ptr(),
              resid.data_ptr() if resid is not None else 0, M, H, dx.data_ptr(), *qp, _stream())
    return dx, q


def mx_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out: torch.Tensor | None = None, accumulate: bool = False):
    """C = bf16([f32(C) +] deq(a) deq(b)^T) for MXFP4 a [M x K], b [N x K]."""
    M, K = a.rows, a.cols
    N = b.rows
    if b.cols != K:
        raise ValueError(f"K mismatch: {K} vs {b.cols}")
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing output")
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    _lib.call("mxfp4_gemm", *a.ptrs(), M, K, *b.ptrs(), N, out.data_ptr(), out.stride(0), int(accumulate),
              _stream())
    return out


# fail loudly at import if the native library is missing
load()
