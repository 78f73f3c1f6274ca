#!/usr/bin/env python3
"""Benchmark of the NVFP4 frozen-projection hot path on one MI355X.

One step is one pass of the whole path over --layers (default 4) distinct
Llama-3B-shaped decoder layers' frozen projections at M = 4096 tokens
(batch 4 x seq 1024), LoRA rank 16 -- distinct weights and buffers per layer,
about 1 GB each, so operands stream from HBM rather than the 256 MB
last-level cache.  Forward through every layer, then backward from the top
layer down, each layer's input gradient (the residual stream) being the
output gradient of the layer below:

  forward   rmsnorm_quant -> q/k/v (lora_down + NVFP4 GEMM with LoRA term)
            nvfp4_quantize(attention output) -> o
            rmsnorm_quant -> gate/up -> silu_mul_quant -> down
  backward  down (its dY = the layer's output gradient, already NVFP4)
            silu_mul_bwd_quant (BF16 da, db and their NVFP4 copies) -> gate, up
            rmsnorm_bwd_residual (+ the output gradient; NVFP4 copy) -> o
            q/k/v (nvfp4_quantize of the attention-backward gradients)
            rmsnorm_bwd_residual (+ the MLP-block residual gradient; NVFP4 copy)
  per projection: lora_bwd; per input: one NVFP4 dgrad launch with the LoRA
  input-gradient terms (q/k/v and gate/up each sum into one dX in a single
  nvfp4_gemm_dgrad_multi launch; down and o alone)

The metric is the NVFP4 fwd + dgrad GEMM throughput of the step:
  value = (GEMM FLOPs per step) / (wall time per step)   [TFLOP/s]
with every other kernel of the step inside the timed region.  Inputs are
synthetic (seeded, BF16, resident in HBM before timing); weights are random
N(0, 0.02) quantized once to their two cached NVFP4 layouts (one per direction)
(offline, untimed).

A second leg times the MXFP4 variant (32-element blocks, E8M0 scales) on the
same shapes: the 7 forward and 7 input-gradient GEMMs of each layer instance,
with MXFP4 operands quantized beforehand, as HIP-graph replays; it is reported
under "mxfp4_variant" and is not part of "value".

A third leg ("recipe_variants") times the Q/K/V and gate/up GEMMs with
stacked weights against separate ones, and the quantizer's variants; a fourth
("single_layout_dgrad") the input-gradient GEMMs over the forward weight
layout only against the dual-layout ones.  "quantizer_bandwidth" times nvfp4_quantize
alone at the workloads' activation shapes (up to the 8B-scale 16384 x 14336).  "lora_term" times each
projection's GEMMs with and without the fused LoRA term; "mfma_loop_peak" is
the measured back-to-back MFMA rate (FP16 and scaled FP4) and the clock held
under it, reported beside the published peaks.

Prints one JSON line.  --gpus must be 1: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp16_mfma_tflops": 2500.0, "fp4_mfma_tflops": 10100.0, "hbm_gbs": 8000.0}
LORA_SCALE = 2.0
HEAD_START_CYCLES = 40_000_000      # spin ahead of each instrumented step (about 20 ms)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on host cores")
    ap.add_argument("--cpu-sample-rows", type=int, default=256)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--sequential", action="store_true",
                    help="one stream: no concurrent branches (q/k/v and gate/up forward, their LoRA backwards)")
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct decoder-layer instances a step runs through (their weights and buffers "
                         "together exceed the 256 MB last-level cache, so every operand streams from HBM)")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip the MXFP4-variant GEMM leg")
    ap.add_argument("--no-recipes", action="store_true",
                    help="skip the recipe, single-layout, quantizer-bandwidth and LoRA-term legs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB read + 1 GiB write elementwise kernel (counter calibration)")
    return ap.parse_args()


class Layer:
    """Device state of one synthetic Llama-3B decoder layer's frozen-projection path."""

    def __init__(self, fw, torch, synth, wl, index=0):
        self.fw, self.torch = fw, torch
        off = 1000 * index                     # distinct seeded tensors per layer instance
        M = wl.tokens
        H, I = 3072, 8192
        KV = [p.d_out for p in wl.projections if p.name == "k"][0]
        r = wl.lora_rank
        self.M, self.H, self.I, self.KV, self.r = M, H, I, KV, r
        dev = torch.device("cuda:0")

        def up(bits):
            import numpy as np
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        act = lambda tid, cols: up(synth.workload_activation(wl, M, cols, off + tid))
        self.h1, self.h2, self.attn = act(10, H), act(11, H), act(12, H)
        self.g1 = up(synth.uniform_bf16((H,), 0.9, 1.1, wl.wid, off + 13))
        self.g2 = up(synth.uniform_bf16((H,), 0.9, 1.1, wl.wid, off + 14))
        grad = lambda tid, cols: up(synth.normal_bf16((M, cols), wl.dy_std, wl.wid, off + tid))
        self.dOut = grad(15, H)                    # output gradient entering the stack (top layer)
        self.dOut_q = fw.empty_nvfp4(M, H, dev)
        self.dq, self.dk, self.dv = grad(17, H), grad(18, KV), grad(19, KV)

        self.proj = {}
        for i, p in enumerate(wl.projections):
            w = up(synth.normal_bf16((p.d_out, p.d_in), wl.w_std, wl.wid, off + 20 + i))
            wf, wb = fw.weight_layouts(w)
            del w                                # only the cached NVFP4 layouts stay resident
            A = up(synth.normal_bf16((r, p.d_in), wl.a_std, wl.wid, off + 40 + i))
            B = torch.zeros((p.d_out, r), dtype=torch.bfloat16, device=dev)
            self.proj[p.name] = dict(p=p, wf=wf, wb=wb, A=A, B=B,
                                     T=torch.empty((M, r), dtype=torch.bfloat16, device=dev),
                                     Y=torch.empty((M, p.d_out), dtype=torch.bfloat16, device=dev),
                                     dT=torch.empty((M, r), dtype=torch.bfloat16, device=dev),
                                     dA=torch.empty((r, p.d_in), dtype=torch.bfloat16, device=dev),
                                     dB=torch.empty((p.d_out, r), dtype=torch.bfloat16, device=dev),
                                     dyq=fw.empty_nvfp4(M, p.d_out, dev))
        # a LoRA-backward workspace per projection (the gate/up and q/k/v LoRA
        # backwards may run concurrently on side streams)
        for P in self.proj.values():
            p = P["p"]
            P["ws"] = torch.empty((fw._lib.lora_bwd_workspace_size(M, p.d_in, p.d_out, r),), dtype=torch.uint8,
                                  device=dev)
        nv = lambda cols: fw.empty_nvfp4(M, cols, dev)
        self.y1q, self.y2q, self.aq = nv(H), nv(H), nv(H)
        self.rstd1 = torch.empty((M,), dtype=torch.float32, device=dev)
        self.rstd2 = torch.empty((M,), dtype=torch.float32, device=dev)
        self.hq, self.gq, self.uq = nv(I), nv(I), nv(I)
        bf = lambda cols: torch.empty((M, cols), dtype=torch.bfloat16, device=dev)
        self.dh, self.da, self.db = bf(I), bf(I), bf(I)
        self.daq, self.dbq = nv(I), nv(I)
        self.dy1, self.dy2, self.dattn = bf(H), bf(H), bf(H)
        self.dh2, self.dh1 = bf(H), bf(H)                   # residual-stream gradients (BF16)
        self.dh2q, self.dh1q = nv(H), nv(H)                 # their NVFP4 copies
        self.record = None       # list to append (category, name, start_event, end_event, work) into
        self.streams = None      # two side streams: independent branches of the step run concurrently

    # ---- instrumented launch helper ----
    def _ev(self, cat, name, work, fn):
        if self.record is None:
            return fn()
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fn()
        e1.record()
        self.record.append((cat, name, e0, e1, work))
        return out

    def _fwd_proj(self, name, xq):
        fw, P = self.fw, self.proj[name]
        p = P["p"]
        self._ev("lora", "lora_down", None, lambda: fw.lora_down(xq, P["A"], out=P["T"]))
        work = ("gemm", self.M, p.d_out, (p.d_in,), False)      # M, Nout, contraction segments, accumulate
        self._ev("gemm", f"fwd {name}", work,
                 lambda: fw.gemm_fwd(xq, P["wf"], lora_t=P["T"], lora_b=P["B"], lora_scale=LORA_SCALE, out=P["Y"]))
        return P["Y"]

    def _bwd_lora(self, name, xq, dy, dyq=None):
        """dY's NVFP4 copy (unless a fused kernel made it) and the LoRA
        backward of one projection; returns the NVFP4 dY."""
        fw, P = self.fw, self.proj[name]
        p = P["p"]
        if dyq is None:
            dyq = P["dyq"]
            self._ev("quant", "nvfp4_quantize", ("quant", self.M, p.d_out), lambda: fw.quantize(dy, out=dyq))
        self._ev("lora", "lora_bwd", None,
                 lambda: fw.lora_bwd(xq, P["A"], P["B"], dy, LORA_SCALE, out=(P["dT"], P["dA"], P["dB"]),
                                     workspace=P["ws"]))
        return dyq

    def _bwd_dgrad(self, name, dyq, dx, accumulate):
        """Input-gradient GEMM of one projection with its LoRA term dT A."""
        fw, P = self.fw, self.proj[name]
        p = P["p"]
        work = ("gemm", self.M, p.d_in, (p.d_out,), bool(accumulate))
        self._ev("gemm", f"dgrad {name}", work,
                 lambda: fw.gemm_dgrad(dyq, P["wb"], out=dx, accumulate=accumulate, lora_dt=P["dT"],
                                       lora_a=P["A"]))

    def _bwd_proj(self, name, xq, dy, dx, accumulate, dyq=None):
        self._bwd_dgrad(name, self._bwd_lora(name, xq, dy, dyq), dx, accumulate)

    def _bwd_dgrad_multi(self, names, dx):
        """One input-gradient launch summing the projections that read one
        input (each with its LoRA term dT A)."""
        fw = self.fw
        Ps = [self.proj[n] for n in names]
        work = ("gemm", self.M, Ps[0]["p"].d_in, tuple(P["p"].d_out for P in Ps), False)
        self._ev("gemm", "dgrad " + "/".join(names), work,
                 lambda: fw.gemm_dgrad_multi([(P["dyq"], P["wb"]) for P in Ps], out=dx,
                                             lora=[(P["dT"], P["A"]) for P in Ps]))

    def _fork(self, fns):
        """Launch fns on the side streams, each after the current stream's
        work so far; returns a join function that makes the current stream wait
        for side branch i (or all of them).  Without side streams (or while the
        step is instrumented) the branches run in place, in order."""
        if self.streams is None or self.record is not None:
            for f in fns:
                f()
            return lambda i=None: None
        torch = self.torch
        cur = torch.cuda.current_stream()
        side = self.streams[:len(fns)]
        for st, f in zip(side, fns):
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                f()

        def join(i=None):
            for st in (side if i is None else [side[i]]):
                cur.wait_stream(st)
        return join

    def _branches(self, fns):
        """fns[0] on the current stream, fns[1:] concurrently on side streams;
        the current stream then waits for all of them."""
        join = self._fork(fns[1:])
        fns[0]()
        join()

    def forward(self):
        fw = self.fw
        M, H, I = self.M, self.H, self.I
        self._ev("quant", "rmsnorm_quant", ("rmsq", M, H),
                 lambda: fw.rmsnorm_quant(self.h1, self.g1, 1e-5, out=(self.y1q, self.rstd1)))
        # q, k and v read the same NVFP4 input and are independent
        self._branches([lambda n=n: self._fwd_proj(n, self.y1q) for n in ("q", "k", "v")])
        self._ev("quant", "nvfp4_quantize", ("quant", M, H), lambda: fw.quantize(self.attn, out=self.aq))
        self._fwd_proj("o", self.aq)
        self._ev("quant", "rmsnorm_quant", ("rmsq", M, H),
                 lambda: fw.rmsnorm_quant(self.h2, self.g2, 1e-5, out=(self.y2q, self.rstd2)))
        self._branches([lambda: self._fwd_proj("gate", self.y2q), lambda: self._fwd_proj("up", self.y2q)])
        a, b = self.proj["gate"]["Y"], self.proj["up"]["Y"]
        self._ev("quant", "silu_mul_quant", ("silu", M, I),
                 lambda: fw.silu_mul_quant(a, b, out=(self.hq, self.gq, self.uq)))
        self._fwd_proj("down", self.hq)

    def backward(self, dout, dout_q):
        """Backward of the layer given the gradient of its output (BF16 and its
        NVFP4 copy); returns the gradient of its input, the residual stream
        (Table 7 row "Residuals": the residual gradients are summed in BF16)."""
        fw = self.fw
        M, H, I = self.M, self.H, self.I
        # MLP block: out = h2 + down(silu(gate(n2)) * up(n2)),  n2 = rmsnorm(h2)
        self._bwd_proj("down", self.hq, dout, self.dh, False, dyq=dout_q)
        self._ev("bwd", "silu_mul_bwd_quant", ("silubq", M, I),
                 lambda: fw.silu_mul_bwd_quant(self.gq, self.uq, self.dh, out=(self.da, self.db, self.daq, self.dbq)))
        # the gate and up LoRA backwards run side by side; one input-gradient
        # launch sums both projections into dX
        self.proj["gate"]["dyq"], self.proj["up"]["dyq"] = self.daq, self.dbq
        self._branches([lambda: self._bwd_lora("gate", self.y2q, self.da, self.daq),
                        lambda: self._bwd_lora("up", self.y2q, self.db, self.dbq)])
        self._bwd_dgrad_multi(("gate", "up"), self.dy2)
        self._ev("bwd", "rmsnorm_bwd_residual", ("rmsbr", M, H),
                 lambda: fw.rmsnorm_bwd_residual(self.y2q, self.rstd2, self.g2, self.dy2, resid=dout,
                                                 out=(self.dh2, self.dh2q)))
        # attention block: h2 = h1 + o(attn(q, k, v of n1)),  n1 = rmsnorm(h1); the
        # attention backward itself is not part of the path (dq, dk, dv are inputs)
        self._bwd_proj("o", self.aq, self.dh2, self.dattn, False, dyq=self.dh2q)
        self._branches([lambda n=n, d=d: self._bwd_lora(n, self.y1q, d)
                        for n, d in (("q", self.dq), ("k", self.dk), ("v", self.dv))])
        self._bwd_dgrad_multi(("q", "k", "v"), self.dy1)
        self._ev("bwd", "rmsnorm_bwd_residual", ("rmsbr", M, H),
                 lambda: fw.rmsnorm_bwd_residual(self.y1q, self.rstd1, self.g1, self.dy1, resid=self.dh2,
                                                 out=(self.dh1, self.dh1q)))
        return self.dh1, self.dh1q

    def gemm_flops(self):
        return sum(4 * self.M * P["p"].d_in * P["p"].d_out for P in self.proj.values())


class MxLayer:
    """The same layer's projections in the MXFP4 variant: cached W_fwd / W_bwd in
    MXFP4 (quantized once, untimed) and MXFP4 GEMM inputs; a step is the 7
    forward and 7 input-gradient GEMMs."""

    def __init__(self, fw, torch, synth, wl, index=0):
        import numpy as np
        self.fw, self.torch = fw, torch
        off = 5000 + 1000 * index
        M = wl.tokens
        dev = torch.device("cuda:0")
        up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
        self.M, self.items = M, []
        for i, p in enumerate(wl.projections):
            w = up(synth.normal_bf16((p.d_out, p.d_in), wl.w_std, wl.wid, off + 20 + i))
            wf, wb = fw.mx_weight_layouts(w)
            del w
            xq = fw.mx_quantize(up(synth.workload_activation(wl, M, p.d_in, off + 60 + i)))
            dyq = fw.mx_quantize(up(synth.normal_bf16((M, p.d_out), wl.dy_std, wl.wid, off + 80 + i)))
            self.items.append(dict(p=p, wf=wf, wb=wb, xq=xq, dyq=dyq,
                                   Y=torch.empty((M, p.d_out), dtype=torch.bfloat16, device=dev),
                                   dX=torch.empty((M, p.d_in), dtype=torch.bfloat16, device=dev)))
        self.record = None

    def step(self):
        fw, torch = self.fw, self.torch
        for it in self.items:
            p = it["p"]
            for what, a, b, out, n, k in (("fwd", it["xq"], it["wf"], it["Y"], p.d_out, p.d_in),
                                          ("dgrad", it["dyq"], it["wb"], it["dX"], p.d_in, p.d_out)):
                if self.record is None:
                    fw.mx_gemm(a, b, out=out)
                else:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fw.mx_gemm(a, b, out=out)
                    e1.record()
                    self.record.append((e0, e1, (self.M, n, k)))

    def gemm_flops(self):
        return sum(4 * self.M * it["p"].d_in * it["p"].d_out for it in self.items)


def mxfp4_leg(fw, torch, synth, wl, nlayers, steps, warmup, eager=False):
    """Throughput of the MXFP4 variant's GEMMs (same shapes, same rotation over
    distinct layer instances, HIP-graph replays unless ``eager``) and its
    dominant kernel."""
    from frozen_weight_gemms_amd import _lib
    layers = [MxLayer(fw, torch, synth, wl, li) for li in range(nlayers)]

    def step():
        for ly in layers:
            ly.step()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if not eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run = graph.replay
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    recs = []
    for ly in layers:
        ly.record = recs
    for _ in range(steps):
        torch.cuda._sleep(HEAD_START_CYCLES)
        step()
    torch.cuda.synchronize()
    by_tile = {}
    for e0, e1, (M, N, K) in recs:
        t = by_tile.setdefault(_lib.gemm_tile(M, N, K), [0.0, 0.0, 0])
        t[0] += e0.elapsed_time(e1)
        t[1] += 2.0 * M * N * K
        t[2] += 1
    dom = max(by_tile, key=lambda k: by_tile[k][0])
    dt, dfl, dn = by_tile[dom]
    ach = dfl / (dt * 1e-3) / 1e12
    flops = sum(ly.gemm_flops() for ly in layers)
    gemm_ms = sum(v[0] for v in by_tile.values()) / steps
    value = flops / (ms * 1e-3) / 1e12
    del layers, run
    torch.cuda.synchronize()
    kname = f"pact::k_gemm_mxfp4<{dom[0] // 64}, {dom[1] // 64}>"
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "mxfp4_gemm_traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            if tj.get("src_hash") == src_hash("mxfp4.hip", "lds_dma.h") and tj.get("kernel") == kname:
                traffic = tj.get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None
    return {"gemm_tflops": round(value, 1), "frac_fp4_peak": round(value / PEAK["fp4_mfma_tflops"], 4),
            "ms_per_step": round(ms, 4), "layers": nlayers,
            "gemm_only_tflops_events": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
            "timed_region": ("eager" if eager else "hip graph replays") + " of 14 MXFP4 GEMMs per layer",
            "roofline": {"kernel": kname, "bound": "mfma",
                         "achieved": round(ach, 1), "peak": PEAK["fp4_mfma_tflops"], "unit": "TFLOP/s",
                         "frac": round(ach / PEAK["fp4_mfma_tflops"], 4), "launches_per_step": dn // steps,
                         "avg_launch_us": round(dt * 1e3 / dn, 2), "traffic": traffic}}


def recipe_leg(fw, torch, synth, wl, n_inst=4, reps=5):
    """The recipe variants at the Llama-3B shapes (M = 4096), over n_inst
    rotating instances: the Q/K/V and gate/up forward and input-gradient GEMMs
    with separate weights versus stacked weights (one GEMM per group, the
    stacked dgrad summing every consumer), and the quantizer's variants on a
    [4096 x 3072] output gradient."""
    import numpy as np
    M, H, I, KV = wl.tokens, 3072, 8192, 1024
    dev = torch.device("cuda:0")
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    bf = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=dev)
    inst = []
    for i in range(n_inst):
        off = 9000 + 100 * i
        d = {"x": fw.quantize(up(synth.workload_activation(wl, M, H, off)))}
        w = {n: up(synth.normal_bf16((rows, H), wl.w_std, wl.wid, off + k))
             for k, (n, rows) in enumerate((("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I)))}
        d["sep"] = {n: fw.weight_layouts(t) for n, t in w.items()}
        d["qkv"] = fw.weight_layouts(torch.cat([w["q"], w["k"], w["v"]], 0).contiguous())
        d["gu"] = fw.weight_layouts(torch.cat([w["gate"], w["up"]], 0).contiguous())
        del w
        dy = {n: up(synth.normal_bf16((M, c), wl.dy_std, wl.wid, off + 10 + k))
              for k, (n, c) in enumerate((("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I)))}
        d["dyq"] = {n: fw.quantize(t) for n, t in dy.items()}
        d["dy_qkv"] = fw.quantize(torch.cat([dy["q"], dy["k"], dy["v"]], 1).contiguous())
        d["dy_gu"] = fw.quantize(torch.cat([dy["gate"], dy["up"]], 1).contiguous())
        del dy
        d["y"] = {n: bf(M, c) for n, c in (("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I))}
        d["y_qkv"], d["y_gu"], d["dx1"], d["dx2"] = bf(M, H + 2 * KV), bf(M, 2 * I), bf(M, H), bf(M, H)
        inst.append(d)

    def separate(d):
        for n in ("q", "k", "v", "gate", "up"):
            fw.gemm_fwd(d["x"], d["sep"][n][0], out=d["y"][n])
        for k, n in enumerate(("q", "k", "v")):
            fw.gemm_dgrad(d["dyq"][n], d["sep"][n][1], out=d["dx1"], accumulate=k > 0)
        for k, n in enumerate(("gate", "up")):
            fw.gemm_dgrad(d["dyq"][n], d["sep"][n][1], out=d["dx2"], accumulate=k > 0)

    def stacked(d):
        fw.gemm_fwd(d["x"], d["qkv"][0], out=d["y_qkv"])
        fw.gemm_fwd(d["x"], d["gu"][0], out=d["y_gu"])
        fw.gemm_dgrad(d["dy_qkv"], d["qkv"][1], out=d["dx1"])
        fw.gemm_dgrad(d["dy_gu"], d["gu"][1], out=d["dx2"])

    def timed(fn):
        best = 1e30
        for _ in range(reps):
            torch.cuda._sleep(HEAD_START_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for d in inst:
                fn(d)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / len(inst))
        return best

    for fn in (separate, stacked):
        for d in inst:
            fn(d)
    torch.cuda.synchronize()
    flops = 2.0 * M * H * (H + 2 * KV + 2 * I) * 2          # forward + input gradient
    t_sep, t_cat = timed(separate), timed(stacked)
    out = {"stacked_qkv_gate_up": {"separate_tflops": round(flops / (t_sep * 1e-3) / 1e12, 1),
                                   "stacked_tflops": round(flops / (t_cat * 1e-3) / 1e12, 1),
                                   "separate_ms": round(t_sep, 4), "stacked_ms": round(t_cat, 4),
                                   "launches": {"separate": 10, "stacked": 4}}}
    # quantizer variants on [M x H]
    xs = [up(synth.normal_bf16((M, H), wl.dy_std, wl.wid, 9900 + i)) for i in range(n_inst)]
    qs = [fw.empty_nvfp4(M, H, dev) for _ in range(n_inst)]
    amax = torch.empty((), dtype=torch.float32, device=dev)
    variants = {"default": lambda x, q: fw.quantize(x, out=q),
                "round_up_scales": lambda x, q: fw.quantize_ex(x, round_up=True, out=q),
                "tensor_scale_two_pass": lambda x, q: fw.quantize_ex(x, tensor_scale=True, amax=amax, out=q)}
    qb = {}
    for name, f in variants.items():
        for x, q in zip(xs, qs):
            f(x, q)
        torch.cuda.synchronize()
        best = 1e30
        for _ in range(reps):
            torch.cuda._sleep(HEAD_START_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for x, q in zip(xs, qs):
                f(x, q)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / len(xs))
        qb[name] = {"us": round(best * 1e3, 2),
                    "GB/s": round(kernel_bytes("quant", M, H) / (best * 1e-3) / 1e9, 1)}
    out["quantizer_4096x3072"] = qb
    del inst, xs, qs
    torch.cuda.synchronize()
    return out


def quantizer_leg(fw, torch, reps=5):
    """nvfp4_quantize alone on the activation shapes of the workloads: the
    Llama-3B hidden and intermediate widths at M = 4096 and the 8B-scale ones
    at M = 16384.  Four distinct seeded inputs per shape (the same rotation
    rule as the step, so small shapes are not served from the Infinity Cache),
    back-to-back launches after a spin-kernel head start, best of `reps`."""
    dev = "cuda"
    gen = torch.Generator(device=dev)
    out = {}
    for M, K in ((4096, 3072), (4096, 8192), (16384, 4096), (16384, 14336)):
        gen.manual_seed(M * 7 + K)
        xs = [(torch.randn((M, K), generator=gen, device=dev) * 0.01).to(torch.bfloat16) for _ in range(4)]
        qs = [fw.empty_nvfp4(M, K, dev) for _ in range(4)]
        for x, q in zip(xs, qs):
            fw.quantize(x, out=q)
        torch.cuda.synchronize()
        best = 1e30
        for _ in range(reps):
            torch.cuda._sleep(HEAD_START_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for x, q in zip(xs, qs):
                fw.quantize(x, out=q)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / len(xs))
        gbs = kernel_bytes("quant", M, K) / (best * 1e-3) / 1e9
        out[f"{M}x{K}"] = {"us": round(best * 1e3, 2), "GB/s": round(gbs, 1),
                           "frac_hbm": round(gbs / PEAK["hbm_gbs"], 3)}
        del xs, qs
        torch.cuda.synchronize()
    return out


def lora_term_leg(fw, torch, synth, wl, reps=3, n=10):
    """Cost of the LoRA term inside the frozen GEMMs: each projection's forward
    (s T B^T) and input-gradient (dT A) GEMM timed with and without the term,
    back-to-back launches after a spin-kernel head start, best of `reps`.
    Reported per projection and as the sum over one decoder layer's seven
    projections (each with its own launch; the step merges q/k/v and gate/up
    input gradients, so this is an upper bound for those)."""
    dev = "cuda"
    M, r = wl.tokens, wl.lora_rank
    up = lambda b: torch.from_numpy(b.view("int16")).view(torch.bfloat16).to(dev)

    def best_us(fn):
        fn()
        torch.cuda.synchronize()
        best = 1e30
        for _ in range(reps):
            torch.cuda._sleep(HEAD_START_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / n)
        return best

    out, tot = {}, 0.0
    seen = {}
    for i, p in enumerate(wl.projections):
        key = (p.d_in, p.d_out)
        if key not in seen:
            x = up(synth.activations_bf16((M, p.d_in), wl.wid, 9800 + i))
            w = up(synth.normal_bf16((p.d_out, p.d_in), wl.w_std, wl.wid, 9810 + i))
            dy = up(synth.normal_bf16((M, p.d_out), wl.dy_std, wl.wid, 9820 + i))
            T = up(synth.normal_bf16((M, r), 0.3, wl.wid, 9830 + i))
            B = up(synth.normal_bf16((p.d_out, r), wl.a_std, wl.wid, 9840 + i))
            A = up(synth.normal_bf16((r, p.d_in), wl.a_std, wl.wid, 9850 + i))
            dT = up(synth.normal_bf16((M, r), 0.01, wl.wid, 9860 + i))
            xq, wf, wb, dyq = fw.quantize(x), fw.quantize(w), fw.quantize(w, transpose=True), fw.quantize(dy)
            y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device=dev)
            dx = torch.empty((M, p.d_in), dtype=torch.bfloat16, device=dev)
            f0 = best_us(lambda: fw.gemm_fwd(xq, wf, out=y))
            f1 = best_us(lambda: fw.gemm_fwd(xq, wf, lora_t=T, lora_b=B, lora_scale=LORA_SCALE, out=y))
            d0 = best_us(lambda: fw.gemm_dgrad(dyq, wb, out=dx))
            d1 = best_us(lambda: fw.gemm_dgrad(dyq, wb, out=dx, lora_dt=dT, lora_a=A))
            seen[key] = {"fwd_us": round(f0, 2), "fwd_lora_us": round(f1, 2),
                         "dgrad_us": round(d0, 2), "dgrad_lora_us": round(d1, 2)}
            del x, w, dy, xq, wf, wb, dyq, y, dx
        out[p.name] = seen[key]
        tot += (seen[key]["fwd_lora_us"] - seen[key]["fwd_us"]) + (seen[key]["dgrad_lora_us"] - seen[key]["dgrad_us"])
    torch.cuda.synchronize()
    return {"per_projection": out, "lora_term_us_per_layer": round(tot, 1)}


def single_layout_leg(fw, torch, synth, wl, n_inst=4, reps=5):
    """Input-gradient GEMMs of the 7 projections per layer over the forward
    layout only (single-layout dgrad) versus over the cached backward layout,
    same shapes and rotation over n_inst layer instances; cached weight bytes
    per layer for both."""
    import numpy as np
    M = wl.tokens
    dev = torch.device("cuda:0")
    up = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    inst = []
    for i in range(n_inst):
        off = 12000 + 100 * i
        items = []
        for k, p in enumerate(wl.projections):
            w = up(synth.normal_bf16((p.d_out, p.d_in), wl.w_std, wl.wid, off + k))
            wf, wb = fw.weight_layouts(w)
            del w
            items.append(dict(p=p, wf=wf, wb=wb, sl=fw.SingleLayoutWeight(wf),
                              dyq=fw.quantize(up(synth.normal_bf16((M, p.d_out), wl.dy_std, wl.wid, off + 20 + k))),
                              dx=torch.empty((M, p.d_in), dtype=torch.bfloat16, device=dev)))
        inst.append(items)

    def dual(items):
        for it in items:
            fw.gemm_dgrad(it["dyq"], it["wb"], out=it["dx"])

    def single(items):
        for it in items:
            fw.gemm_dgrad_fwd_layout(it["dyq"], it["sl"], out=it["dx"])

    for fn in (dual, single):
        for items in inst:
            fn(items)
    torch.cuda.synchronize()

    def timed(fn):
        best = 1e30
        for _ in range(reps):
            torch.cuda._sleep(HEAD_START_CYCLES)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for items in inst:
                fn(items)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / len(inst))
        return best

    # dominant launch of the single-layout kernel: per-launch times of the largest shapes
    per = {}
    for it in inst[0]:
        p = it["p"]
        best = 1e30
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for items in inst:
                fw.gemm_dgrad_fwd_layout(items[[q["p"].name for q in items].index(p.name)]["dyq"],
                                         items[[q["p"].name for q in items].index(p.name)]["sl"],
                                         out=items[[q["p"].name for q in items].index(p.name)]["dx"])
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) / len(inst))
        per[p.name] = (best, 2.0 * M * p.d_in * p.d_out)
    flops = sum(2.0 * M * it["p"].d_in * it["p"].d_out for it in inst[0])
    t_dual, t_single = timed(dual), timed(single)
    nv = lambda r, c: r * c * 9 // 16 + 4 * r
    bytes_dual = sum(nv(it["p"].d_out, it["p"].d_in) + nv(it["p"].d_in, it["p"].d_out) for it in inst[0])
    bytes_single = sum(nv(it["p"].d_out, it["p"].d_in) + 4 for it in inst[0])
    name = max(per, key=lambda k: per[k][0])
    t, f = per[name]
    del inst
    torch.cuda.synchronize()
    return {"dual_layout_tflops": round(flops / (t_dual * 1e-3) / 1e12, 1),
            "single_layout_tflops": round(flops / (t_single * 1e-3) / 1e12, 1),
            "dual_ms_per_layer": round(t_dual, 4), "single_ms_per_layer": round(t_single, 4),
            "cached_weight_mb_per_layer": {"dual": round(bytes_dual / 1e6, 2), "single": round(bytes_single / 1e6, 2)},
            "roofline": {"kernel": "pact::k_gemm_dgrad_fwdlayout<4>", "projection": name, "bound": "mfma",
                         "achieved": round(f / (t * 1e-3) / 1e12, 1), "peak": PEAK["fp16_mfma_tflops"],
                         "unit": "TFLOP/s", "frac": round(f / (t * 1e-3) / 1e12 / PEAK["fp16_mfma_tflops"], 4),
                         "avg_launch_us": round(t * 1e3, 2)}}


# algorithmic bytes per element of each bandwidth-bound kernel (inputs read + outputs written)
BYTES_PER_ELEM = {"quant": 2.0 + 0.5 + 1 / 16, "rmsq": 2.0 + 0.5 + 1 / 16, "silu": 4.0 + 3 * (0.5 + 1 / 16),
                  "silubq": 2 * (0.5 + 1 / 16) + 2.0 + 4.0 + 2 * (0.5 + 1 / 16),
                  "rmsbr": (0.5 + 1 / 16) + 2.0 + 2.0 + 2.0 + (0.5 + 1 / 16)}
BYTES_PER_ROW = {"quant": 4, "rmsq": 8, "silu": 12, "silubq": 16, "rmsbr": 12}


def gemm_bytes(M, N, segs, accumulate):
    """Algorithmic HBM bytes of one GEMM launch: every segment's NVFP4 A
    [M x K_i] and B [N x K_i] (codes, block scales, row scales), the BF16
    output, and the output read back when accumulating."""
    nv = lambda rows, cols: rows * cols * 9 // 16 + 4 * rows
    return sum(nv(M, k) + nv(N, k) for k in segs) + 2 * M * N * (2 if accumulate else 1)


def gemm_kernel_name(bm, bn, staged, segmented):
    """The kernel a launch of this group runs, as the profiler names it."""
    if staged:
        return f"pact::k_gemm_nvfp4_fast<{bm // 64}, {bn // 64}, {'true' if segmented else 'false'}>"
    return f"pact::k_gemm_nvfp4<{bm // 64}, {bn // 64}>"


def kernel_bytes(kind, rows, cols):
    return BYTES_PER_ELEM[kind] * rows * cols + BYTES_PER_ROW[kind] * rows


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "frozen_weight_gemms_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def cpu_baseline(wl, layer_bits, sample_rows):
    """Time the oracle (as it stands) on a bounded row sample of the same step's GEMMs."""
    import numpy as np
    import synth
    from oracle import gemm as ogemm
    from oracle import nvfp4 as onv

    vals = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(wl.tokens, size=sample_rows, replace=False))
    # offline weight layouts (not timed)
    wts = {}
    for i, p in enumerate(wl.projections):
        w = vals(synth.normal_bf16((p.d_out, p.d_in), wl.w_std, wl.wid, 20 + i))
        wts[p.name] = ogemm.weight_layouts(w)
    xs = {n: vals(b[rows]) for n, b in layer_bits.items()}
    t0 = time.perf_counter()
    flops = 0
    for p in wl.projections:
        wf, wb = wts[p.name]
        xq = onv.quantize(xs["x_" + p.name])
        ogemm.gemm_fwd(xq, wf)
        dyq = onv.quantize(xs["dy_" + p.name])
        ogemm.gemm_dgrad(dyq, wb)
        flops += 4 * sample_rows * p.d_in * p.d_out
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample_rows} of {wl.tokens} token rows of every projection's input and output "
                      f"gradient: oracle quantize of the rows, then its float64 fwd and dgrad GEMMs against "
                      f"the full cached weight layouts (dequantized per call); {dt:.1f} s wall, "
                      f"{flops / 1e9:.1f} GFLOP"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              f"described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import frozen_weight_gemms_amd as fw
    import synth
    from frozen_weight_gemms_amd import _lib

    wl = synth.WORKLOADS[2]
    torch.cuda.set_device(0)
    layers = [Layer(fw, torch, synth, wl, li) for li in range(max(1, args.layers))]
    layer = layers[0]
    # independent branches of the step (the q/k/v and gate/up forward
    # projections, the LoRA backwards beside the input-gradient GEMMs) go to
    # two side streams at default priority, forked from and joined back into
    # the launch stream
    side_streams = None if args.sequential else [torch.cuda.Stream(), torch.cuda.Stream()]
    for ly in layers:
        ly.streams = side_streams
    torch.cuda.synchronize()
    resident = torch.cuda.memory_allocated()

    def step():
        # forward through every layer, then backward from the top: each layer's
        # input gradient (and its NVFP4 copy) is the output gradient of the one below
        for ly in layers:
            ly.forward()
        top = layers[-1]
        top._ev("quant", "nvfp4_quantize", ("quant", top.M, top.H), lambda: fw.quantize(top.dOut, out=top.dOut_q))
        d, dq = top.dOut, top.dOut_q
        for ly in reversed(layers):
            d, dq = ly.backward(d, dq)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The step is captured once into a HIP graph (every output buffer and the
    # LoRA workspace are preallocated, so the step allocates nothing); the timed
    # region replays it.  If capture is unavailable the timed region runs the
    # step eagerly.
    graph = None
    try:
        if args.eager:
            raise RuntimeError("--eager")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    except Exception as ex:            # capture not supported: time eagerly
        if not args.eager:
            print(f"graph capture unavailable ({ex}); timing eager steps", file=sys.stderr)
        graph = None
    run = graph.replay if graph is not None else step

    # timed region: K steps, wall clock and events on the launch stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)

    # the concurrent schedule computes what the one-stream order does, bit for
    # bit (same kernels, same inputs; only their overlap differs)
    def snapshot():
        return [t.clone() for t in (layers[0].dh1, layers[0].dy1, layers[-1].proj["v"]["Y"],
                                    layers[0].proj["up"]["dB"], layers[-1].proj["k"]["dB"],
                                    layers[0].proj["q"]["dT"])]
    run()
    torch.cuda.synchronize()
    conc = snapshot()
    for ly in layers:
        ly.streams = None
    step()
    torch.cuda.synchronize()
    seq = snapshot()
    for ly in layers:
        ly.streams = side_streams
    schedule_matches = all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(conc, seq))
    if not schedule_matches:
        print("concurrent schedule differs from the one-stream order", file=sys.stderr)

    # instrumented pass over the same K steps: events around every launch give
    # per-kernel durations (events add queue overhead between kernels, so this
    # pass is not the one the step time comes from).  A spin kernel ahead of each
    # step lets the host enqueue the step's launches before the GPU reaches
    # them, so an event pair brackets the kernel and not the host's launch time.
    recs = []
    for ly in layers:
        ly.record = recs
    torch.cuda.synchronize()
    for _ in range(args.steps):
        torch.cuda._sleep(HEAD_START_CYCLES)
        step()
    torch.cuda.synchronize()
    for ly in layers:
        ly.record = None

    ms_per_step = wall * 1e3 / args.steps
    flops = sum(ly.gemm_flops() for ly in layers)
    value = flops / (ms_per_step * 1e-3) / 1e12

    # per-kernel times from the events
    cat_ms, gemm_by_tile, bw = {}, {}, {}
    for cat, name, e0, e1, work in recs:
        t = e0.elapsed_time(e1)
        cat_ms[cat] = cat_ms.get(cat, 0.0) + t
        if cat == "gemm":
            _, M, N, segs, acc = work
            K = sum(segs)
            # kernel group: (bm, bn, stage-pipelined path, segmented)
            seg = len(segs) > 1
            tile = (_lib.gemm_multi_tile(M, N) if seg else _lib.gemm_tile(M, N, K)) + \
                (all(k % 256 == 0 for k in segs), seg)
            g = gemm_by_tile.setdefault(tile, [0.0, 0.0, 0, 0.0])
            g[0] += t
            g[1] += 2.0 * M * N * K
            g[2] += 1
            g[3] += gemm_bytes(M, N, segs, acc)
        elif work is not None:
            kind, rows, cols = work
            b = bw.setdefault(name, [0.0, 0.0, 0])
            b[0] += t
            b[1] += kernel_bytes(kind, rows, cols)
            b[2] += 1
    steps = args.steps
    gemm_ms = cat_ms.get("gemm", 0.0) / steps
    dom_tile = max(gemm_by_tile, key=lambda k: gemm_by_tile[k][0])
    dt_ms, dflops, dcount, dbytes = gemm_by_tile[dom_tile]
    achieved = dflops / (dt_ms * 1e-3) / 1e12
    kname = gemm_kernel_name(*dom_tile)

    # every GEMM kernel of the step: launches, time and algorithmic bytes
    gemm_kernels = {gemm_kernel_name(*k): {"launches_per_step": g[2] // steps,
                                           "avg_launch_us": round(g[0] * 1e3 / g[2], 2),
                                           "tflops": round(g[1] / (g[0] * 1e-3) / 1e12, 1),
                                           "algorithmic_bytes_per_launch": round(g[3] / g[2])}
                    for k, g in sorted(gemm_by_tile.items(), key=lambda kv: -kv[1][0])}

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            if tj.get("src_hash") == src_hash("gemm.hip", "nvfp4_device.h", "lds_dma.h", "mfma_fp16.h"):
                traffic = tj.get("kernels", {}).get(kname, {}).get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None

    quant = {n: {"GB/s": round(b[1] / (b[0] * 1e-3) / 1e9, 1), "frac_hbm": round(b[1] / (b[0] * 1e-3) / 8e12, 3),
                 "us_per_launch": round(b[0] * 1e3 / b[2], 2)} for n, b in bw.items()}

    result = {
        "metric": "NVFP4 fwd+dgrad GEMM TFLOP/s at Llama-3B shapes; % FP4 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, fp16 MFMA (exact products), fp32 accumulation, bf16 output",
        "data": "synthetic (seeded BF16 activations with 1% outlier channels, N(0,0.02) weights, N(0,0.01) grads)",
        "config": {"workload": f"llama3b decoder-layer frozen projections fwd+dgrad + fused quantizers + LoRA r16, "
                               f"{len(layers)} distinct layer instances per step, backward chained through "
                               f"BF16 residual gradients",
                   "layers": len(layers), "resident_gb": round(resident / 1e9, 2),
                   "tokens": layer.M, "hidden": layer.H, "intermediate": layer.I, "kv": layer.KV,
                   "lora_rank": layer.r, "gemm_gflop_per_step": round(flops / 1e9, 1), "parallelism": "single-gpu"},
        "frac_fp4_peak": round(value / PEAK["fp4_mfma_tflops"], 4),
        "frac_fp16_peak": round(value / PEAK["fp16_mfma_tflops"], 4),
        "gemm_only_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gpu_ms_per_step_events": round(gpu_ms / steps, 4),
        "timed_region": "hip graph replays of the step" if graph is not None else "eager steps",
        "schedule": ("one stream" if side_streams is None else
                     "independent branches on 2 side streams (q/k/v and gate/up forward, their LoRA "
                     "backwards); one input-gradient launch each for q/k/v and gate/up"),
        "schedule_matches_one_stream": schedule_matches,
        "kernel_ms_per_step_by_category": {k: round(v / steps, 4) for k, v in sorted(cat_ms.items())},
        "bandwidth_kernels": quant,
        "gemm_kernels": gemm_kernels,
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK["fp16_mfma_tflops"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK["fp16_mfma_tflops"], 4),
                     "frac_of_fp4_peak": round(achieved / PEAK["fp4_mfma_tflops"], 4),
                     "launches_per_step": dcount // steps,
                     "avg_launch_us": round(dt_ms * 1e3 / dcount, 2),
                     "algorithmic_bytes_per_launch": round(dbytes / dcount),
                     "traffic": traffic},
    }
    if not args.no_recipes:
        result["recipe_variants"] = recipe_leg(fw, torch, synth, wl)
        result["single_layout_dgrad"] = single_layout_leg(fw, torch, synth, wl)
        result["quantizer_bandwidth"] = quantizer_leg(fw, torch)
        result["lora_term"] = lora_term_leg(fw, torch, synth, wl)
    if not args.no_mxfp4:
        del graph
        result["mxfp4_variant"] = mxfp4_leg(fw, torch, synth, wl, max(1, args.layers), args.steps, args.warmup,
                                            eager=args.eager)
    # measured MFMA-loop peak beside the published dense peaks (no memory traffic in the loop)
    p16, c16 = fw.mfma_probe(0)
    p4, c4 = fw.mfma_probe(1)
    result["mfma_loop_peak"] = {"fp16_tflops": round(p16, 1), "fp16_clock_ghz": round(c16, 3),
                                "fp4_tflops": round(p4, 1), "fp4_clock_ghz": round(c4, 3),
                                "probe": "pact_mfma_probe: 512 workgroups x 4 waves, 16 independent MFMA chains "
                                         "per wave, 4000 iterations; clock from s_memtime / s_memrealtime"}
    result["roofline"]["measured_peak"] = round(p16, 1)
    result["roofline"]["frac_of_measured_peak"] = round(result["roofline"]["achieved"] / p16, 4)
    if "mxfp4_variant" in result and "roofline" in result["mxfp4_variant"]:
        mr = result["mxfp4_variant"]["roofline"]
        mr["measured_peak"] = round(p4, 1)
        mr["frac_of_measured_peak"] = round(mr["achieved"] / p4, 4)
    result["device"] = {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                        "torch": torch.__version__}
    if args.copy_calibration:
        x = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        rows_bits = {}
        H, KV, I = layer.H, layer.KV, layer.I
        for name, cols, tid in (("x_q", H, 10), ("x_k", H, 10), ("x_v", H, 10), ("x_o", H, 12),
                                ("x_gate", H, 11), ("x_up", H, 11)):
            rows_bits[name] = synth.workload_activation(wl, wl.tokens, cols, tid)
        # the down projection's input in the step is silu(gate) * up; a fresh activation of that shape
        rows_bits["x_down"] = synth.workload_activation(wl, wl.tokens, I, 99)
        for name, cols, tid in (("dy_down", H, 15), ("dy_o", H, 16), ("dy_q", H, 17), ("dy_k", KV, 18),
                                ("dy_v", KV, 19), ("dy_gate", I, 98), ("dy_up", I, 97)):
            rows_bits[name] = synth.normal_bf16((wl.tokens, cols), wl.dy_std, wl.wid, tid)
        result["cpu_baseline"] = cpu_baseline(wl, rows_bits, args.cpu_sample_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
