#!/usr/bin/env python3
"""Benchmark of the NVFP4 frozen-projection hot path on one MI355X.

One step is one pass of the whole path over --layers (default 4) distinct
Llama-3B-shaped decoder layers' frozen projections at M = 4096 tokens
(batch 4 x seq 1024), LoRA rank 16 -- distinct weights and buffers per layer,
about 1 GB each, so operands stream from HBM rather than the 256 MB
last-level cache.  Forward through every layer, then backward from the top
layer down, each layer's input gradient (the residual stream) being the
output gradient of the layer below:

  forward   rmsnorm_quant -> q/k/v (one lora_down over the stacked adapters,
            one NVFP4 GEMM over the stacked weights, LoRA term fused)
            nvfp4_quantize(attention output) -> o
            rmsnorm_quant -> gate/up (stacked, as q/k/v) -> silu_mul_quant -> down
  backward  down (its dY = the layer's output gradient, already NVFP4)
            silu_mul_bwd_quant (BF16 da, db and their NVFP4 copies) -> gate, up
            rmsnorm_bwd_residual (+ the output gradient; NVFP4 copy) -> o
            q/k/v (nvfp4_quantize of the attention-backward gradients)
            rmsnorm_bwd_residual (+ the MLP-block residual gradient; NVFP4 copy)
  per projection: lora_bwd_dt (dT); per input: one NVFP4 dgrad launch with
  the LoRA input-gradient terms (q/k/v and gate/up each sum into one dX in a
  single nvfp4_gemm_dgrad_multi launch; down and o alone); per layer two
  lora_bwd_ab_batch calls (dA and dB of down/gate/up, then of o/q/k/v), each
  after T = X_q A^T is recomputed from the saved NVFP4 input (one stacked
  lora_down per input)

The metric is the NVFP4 fwd + dgrad GEMM throughput of the step:
  value = (GEMM FLOPs per step) / (median time per step)   [TFLOP/s]
with every other kernel of the step inside the timed region.  Inputs are
synthetic (seeded, BF16, drawn on the device, resident in HBM before timing);
weights are random N(0, 0.02) quantized once to their two cached NVFP4
layouts, one per direction (offline, untimed); LoRA B ~ N(0, 0.01) so that
every adapter gradient is nonzero.

Timing: --warmup untimed steps, then exactly --steps HIP-graph replays of the
step, each bracketed by an event pair on the launch stream, the whole run by
device synchronizations and the wall clock; median, minimum and mean per step
are reported, the headline from the median.

Measured beside it (each under its own key, none part of "value"):
  parity            the oracle recomputes, stage by stage from the device's own
                    inputs to each stage, sampled rows of the timed step's
                    outputs (and adapter gradients over all tokens); codes bit
                    for bit, GEMMs within one BF16 ulp + 1e-5 sum |a b|.  Its
                    timing is "cpu_baseline".
  configs           the same step at the other workloads: Llama-1B projections
                    (M 4096), the Llama-3B MLP block (M 8192) and the 8B-scale
                    projections (M 16384, Student-t activations, LoRA r 64),
                    each with its own roofline, parity and oracle timing.
  hbm_copy          a plain device copy: 1 GiB read + 1 GiB write, and at the
                    byte counts of every bandwidth-bound kernel of the step.
  mxfp4_variant, recipe_variants, single_layout_dgrad, quantizer_bandwidth,
  lora_term, mfma_loop_peak   (see their functions).

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
HEAD_START_CYCLES = 40_000_000      # spin ahead of a timed launch sequence (about 20 ms)
QKV_GRAD_QUANT = "branches"              # how the step quantizes dq, dk, dv (--qkv-grad-quant)
STEP_HEAD_START_CYCLES = 200_000_000  # spin ahead of each instrumented step (about 100 ms)
METRIC = "NVFP4 fwd+dgrad GEMM TFLOP/s at Llama-3B shapes; % FP4 MFMA peak"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (its timing on host cores and the parity of the timed outputs)")
    ap.add_argument("--cpu-sample-rows", type=int, default=1536,
                    help="token rows the oracle recomputes per stage for the headline step (about 10 s of oracle time)")
    ap.add_argument("--config-sample-rows", type=int, default=24,
                    help="token rows the oracle recomputes per stage for the other configurations")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--sequential", action="store_true",
                    help="one stream: no concurrent branches (the LoRA backwards beside each other)")
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct decoder-layer instances a step runs through (their weights and buffers "
                         "together exceed the 256 MB last-level cache, so every operand streams from HBM)")
    ap.add_argument("--no-configs", action="store_true", help="skip the Llama-1B, MLP-block and 8B-scale legs")
    ap.add_argument("--no-mxfp4", action="store_true", help="skip the MXFP4-variant leg")
    ap.add_argument("--no-recipes", action="store_true",
                    help="skip the recipe, single-layout, quantizer-bandwidth, LoRA-term and copy legs")
    ap.add_argument("--step-only", action="store_true",
                    help="only the headline step (for profiler runs: every kernel launched is one of the step's)")
    ap.add_argument("--instr-steps", type=int, default=10, help="steps of the per-kernel event pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB read + 1 GiB write copy (counter calibration)")
    ap.add_argument("--qkv-grad-quant", choices=("branches", "batched"), default="branches",
                    help="attention gradients dq, dk, dv: quantized in each projection's branch beside its dT, "
                         "or in one nvfp4_quantize_batch launch before the branches")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# one decoder layer's frozen-projection path
# ---------------------------------------------------------------------------
class Layer:
    """Device state of one synthetic decoder layer (or, with mlp_only, one MLP
    block) of the workload: the projections' cached NVFP4 layouts, LoRA
    adapters, inputs and every intermediate buffer, preallocated."""

    def __init__(self, fw, torch, synth, wl, index=0, mlp_only=False, shared_t=None):
        self.fw, self.torch, self.wl = fw, torch, wl
        self.mlp_only = mlp_only
        P = {p.name: p for p in wl.projections}
        M, r = wl.tokens, wl.lora_rank
        H, I = P["gate"].d_in, P["gate"].d_out
        KV = None if mlp_only else P["k"].d_out
        self.M, self.H, self.I, self.KV, self.r = M, H, I, KV, r
        dev = torch.device("cuda:0")
        off, wid = 1000 * index, wl.wid
        act = lambda tid, cols: synth.activation_torch(wl, M, cols, off + tid)
        grad = lambda tid, cols: synth.normal_torch((M, cols), wl.dy_std, wid, off + tid)
        gain = lambda tid: synth.uniform_torch((H,), 0.9, 1.1, wid, off + tid)
        nv = lambda cols: fw.empty_nvfp4(M, cols, dev)
        bf = lambda cols: torch.empty((M, cols), dtype=torch.bfloat16, device=dev)
        self.h2, self.g2 = act(11, H), gain(14)
        self.dOut, self.dOut_q = grad(15, H), nv(H)          # output gradient entering the stack (top layer)
        if not mlp_only:
            self.h1, self.attn, self.g1 = act(10, H), act(12, H), gain(13)
            self.dq, self.dk, self.dv = grad(17, H), grad(18, KV), grad(19, KV)

        self.proj = {}
        self.w_check = None
        for i, p in enumerate(wl.projections):
            w = synth.normal_torch((p.d_out, p.d_in), wl.w_std, wid, off + 20 + i)
            wf, wb = fw.weight_layouts(w)
            if index == 0 and p.name == ("gate" if mlp_only else "k"):
                self.w_check = (p.name, w)           # BF16 W kept for the layout parity check
            del w                                    # only the cached NVFP4 layouts stay resident
            A = synth.normal_torch((r, p.d_in), wl.a_std, wid, off + 40 + i)
            B = synth.normal_torch((p.d_out, r), wl.a_std, wid, off + 60 + i)
            ws = torch.empty((fw._lib.lora_bwd_workspace_size(M, p.d_in, p.d_out, r),), dtype=torch.uint8,
                             device=dev)
            # q, k and v quantize their own dY (the others read NVFP4 copies made by fused kernels)
            self.proj[p.name] = dict(p=p, wf=wf, wb=wb, A=A, B=B, ws=ws,
                                     dyq=nv(p.d_out) if p.name in ("q", "k", "v") else None,
                                     dT=torch.empty((M, r), dtype=torch.bfloat16, device=dev),
                                     dA=torch.empty((r, p.d_in), dtype=torch.bfloat16, device=dev),
                                     dB=torch.empty((p.d_out, r), dtype=torch.bfloat16, device=dev))
        # the attention gradients' NVFP4 copies in one launch (when the step batches them)
        self.qkv_quant = None if mlp_only else fw.QuantizeBatch(
            [self.dq, self.dk, self.dv], [self.proj[n]["dyq"] for n in ("q", "k", "v")])
        # forward groups: the projections that read one input run as one GEMM over
        # their stacked weights (rows of Q(W) are independent, so the stacked
        # layout is the row concatenation of the separate ones) with one
        # lora_down over the stacked adapters and a block-diagonal B
        groups = [("gu", ("gate", "up")), ("down", ("down",))]
        if not mlp_only:
            groups = [("qkv", ("q", "k", "v")), ("o", ("o",))] + groups
        # (a group is stacked while its stacked LoRA rank fits the GEMM's limit
        # of 128; otherwise its projections run as separate GEMMs)
        split = [(n, (n,)) for g, names in groups if len(names) * r > 128 for n in names]
        groups = [(g, names) for g, names in groups if len(names) * r <= 128] + split
        self.fwd_order = [g for g, _ in groups]
        self.grp = {}
        for g, names in groups:
            Ps = [self.proj[n] for n in names]
            K = Ps[0]["p"].d_in
            if len(names) == 1:
                wf, A, B = Ps[0]["wf"], Ps[0]["A"], Ps[0]["B"]
            else:
                wf = fw.NVFP4Tensor(torch.cat([q["wf"].codes for q in Ps]), torch.cat([q["wf"].scales for q in Ps]),
                                    torch.cat([q["wf"].rscale for q in Ps]))
                A = torch.cat([q["A"] for q in Ps]).contiguous()
                B = torch.zeros((sum(q["p"].d_out for q in Ps), r * len(Ps)), dtype=torch.bfloat16, device=dev)
            nout = wf.rows
            T = torch.empty((M, A.shape[0]), dtype=torch.bfloat16, device=dev)
            # the backward recomputes T from X_q into a transient buffer, one per
            # group shared by every layer (T is not state kept for the backward)
            shared_t = {} if shared_t is None else shared_t
            if g not in shared_t:
                shared_t[g] = torch.empty((M, A.shape[0]), dtype=torch.bfloat16, device=dev)
            Tb = shared_t[g]
            Y = torch.empty((M, nout), dtype=torch.bfloat16, device=dev)
            n0 = 0
            for j, q in enumerate(Ps):
                n = q["p"].d_out
                if len(names) > 1:
                    B[n0:n0 + n, j * r:(j + 1) * r] = q["B"]
                    q["A"] = A[j * r:(j + 1) * r]                    # contiguous row block of the stacked A
                    q["wf"] = fw.NVFP4Tensor(wf.codes[n0:n0 + n], wf.scales[n0:n0 + n], wf.rscale[n0:n0 + n])
                q["Y"], q["T"], q["Tb"] = Y[:, n0:n0 + n], T[:, j * r:(j + 1) * r], Tb[:, j * r:(j + 1) * r]
                n0 += n
            self.grp[g] = dict(names=names, wf=wf, A=A, B=B, T=T, Tb=Tb, Y=Y, K=K, xq=None,
                               launches=self._launch_split(M, K, [q["p"].d_out for q in Ps]))

        self.y2q, self.rstd2 = nv(H), torch.empty((M,), dtype=torch.float32, device=dev)
        self.hq, self.gq, self.uq = nv(I), nv(I), nv(I)
        self.dh, self.da, self.db = bf(I), bf(I), bf(I)
        self.daq, self.dbq = nv(I), nv(I)
        self.dy2, self.dh2, self.dh2q = bf(H), bf(H), nv(H)
        if not mlp_only:
            self.y1q, self.aq = nv(H), nv(H)
            self.rstd1 = torch.empty((M,), dtype=torch.float32, device=dev)
            self.dy1, self.dattn, self.dh1, self.dh1q = bf(H), bf(H), bf(H), nv(H)
        self.proj["gate"]["dyq"], self.proj["up"]["dyq"] = self.daq, self.dbq
        self.record = None       # list to append (category, name, start_event, end_event, work) into
        self.streams = None      # side streams: independent branches of the step run concurrently
        self.ab_jobs = []        # adapter-gradient problems of the backward so far
        self.ab_plan = {}        # batch tag -> (buffer addresses, LoraAbBatch, work)
        self.pending = None      # list (shared by the layers) of side-stream work the next GEMM waits for
        self.dout = None         # the output gradient this layer received in the last step

    @staticmethod
    def _launch_split(M, K, widths):
        """Row ranges of a group's stacked weight, one forward GEMM launch
        each: the whole stack, or its first projection and the rest, whichever
        needs fewer tile rounds on 256 CUs (tile area times rounds).  Either
        way every output element is the same sum in the same order (the LoRA
        term of a part is the stacked one with the other parts' zero B blocks)."""
        from frozen_weight_gemms_amd import _lib

        def cost(n):
            bm, bn = _lib.gemm_tile(M, n, K)
            tiles = -(-M // bm) * -(-n // bn)
            return -(-tiles // 256) * bm * bn
        total = sum(widths)
        if len(widths) > 1 and cost(widths[0]) + cost(total - widths[0]) < cost(total):
            return [(0, widths[0]), (widths[0], total)]
        return [(0, total)]

    # ---- instrumented launch helper ----
    def _ev(self, cat, name, work, fn):
        if self.record is None:
            return fn()
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        out = fn()
        e1.record()
        self.record.append((cat, name, e0, e1, work, fn))
        return out

    def _fwd_group(self, g, xq):
        fw, G = self.fw, self.grp[g]
        M, K = self.M, G["K"]
        G["xq"] = xq
        self._ev("lora", "lora_down", ("lora_down", M, K, G["A"].shape[0]),
                 lambda: fw.lora_down(xq, G["A"], out=G["T"]))
        wf = G["wf"]
        for a, b in G["launches"]:
            part = wf if (a, b) == (0, wf.rows) else fw.NVFP4Tensor(wf.codes[a:b], wf.scales[a:b], wf.rscale[a:b])
            self._ev("gemm", f"fwd {g}", ("gemm", M, b - a, (K,), False),
                     lambda part=part, a=a, b=b: fw.gemm_fwd(xq, part, lora_t=G["T"], lora_b=G["B"][a:b],
                                                             lora_scale=LORA_SCALE, out=G["Y"][:, a:b]))

    def _bwd_lora(self, name, xq, dy, dyq=None):
        """dY's NVFP4 copy (unless a fused kernel made it) and the LoRA
        backward of one projection."""
        fw, P = self.fw, self.proj[name]
        p = P["p"]
        if dyq is None:
            self._ev("quant", "nvfp4_quantize", ("quant", self.M, p.d_out), lambda: fw.quantize(dy, out=P["dyq"]))
        P["dyq_used"] = dyq if dyq is not None else P["dyq"]     # the NVFP4 dY its input gradient reads
        # dT, which the input-gradient GEMM's LoRA term needs, now; dA and dB
        # (read by nothing else in the step) for every projection of the layer
        # in one batched call at the end of its backward, from the T that the
        # forward's lora_down left (X_q A^T is not recomputed).  (On a stream of
        # their own, beside the GEMMs, the adapter gradients measured slower:
        # they take CUs from the GEMM's one-workgroup-per-CU tiles.)
        self._ev("lora", "lora_bwd_dt", ("lora_bwd_dt", self.M, p.d_out, self.r),
                 lambda: fw.lora_bwd_dt(dy, P["B"], LORA_SCALE, out=P["dT"]))
        self.ab_jobs.append((xq, P["Tb"], dy, P["dT"], (P["dA"], P["dB"]), P["ws"]))

    def _side(self, fn):
        """fn on the side stream of the adapter-gradient work (after the
        current stream's work so far), recorded for the next join; in place
        without side streams or while the step is instrumented."""
        if self.streams is None or self.record is not None or self.pending is None:
            fn()
            return
        torch = self.torch
        cur, st = torch.cuda.current_stream(), self.streams[-1]
        st.wait_stream(cur)
        with torch.cuda.stream(st):
            fn()
        ev = torch.cuda.Event()
        ev.record(st)
        self.pending.append(ev)

    def _recompute_t(self, names):
        """T = X~ A^T of these projections' groups, recomputed from the saved
        NVFP4 input (one stacked lora_down per input) into the transient
        buffers: the LoRA branch keeps only the shared NVFP4 input and its
        adapters for the backward."""
        fw = self.fw
        groups = [G for G in self.grp.values() if set(G["names"]) <= set(names)]

        def run():
            for G in groups:
                self._ev("lora", "lora_down", ("lora_down", self.M, G["K"], G["A"].shape[0]),
                         lambda G=G: fw.lora_down(G["xq"], G["A"], out=G["Tb"]))
        self._side(run)

    def _adapter_grads(self, tag):
        """dA and dB of the projections whose dT is done (one batched call,
        from the recomputed T).  Nothing later in the step reads them, so with
        side streams this runs on a stream of its own beside the next non-GEMM
        kernels, and the next input-gradient GEMM waits for it (GEMM tiles fill
        every CU, so work running beside one would delay its tiles)."""
        jobs, self.ab_jobs = self.ab_jobs, []
        # the batch's argument arrays are built once: every step passes the
        # same buffers (checked by their addresses)
        key = tuple(t.data_ptr() for j in jobs for t in (j[0].codes, j[1], j[2], j[3], j[4][0], j[4][1], j[5]))
        if tag not in self.ab_plan or self.ab_plan[tag][0] != key:
            work = ("lora_ab_batch", tuple((self.M, j[0].cols, j[2].shape[1], j[1].shape[1]) for j in jobs))
            self.ab_plan[tag] = (key, self.fw.LoraAbBatch(jobs, LORA_SCALE), work)
        _, plan, work = self.ab_plan[tag]
        self._side(lambda: self._ev("lora", "lora_bwd_ab_batch", work, plan.run))

    def join(self):
        """The current stream waits for the side-stream work started so far."""
        if self.pending:
            cur = self.torch.cuda.current_stream()
            for ev in self.pending:
                cur.wait_event(ev)
            self.pending.clear()

    def _bwd_dgrad(self, name, dyq, dx):
        fw, P = self.fw, self.proj[name]
        p = P["p"]
        self.join()
        self._ev("gemm", f"dgrad {name}", ("gemm", self.M, p.d_in, (p.d_out,), False),
                 lambda: fw.gemm_dgrad(dyq, P["wb"], out=dx, lora_dt=P["dT"], lora_a=P["A"]))

    def _bwd_dgrad_multi(self, names, dx):
        """One input-gradient launch summing the projections that read one
        input (each with its LoRA term dT A)."""
        fw = self.fw
        Ps = [self.proj[n] for n in names]
        self.join()
        work = ("gemm", self.M, Ps[0]["p"].d_in, tuple(P["p"].d_out for P in Ps), False)
        self._ev("gemm", "dgrad " + "/".join(names), work,
                 lambda: fw.gemm_dgrad_multi([(P["dyq"], P["wb"]) for P in Ps], out=dx,
                                             lora=[(P["dT"], P["A"]) for P in Ps]))

    def _branches(self, fns):
        """fns[0] on the current stream, fns[1:] concurrently on side streams
        (each after the current stream's work so far); the current stream then
        waits for all of them.  Without side streams (or while the step is
        instrumented) the branches run in place, in order."""
        if self.streams is None or self.record is not None:
            for f in fns:
                f()
            return
        torch = self.torch
        cur = torch.cuda.current_stream()
        side = self.streams[:len(fns) - 1]
        for st, f in zip(side, fns[1:]):
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                f()
        fns[0]()
        for st in side:
            cur.wait_stream(st)

    def forward(self):
        fw = self.fw
        M, H, I = self.M, self.H, self.I
        if not self.mlp_only:
            self._ev("quant", "rmsnorm_quant", ("rmsq", M, H),
                     lambda: fw.rmsnorm_quant(self.h1, self.g1, 1e-5, out=(self.y1q, self.rstd1)))
            for g in (("qkv",) if "qkv" in self.grp else ("q", "k", "v")):
                self._fwd_group(g, self.y1q)
            self._ev("quant", "nvfp4_quantize", ("quant", M, H), lambda: fw.quantize(self.attn, out=self.aq))
            self._fwd_group("o", self.aq)
        self._ev("quant", "rmsnorm_quant", ("rmsq", M, H),
                 lambda: fw.rmsnorm_quant(self.h2, self.g2, 1e-5, out=(self.y2q, self.rstd2)))
        for g in (("gu",) if "gu" in self.grp else ("gate", "up")):
            self._fwd_group(g, self.y2q)
        a, b = self.proj["gate"]["Y"], self.proj["up"]["Y"]
        self._ev("quant", "silu_mul_quant", ("silu", M, I),
                 lambda: fw.silu_mul_quant(a, b, out=(self.hq, self.gq, self.uq)))
        self._fwd_group("down", self.hq)

    def backward(self, dout, dout_q):
        """Backward of the layer given the gradient of its output (BF16 and its
        NVFP4 copy); returns the gradient of its input, the residual stream
        (Table 7 row "Residuals": the residual gradients are summed in BF16)."""
        fw = self.fw
        M, H, I = self.M, self.H, self.I
        self.dout = (dout, dout_q)
        # MLP block: out = h2 + down(silu(gate(n2)) * up(n2)),  n2 = rmsnorm(h2)
        self._bwd_lora("down", self.hq, dout, dout_q)
        self._bwd_dgrad("down", dout_q, self.dh)
        # T of the MLP projections, beside silu_mul_bwd_quant and the gate/up dT
        # (recomputing every projection's T there measured slower: it slows
        # silu_mul_bwd_quant more than the later stretches gain)
        self._recompute_t(("gate", "up", "down"))
        self._ev("bwd", "silu_mul_bwd_quant", ("silubq", M, I),
                 lambda: fw.silu_mul_bwd_quant(self.gq, self.uq, self.dh, out=(self.da, self.db, self.daq, self.dbq)))
        # the gate and up LoRA backwards run side by side; one input-gradient
        # launch sums both projections into dX
        self._branches([lambda: self._bwd_lora("gate", self.y2q, self.da, self.daq),
                        lambda: self._bwd_lora("up", self.y2q, self.db, self.dbq)])
        self._bwd_dgrad_multi(("gate", "up"), self.dy2)
        self._adapter_grads("mlp")
        self._ev("bwd", "rmsnorm_bwd_residual", ("rmsbr", M, H),
                 lambda: fw.rmsnorm_bwd_residual(self.y2q, self.rstd2, self.g2, self.dy2, resid=dout,
                                                 out=(self.dh2, self.dh2q)))
        if self.mlp_only:
            return self.dh2, self.dh2q
        # attention block: h2 = h1 + o(attn(q, k, v of n1)),  n1 = rmsnorm(h1); the
        # attention backward itself is not part of the path (dq, dk, dv are inputs)
        self._bwd_lora("o", self.aq, self.dh2, self.dh2q)
        self._bwd_dgrad("o", self.dh2q, self.dattn)
        # T of the attention projections, beside the q/k/v quantizations and dT
        self._recompute_t(("q", "k", "v", "o"))
        if QKV_GRAD_QUANT == "batched":
            self._ev("quant", "nvfp4_quantize_batch", ("quant", self.M, self.H + 2 * self.KV, 3), self.qkv_quant.run)
            self._branches([lambda n=n, d=d: self._bwd_lora(n, self.y1q, d, self.proj[n]["dyq"])
                            for n, d in (("q", self.dq), ("k", self.dk), ("v", self.dv))])
        else:
            self._branches([lambda n=n, d=d: self._bwd_lora(n, self.y1q, d)
                            for n, d in (("q", self.dq), ("k", self.dk), ("v", self.dv))])
        self._bwd_dgrad_multi(("q", "k", "v"), self.dy1)
        self._adapter_grads("attn")
        self._ev("bwd", "rmsnorm_bwd_residual", ("rmsbr", M, H),
                 lambda: fw.rmsnorm_bwd_residual(self.y1q, self.rstd1, self.g1, self.dy1, resid=self.dh2,
                                                 out=(self.dh1, self.dh1q)))
        return self.dh1, self.dh1q

    def gemm_flops(self):
        return sum(4 * self.M * P["p"].d_in * P["p"].d_out for P in self.proj.values())


# ---------------------------------------------------------------------------
# algorithmic bytes of the bandwidth-bound kernels (inputs read + outputs written)
# ---------------------------------------------------------------------------
NV_B = 0.5 + 1 / 16                     # NVFP4 bytes per element (codes + block scales)
BYTES_PER_ELEM = {"quant": 2.0 + NV_B, "rmsq": 2.0 + NV_B, "silu": 4.0 + 3 * NV_B,
                  "silubq": 2 * NV_B + 2.0 + 4.0 + 2 * NV_B,
                  "rmsbr": NV_B + 2.0 + 2.0 + 2.0 + NV_B}
BYTES_PER_ROW = {"quant": 4, "rmsq": 8, "silu": 12, "silubq": 16, "rmsbr": 12}


def kernel_bytes(work):
    """Algorithmic bytes of one launch described by its work tuple."""
    kind = work[0]
    if kind == "lora_down":                  # X_q read once, A read, T written
        _, M, K, r = work
        return NV_B * M * K + 4 * M + 2 * r * K + 2 * M * r
    if kind == "lora_bwd":                   # X_q and dY read once, A, B read; dT, dA, dB written
        _, M, K, N, r = work
        return NV_B * M * K + 4 * M + 2 * M * N + 2 * r * K + 2 * N * r + 2 * M * r + 2 * r * K + 2 * N * r
    if kind == "lora_bwd_dt":                # dY and B read, dT written
        _, M, N, r = work
        return 2 * M * N + 2 * N * r + 2 * M * r
    if kind == "lora_ab_batch":              # per projection: X_q, T, dY, dT read once; dA, dB written
        return sum(NV_B * M * K + 4 * M + 2 * M * N + 4 * M * r + 2 * r * K + 2 * N * r
                   for M, K, N, r in work[1])
    _, rows, cols, *tensors = work           # a batched launch: the row bytes of each of its tensors
    return BYTES_PER_ELEM[kind] * rows * cols + BYTES_PER_ROW[kind] * rows * (tensors[0] if tensors else 1)


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


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "frozen_weight_gemms_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def stats(ms):
    s = sorted(ms)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"median": med, "min": s[0], "mean": sum(s) / n, "max": s[-1]}


# ---------------------------------------------------------------------------
# one workload: build, time, instrument, check
# ---------------------------------------------------------------------------
def run_config(fw, torch, synth, wl, nlayers, steps, warmup, instr_steps, args, mlp_only=False, check=True,
               sample_rows=None):
    from frozen_weight_gemms_amd import _lib
    shared_t = {}                # transient T of the backward's recomputation, one buffer per group
    layers = [Layer(fw, torch, synth, wl, li, mlp_only=mlp_only, shared_t=shared_t) for li in range(max(1, nlayers))]
    side_streams = None if args.sequential else [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()]
    pending = []                 # side-stream work of one layer that a later GEMM (maybe the next layer's) waits for
    for ly in layers:
        ly.streams = side_streams
        ly.pending = pending
    torch.cuda.synchronize()
    top = layers[-1]

    def step():
        # forward through every layer, then backward from the top: each layer's
        # input gradient (and its NVFP4 copy) is the output gradient of the one below
        for ly in layers:
            ly.forward()
        top._ev("quant", "nvfp4_quantize", ("quant", top.M, top.H), lambda: fw.quantize(top.dOut, out=top.dOut_q))
        d, dq = top.dOut, top.dOut_q
        for ly in reversed(layers):
            d, dq = ly.backward(d, dq)
        top.join()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the step is captured once into a HIP graph (every buffer is preallocated,
    # so the step allocates nothing); the timed region replays it
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

    # timed region: exactly `steps` steps, each bracketed by an event pair on
    # the launch stream, the whole bracketed by device synchronizations
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = stats([e0.elapsed_time(e1) for e0, e1 in evs])

    # the concurrent schedule computes what the one-stream order does, bit for
    # bit (same kernels, same inputs; only their overlap differs)
    def snapshot():
        ts = [layers[0].dh2, layers[0].dy2, layers[-1].proj["up"]["dB"], layers[0].proj["gate"]["dA"],
              layers[-1].proj["down"]["Y"], layers[0].proj["down"]["dB"]]
        if not mlp_only:
            ts += [layers[0].dh1, layers[0].dy1, layers[-1].proj["k"]["dB"], layers[0].proj["q"]["dT"],
                   layers[0].proj["o"]["dA"], layers[-1].proj["v"]["dA"]]
        return [t.clone() for t in ts]
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
        print(f"{wl.name}: concurrent schedule differs from the one-stream order", file=sys.stderr)
    del conc, seq

    # instrumented pass: events around every launch give per-kernel durations
    # (events add queue overhead between kernels, so this pass is not the one
    # the step time comes from).  A spin kernel ahead of each step lets the
    # host enqueue the step's launches before the GPU reaches them, so an event
    # pair brackets the kernel and not the host's launch time.
    # The pass checks that the host finished enqueueing each step before the
    # spin ended (else the GPU waited for launches inside the event pairs).
    recs = []
    for ly in layers:
        ly.record = recs
    torch.cuda.synchronize()
    head_start_ok = True
    for _ in range(instr_steps):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        torch.cuda._sleep(STEP_HEAD_START_CYCLES)
        s1.record()
        h0 = time.perf_counter()
        step()
        host_ms = (time.perf_counter() - h0) * 1e3
        torch.cuda.synchronize()
        head_start_ok = head_start_ok and host_ms < s0.elapsed_time(s1)
    for ly in layers:
        ly.record = None
    if not head_start_ok:
        print(f"{wl.name}: the instrumented pass's head start was shorter than the host's enqueue time",
              file=sys.stderr)

    flops = sum(ly.gemm_flops() for ly in layers)
    ms = st["median"]
    value = flops / (ms * 1e-3) / 1e12
    cat_ms, gemm_by_tile, bw, group_fns = {}, {}, {}, {}
    for cat, name, e0, e1, work, fn in recs:
        t = e0.elapsed_time(e1)
        cat_ms[cat] = cat_ms.get(cat, 0.0) + t
        if cat == "gemm":
            _, M, N, segs, acc = work
            K = sum(segs)
            seg = len(segs) > 1
            tile = (_lib.gemm_multi_tile(M, N) if seg else _lib.gemm_tile(M, N, K)) + \
                (all(k % 256 == 0 for k in segs), seg)
            g = gemm_by_tile.setdefault(tile, [0.0, 0.0, 0, 0.0])
            g[0] += t
            g[1] += 2.0 * M * N * K
            g[2] += 1
            g[3] += gemm_bytes(M, N, segs, acc)
            group_fns.setdefault(tile, []).append((fn, 2.0 * M * N * K))
        else:
            b = bw.setdefault(name, [0.0, 0.0, 0])
            b[0] += t
            b[1] += kernel_bytes(work)
            b[2] += 1
    gemm_ms = cat_ms.get("gemm", 0.0) / instr_steps
    dom_tile = max(gemm_by_tile, key=lambda k: gemm_by_tile[k][0])
    dt_ms, dflops, dcount, dbytes = gemm_by_tile[dom_tile]
    kname = gemm_kernel_name(*dom_tile)
    # The dominant kernel's rate: one step's launches of it (the same calls on
    # the same buffers; every launch rewrites its output with the same values)
    # replayed back to back, as they run inside the graph, with one event pair
    # around `reps` rounds on the launch stream (the per-launch events of the
    # eager pass above add a few percent of queue overhead per launch).
    one = group_fns[dom_tile][-(dcount // instr_steps):]
    round_flops = sum(f for _, f in one)
    reps = max(5, int(0.1 / max(1e-6, dt_ms / instr_steps * 1e-3)) + 1)
    for fn, _ in one:
        fn()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    for _ in range(reps):
        for fn, _ in one:
            fn()
    r1.record()
    torch.cuda.synchronize()
    round_ms = r0.elapsed_time(r1) / reps
    achieved = round_flops / (round_ms * 1e-3) / 1e12
    gemm_kernels = {gemm_kernel_name(*k): {"launches_per_step": g[2] // instr_steps,
                                           "avg_launch_us": round(g[0] * 1e3 / g[2], 2),
                                           "tflops": round(g[1] / (g[0] * 1e-3) / 1e12, 1),
                                           "algorithmic_bytes_per_launch": round(g[3] / g[2])}
                    for k, g in sorted(gemm_by_tile.items(), key=lambda kv: -kv[1][0])}
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            ent = tj.get("kernels", {}).get(kname, {})
            # the counters hold for these sources and this kernel's mix of shapes in the step
            if tj.get("src_hash") == src_hash("gemm.hip", "nvfp4_device.h", "lds_dma.h", "mfma_fp16.h", "epilogue.h") and \
                    tj.get("workload") == wl.name and ent.get("algorithmic_bytes_per_launch") == round(dbytes / dcount):
                traffic = ent.get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None
    bandwidth = {n: {"GB/s": round(b[1] / (b[0] * 1e-3) / 1e9, 1), "frac_hbm": round(b[1] / (b[0] * 1e-3) / 8e12, 3),
                     "us_per_launch": round(b[0] * 1e3 / b[2], 2), "launches_per_step": b[2] // instr_steps,
                     "algorithmic_bytes_per_launch": round(b[1] / b[2])}
                 for n, b in sorted(bw.items())}
    res = {
        "value": round(value, 2),
        "ms_per_step": round(ms, 4),
        "ms_per_step_min": round(st["min"], 4),
        "ms_per_step_mean": round(st["mean"], 4),
        "ms_per_step_wall": round(wall * 1e3 / steps, 4),
        "steps": steps, "timed_ms": round(wall * 1e3, 1),
        "frac_fp4_peak": round(value / PEAK["fp4_mfma_tflops"], 4),
        "frac_fp16_peak": round(value / PEAK["fp16_mfma_tflops"], 4),
        "gemm_only_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
        "layers": len(layers), "tokens": layers[0].M, "hidden": layers[0].H, "intermediate": layers[0].I,
        "kv": layers[0].KV, "lora_rank": layers[0].r, "mlp_only": mlp_only,
        "gemm_gflop_per_step": round(flops / 1e9, 1),
        "resident_gb": round(torch.cuda.memory_allocated() / 1e9, 2),
        "timed_region": "hip graph replays of the step" if graph is not None else "eager steps",
        "schedule_matches_one_stream": schedule_matches,
        "kernel_ms_per_step_by_category": {k: round(v / instr_steps, 4) for k, v in sorted(cat_ms.items())},
        "instr_head_start_ok": head_start_ok,
        "bandwidth_kernels": bandwidth,
        "gemm_kernels": gemm_kernels,
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK["fp16_mfma_tflops"], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK["fp16_mfma_tflops"], 4),
                     "frac_of_fp4_peak": round(achieved / PEAK["fp4_mfma_tflops"], 4),
                     "launches_per_step": dcount // instr_steps,
                     "avg_launch_us": round(round_ms * 1e3 / len(one), 2),
                     "timing": f"{len(one)} launches of one step replayed back to back, {reps} rounds, "
                               f"one event pair on the launch stream",
                     "avg_launch_us_eager_events": round(dt_ms * 1e3 / dcount, 2),
                     "algorithmic_bytes_per_launch": round(dbytes / dcount),
                     "traffic": traffic},
    }
    del graph, run
    torch.cuda.synchronize()
    if check:
        res["cpu_baseline"], res["parity"] = cpu_baseline(torch, layers, wl, sample_rows or args.cpu_sample_rows)
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# the oracle leg: its timing on the host cores, and the parity of the timed outputs
# ---------------------------------------------------------------------------
def cpu_baseline(torch, layers, wl, nrows):
    """The oracle as it stands, on a bounded sample of the timed step: after the
    timed replays every buffer of the step holds the last step's values, and
    the oracle recomputes each stage of layer 0 (the bottom layer, reached last
    in backward) for `nrows` sampled token rows from the device's own inputs to
    that stage (stage-wise, so tolerances do not compound), the adapter
    gradients of one projection per block over all tokens on sampled output
    columns, and both cached layouts of one weight.  Returns (cpu_baseline,
    parity).  The oracle's wall time over those stages (device reads
    excluded) gives its rate in the metric's unit: GEMM FLOPs of the sampled
    rows per second."""
    import numpy as np
    from oracle import backward as obwd
    from oracle import fused as ofused
    from oracle import gemm as ogemm
    from oracle import lora as olora
    from oracle import nvfp4 as onv
    from oracle import tolerance as tol

    ly = layers[0]
    M, s = ly.M, LORA_SCALE
    rng = np.random.default_rng(1234 + wl.wid)
    rows = np.sort(rng.choice(M, size=min(nrows, M), replace=False))
    rows[-1] = M - 1
    ridx = torch.as_tensor(rows, device="cuda")
    checks, clock, gemm_flops = [], [0.0], [0.0]

    def oracle(fn):
        t0 = time.perf_counter()
        out = fn()
        clock[0] += time.perf_counter() - t0
        return out

    def nv(q, all_rows=False):
        if all_rows:
            return onv.NVFP4(q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.rscale.cpu().numpy())
        return onv.NVFP4(q.codes.index_select(0, ridx).cpu().numpy(), q.scales.index_select(0, ridx).cpu().numpy(),
                         q.rscale.index_select(0, ridx).cpu().numpy())

    def vals(t, all_rows=False):
        t = t if all_rows else t.index_select(0, ridx)
        b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def f32(t):
        return t.index_select(0, ridx).cpu().numpy()

    def same_nv(name, g, o):
        ok = (np.array_equal(g.codes, o.codes) and np.array_equal(g.scales, o.scales)
              and np.array_equal(np.asarray(g.rscale, np.float32).view(np.uint32),
                                 np.asarray(o.rscale, np.float32).view(np.uint32)))
        checks.append({"stage": name, "kind": "bit-exact", "ok": bool(ok)})

    def same_vals(name, got, want):
        ok = np.array_equal(np.asarray(got, np.float32).view(np.uint32), np.asarray(want, np.float32).view(np.uint32))
        checks.append({"stage": name, "kind": "bit-exact", "ok": bool(ok)})

    def within(name, got, ref, bound):
        n, worst = tol.violations(got, ref, bound)
        checks.append({"stage": name, "kind": "bound", "ok": n == 0, "worst_err_over_bound": round(worst, 4),
                       "elements": int(np.size(ref))})

    wfull = {n: nv(P["wf"], True) for n, P in ly.proj.items()}
    wbfull = {n: nv(P["wb"], True) for n, P in ly.proj.items()}

    def fwd_check(g, xq_dev):
        G = ly.grp[g]
        xq = nv(xq_dev)
        A = vals(G["A"], True)
        t_exact, _, t_abs = oracle(lambda: olora.lora_down(xq, A))
        within(f"lora_down {g}", vals(G["T"]), t_exact, tol.gemm_bound(t_exact, t_abs))
        for n in G["names"]:
            P = ly.proj[n]
            yref, yabs = oracle(lambda: ogemm.gemm_fwd(xq, wfull[n]))
            Tn, Bn = vals(P["T"]), vals(P["B"], True)
            term, tabs, _ = oracle(lambda: olora.lora_term(Tn, Bn.T, s))
            within(f"fwd {n}", vals(P["Y"]), yref + term, tol.gemm_bound(yref + term, yabs + tabs))
            gemm_flops[0] += 2.0 * len(rows) * P["p"].d_in * P["p"].d_out

    def dgrad_check(names, dx_dev):
        segs, lterm, labs = [], 0.0, 0.0
        for n in names:
            P = ly.proj[n]
            segs.append((nv(P["dyq_used"]), wbfull[n]))
            dT, A = vals(P["dT"]), vals(P["A"], True)
            term, tabs, _ = oracle(lambda: olora.lora_term(dT, A, 1.0))
            lterm, labs = lterm + term, labs + tabs
            gemm_flops[0] += 2.0 * len(rows) * P["p"].d_in * P["p"].d_out
        ref, rabs = oracle(lambda: ogemm.gemm_dgrad_multi(segs))
        within("dgrad " + "/".join(names), vals(dx_dev), ref + lterm, tol.gemm_bound(ref + lterm, rabs + labs))

    def lora_bwd_check(n, xq_dev, dy_dev):
        """dT on the sampled rows; dB on sampled rows of B and dA on sampled
        columns of A, each summed over all tokens (dA from the device's dT)."""
        P = ly.proj[n]
        N, K = P["p"].d_out, P["p"].d_in
        A, B = vals(P["A"], True), vals(P["B"], True)
        dyr = vals(dy_dev)
        dt_exact = oracle(lambda: s * (dyr @ B))
        within(f"lora_bwd dT {n}", vals(P["dT"]), dt_exact,
               tol.gemm_bound(dt_exact, abs(s) * (np.abs(dyr) @ np.abs(B))))
        cn = np.sort(rng.choice(N, size=min(32, N), replace=False))
        ck = np.sort(rng.choice(K, size=min(32, K), replace=False))
        xq = nv(xq_dev, True)
        dyc = vals(dy_dev.index_select(1, torch.as_tensor(cn, device="cuda")), True)
        dT_all = vals(P["dT"], True)

        def adapters():
            xt = onv.dequantize(xq)
            t = tol.bf16_rne(xt @ A.T)                           # T recomputed from X_q, rounded to BF16
            db = s * (dyc.T @ t)
            db_abs = abs(s) * (np.abs(dyc).T @ np.abs(t))
            db_slack = abs(s) * (np.abs(dyc).T @ tol.ulp_bf16(t))
            xk = xt[:, ck]
            return db, db_abs, db_slack, dT_all.T @ xk, np.abs(dT_all).T @ np.abs(xk)
        db, db_abs, db_slack, da, da_abs = oracle(adapters)
        within(f"lora_bwd dB {n}", vals(P["dB"], True)[cn], db, tol.gemm_bound(db, db_abs, db_slack))
        within(f"lora_bwd dA {n}", vals(P["dA"], True)[:, ck], da, tol.gemm_bound(da, da_abs))

    # offline weight layouts of one weight: both cached layouts, every row
    wname, wbf = ly.w_check
    wv = vals(wbf, True)
    owf, owb = oracle(lambda: ogemm.weight_layouts(wv))
    same_nv(f"W_fwd {wname}", wfull[wname], owf)
    same_nv(f"W_bwd {wname}", wbfull[wname], owb)

    dout, dout_q = ly.dout
    if not ly.mlp_only:
        # attention block forward
        h1, g1 = vals(ly.h1).astype(np.float32), vals(ly.g1, True).astype(np.float32)
        q, rstd, _ = oracle(lambda: ofused.rmsnorm_quant(h1, g1, 1e-5))
        same_nv("rmsnorm_quant (h1)", nv(ly.y1q), q)
        same_vals("rmsnorm rstd (h1)", f32(ly.rstd1), rstd)
        for g in (("qkv",) if "qkv" in ly.grp else ("q", "k", "v")):
            fwd_check(g, ly.y1q)
        at = vals(ly.attn)
        same_nv("nvfp4_quantize (attn)", nv(ly.aq), oracle(lambda: onv.quantize(at)))
        fwd_check("o", ly.aq)
    h2, g2 = vals(ly.h2).astype(np.float32), vals(ly.g2, True).astype(np.float32)
    q, rstd, _ = oracle(lambda: ofused.rmsnorm_quant(h2, g2, 1e-5))
    same_nv("rmsnorm_quant (h2)", nv(ly.y2q), q)
    same_vals("rmsnorm rstd (h2)", f32(ly.rstd2), rstd)
    for g in (("gu",) if "gu" in ly.grp else ("gate", "up")):
        fwd_check(g, ly.y2q)
    ga, ub = vals(ly.proj["gate"]["Y"]).astype(np.float32), vals(ly.proj["up"]["Y"]).astype(np.float32)
    hq, gq, uq, _ = oracle(lambda: ofused.silu_mul_quant(ga, ub))
    same_nv("silu_mul_quant h", nv(ly.hq), hq)
    same_nv("silu_mul_quant gate copy", nv(ly.gq), gq)
    same_nv("silu_mul_quant up copy", nv(ly.uq), uq)
    fwd_check("down", ly.hq)
    # MLP block backward
    dv = vals(dout)
    same_nv("output-gradient NVFP4 copy", nv(dout_q), oracle(lambda: onv.quantize(dv)))
    lora_bwd_check("down", ly.hq, dout)
    dgrad_check(("down",), ly.dh)
    gqo, uqo, dho = nv(ly.gq), nv(ly.uq), vals(ly.dh)
    da, db, daq, dbq = oracle(lambda: obwd.silu_mul_bwd_quant(gqo, uqo, dho))
    same_vals("silu_mul_bwd dgate", vals(ly.da).astype(np.float32), da)
    same_vals("silu_mul_bwd dup", vals(ly.db).astype(np.float32), db)
    same_nv("silu_mul_bwd dgate copy", nv(ly.daq), daq)
    same_nv("silu_mul_bwd dup copy", nv(ly.dbq), dbq)
    lora_bwd_check("up", ly.y2q, ly.db)
    dgrad_check(("gate", "up"), ly.dy2)
    args2 = (nv(ly.y2q), f32(ly.rstd2), vals(ly.g2, True), vals(ly.dy2), dv)
    out, outq = oracle(lambda: obwd.rmsnorm_bwd_residual(*args2))
    same_vals("rmsnorm_bwd_residual (MLP block)", vals(ly.dh2).astype(np.float32), out)
    same_nv("residual-gradient NVFP4 copy (MLP block)", nv(ly.dh2q), outq)
    if not ly.mlp_only:
        lora_bwd_check("o", ly.aq, ly.dh2)
        dgrad_check(("o",), ly.dattn)
        for n, d in (("q", ly.dq), ("k", ly.dk), ("v", ly.dv)):
            dd = vals(d)
            same_nv(f"nvfp4_quantize (d{n})", nv(ly.proj[n]["dyq_used"]), oracle(lambda: onv.quantize(dd)))
        lora_bwd_check("q", ly.y1q, ly.dq)
        dgrad_check(("q", "k", "v"), ly.dy1)
        args1 = (nv(ly.y1q), f32(ly.rstd1), vals(ly.g1, True), vals(ly.dy1), vals(ly.dh2))
        out, outq = oracle(lambda: obwd.rmsnorm_bwd_residual(*args1))
        same_vals("rmsnorm_bwd_residual (attention block)", vals(ly.dh1).astype(np.float32), out)
        same_nv("residual-gradient NVFP4 copy (attention block)", nv(ly.dh1q), outq)

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    failed = [c["stage"] for c in checks if not c["ok"]]
    parity = {"status": "pass" if not failed else "fail", "checks": len(checks), "failed": failed,
              "sampled_rows": len(rows), "layer": "bottom layer of the stack (instance 0) after the timed replays",
              "detail": checks}
    base = {"value": round(gemm_flops[0] / clock[0] / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} of {M} token rows of every stage of one decoder layer "
                      f"({'MLP block' if ly.mlp_only else 'attention and MLP blocks'}): the oracle's quantizers, "
                      f"fused RMSNorm / SiLU-multiply, float64 fwd and dgrad GEMMs against the full cached layouts, "
                      f"LoRA branch and backward formulas on those rows, plus adapter gradients over all tokens "
                      f"on sampled columns and one weight's two layouts; {clock[0]:.1f} s of oracle time, "
                      f"{gemm_flops[0] / 1e9:.2f} GFLOP of GEMM work counted"}
    return base, parity


# ---------------------------------------------------------------------------
# side legs
# ---------------------------------------------------------------------------
def timed_best(torch, fn, reps=5, per=1):
    """Best event time (ms) of fn over `reps` runs after a spin-kernel head start, divided by `per`."""
    fn()
    torch.cuda.synchronize()
    best = 1e30
    for _ in range(reps):
        torch.cuda._sleep(HEAD_START_CYCLES)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / per)
    return best


def copy_leg(torch, sizes):
    """A plain device copy (torch's elementwise copy kernel): 1 GiB read + 1 GiB
    write, and, for each (name, algorithmic bytes) of a bandwidth-bound kernel,
    a copy of half those bytes read and half written over 4 rotating buffer
    pairs (so small sizes are not served from the last-level cache)."""
    out = {}
    n = 1 << 29                                   # 1 GiB of BF16
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    t = timed_best(torch, lambda: dst.copy_(src), reps=5)
    big = 2 * 2 * n / (t * 1e-3) / 1e9
    out["1GiB"] = {"GB/s": round(big, 1), "frac_hbm": round(big / PEAK["hbm_gbs"], 3), "us": round(t * 1e3, 1)}
    del src, dst
    for name, nbytes in sizes:
        m = max(1, int(nbytes / 4))               # BF16 elements: half the bytes read, half written
        pairs = [(torch.empty(m, dtype=torch.bfloat16, device="cuda").normal_(),
                  torch.empty(m, dtype=torch.bfloat16, device="cuda")) for _ in range(4)]

        def fn():
            for a, b in pairs:
                b.copy_(a)
        t = timed_best(torch, fn, reps=5, per=len(pairs))
        gbs = 4 * m / (t * 1e-3) / 1e9
        out[name] = {"bytes": 4 * m, "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK["hbm_gbs"], 3),
                     "us": round(t * 1e3, 2)}
        del pairs
    torch.cuda.synchronize()
    return out


class MxLayer:
    """The same layer's projections in the MXFP4 variant, grouped like the NVFP4
    step: the projections that read one input (q/k/v, gate/up) run as one
    forward GEMM over their stacked weights and one input-gradient GEMM over
    their stacked gradients and backward layouts (MXFP4 has no row scale and
    every projection width is a multiple of the 32-element block, so stacking
    changes no code or scale); cached W_fwd / W_bwd in MXFP4 (quantized once,
    untimed) and MXFP4 GEMM inputs.  A step is 4 forward and 4 input-gradient
    GEMMs (those of 7 projections)."""

    def __init__(self, fw, torch, synth, wl, index=0):
        self.fw, self.torch = fw, torch
        off = 5000 + 1000 * index
        M = wl.tokens
        dev = torch.device("cuda:0")
        self.M, self.items, self.projections = M, [], list(wl.projections)
        P = {p.name: p for p in wl.projections}
        groups = [g for g in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)) if all(n in P for n in g)]
        for gi, names in enumerate(groups):
            ps = [P[n] for n in names]
            K, N = ps[0].d_in, sum(p.d_out for p in ps)
            w = torch.cat([synth.normal_torch((p.d_out, p.d_in), wl.w_std, wl.wid, off + 20 + wl.projections.index(p))
                           for p in ps])
            wf, wb = fw.mx_weight_layouts(w)                 # Q(W) [N x K] and Q(W^T) [K x N] of the stack
            del w
            xq = fw.mx_quantize(synth.activation_torch(wl, M, K, off + 60 + gi))
            dyq = fw.mx_quantize(synth.normal_torch((M, N), wl.dy_std, wl.wid, off + 80 + gi))
            self.items.append(dict(names=names, K=K, N=N, wf=wf, wb=wb, xq=xq, dyq=dyq,
                                   Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                                   dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev)))
        self.record = None

    def step(self):
        fw, torch = self.fw, self.torch
        for it in self.items:
            for a, b, out, n, k in ((it["xq"], it["wf"], it["Y"], it["N"], it["K"]),
                                    (it["dyq"], it["wb"], it["dX"], it["K"], it["N"])):
                if self.record is None:
                    fw.mx_gemm(a, b, out=out)
                else:
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    fw.mx_gemm(a, b, out=out)
                    e1.record()
                    self.record.append((e0, e1, (self.M, n, k)))

    def gemm_flops(self):
        return sum(4 * self.M * p.d_in * p.d_out for p in self.projections)


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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    st = stats([e0.elapsed_time(e1) for e0, e1 in evs])
    ms = st["median"]
    recs = []
    for ly in layers:
        ly.record = recs
    nsteps = min(steps, 10)
    for _ in range(nsteps):
        torch.cuda._sleep(HEAD_START_CYCLES)
        step()
    torch.cuda.synchronize()
    by_tile = {}
    for e0, e1, (M, N, K) in recs:
        t = by_tile.setdefault(_lib.gemm_tile(M, N, K), [0.0, 0.0, 0, 0.0])
        t[0] += e0.elapsed_time(e1)
        t[1] += 2.0 * M * N * K
        t[2] += 1
        t[3] += (M + N) * K * 17 / 32 + 2.0 * M * N       # MXFP4 A and B (codes + E8M0 scales), BF16 C
    dom = max(by_tile, key=lambda k: by_tile[k][0])
    dt, dfl, dn, dbytes = by_tile[dom]
    ach = dfl / (dt * 1e-3) / 1e12
    flops = sum(ly.gemm_flops() for ly in layers)
    gemm_ms = sum(v[0] for v in by_tile.values()) / nsteps
    value = flops / (ms * 1e-3) / 1e12
    del layers, run
    torch.cuda.synchronize()
    kname = f"pact::k_gemm_mxfp4<{dom[0] // 64}, {dom[1] // 64}>"
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "mxfp4_gemm_traffic.json")
    if os.path.exists(tfile):
        try:
            tj = json.load(open(tfile))
            # the counters hold for this kernel's sources and this leg's mix of shapes
            if tj.get("src_hash") == src_hash("mxfp4.hip", "lds_dma.h", "epilogue.h") and tj.get("kernel") == kname and \
                    tj.get("algorithmic_bytes_per_launch") == round(dbytes / dn):
                traffic = tj.get("bytes_per_launch")
        except (ValueError, OSError):
            traffic = None
    return {"gemm_tflops": round(value, 1), "frac_fp4_peak": round(value / PEAK["fp4_mfma_tflops"], 4),
            "ms_per_step": round(ms, 4), "ms_per_step_min": round(st["min"], 4), "layers": nlayers,
            "gemm_only_tflops_events": round(flops / (gemm_ms * 1e-3) / 1e12, 1),
            "timed_region": ("eager" if eager else "hip graph replays") +
                            " of the MXFP4 GEMMs of 7 projections per layer (q/k/v and gate/up stacked: 8 launches)",
            "roofline": {"kernel": kname, "bound": "mfma",
                         "achieved": round(ach, 1), "peak": PEAK["fp4_mfma_tflops"], "unit": "TFLOP/s",
                         "frac": round(ach / PEAK["fp4_mfma_tflops"], 4), "launches_per_step": dn // nsteps,
                         "avg_launch_us": round(dt * 1e3 / dn, 2),
                         "algorithmic_bytes_per_launch": round(dbytes / dn), "traffic": traffic}}


class MxMlpBlock:
    """One MLP block of the workload entirely in the MXFP4 variant: cached MXFP4
    W_fwd / W_bwd of gate, up and down (gate and up stacked in the forward
    layout), MXFP4 RMSNorm and SiLU-multiply quantizers, MXFP4 copies of every
    GEMM input, backward chained through the BF16 residual gradient.  No LoRA
    branch: the MXFP4 variant is a format comparison of the frozen path."""

    def __init__(self, fw, torch, synth, wl, index=0):
        self.fw, self.torch = fw, torch
        P = {p.name: p for p in wl.projections}
        M, H, I = wl.tokens, P["gate"].d_in, P["gate"].d_out
        self.M, self.H, self.I = M, H, I
        dev = torch.device("cuda:0")
        off, wid = 7000 + 1000 * index, wl.wid
        self.x = synth.activation_torch(wl, M, H, off + 1)
        self.g = synth.uniform_torch((H,), 0.9, 1.1, wid, off + 2)
        self.dout = synth.normal_torch((M, H), wl.dy_std, wid, off + 3)
        wg = synth.normal_torch((I, H), wl.w_std, wid, off + 4)
        wu = synth.normal_torch((I, H), wl.w_std, wid, off + 5)
        wd = synth.normal_torch((H, I), wl.w_std, wid, off + 6)
        self.w_gu = fw.mx_quantize(torch.cat([wg, wu], 0).contiguous())       # [2I x H]
        self.w_gate_b = fw.mx_quantize(wg, transpose=True)                   # [H x I]
        self.w_up_b = fw.mx_quantize(wu, transpose=True)
        self.w_down, self.w_down_b = fw.mx_weight_layouts(wd)               # [H x I], [I x H]
        del wg, wu, wd
        mx = lambda cols: fw.empty_mxfp4(M, cols, dev)
        bf = lambda cols: torch.empty((M, cols), dtype=torch.bfloat16, device=dev)
        self.yq, self.rstd = mx(H), torch.empty((M,), dtype=torch.float32, device=dev)
        self.gu, self.out = bf(2 * I), bf(H)
        self.hq, self.gq, self.uq = mx(I), mx(I), mx(I)
        self.doutq, self.dh = mx(H), bf(I)
        self.dg, self.du, self.dgq, self.duq = bf(I), bf(I), mx(I), mx(I)
        self.dy, self.dx, self.dxq = bf(H), bf(H), mx(H)

    def step(self):
        fw, I = self.fw, self.I
        fw.mx_rmsnorm_quant(self.x, self.g, 1e-5, out=(self.yq, self.rstd))
        fw.mx_gemm(self.yq, self.w_gu, out=self.gu)
        fw.mx_silu_mul_quant(self.gu[:, :I], self.gu[:, I:], out=(self.hq, self.gq, self.uq))
        fw.mx_gemm(self.hq, self.w_down, out=self.out)
        fw.mx_quantize(self.dout, out=self.doutq)
        fw.mx_gemm(self.doutq, self.w_down_b, out=self.dh)
        fw.mx_silu_mul_bwd_quant(self.gq, self.uq, self.dh, out=(self.dg, self.du, self.dgq, self.duq))
        fw.mx_gemm(self.dgq, self.w_gate_b, out=self.dy)
        fw.mx_gemm(self.duq, self.w_up_b, out=self.dy, accumulate=True)
        fw.mx_rmsnorm_bwd_residual(self.yq, self.rstd, self.g, self.dy, resid=self.dout, out=(self.dx, self.dxq))

    def gemm_flops(self):
        return 12.0 * self.M * self.H * self.I          # 3 forward + 3 input-gradient GEMMs of M*H*I MACs


def mxfp4_mlp_parity(torch, blk, nrows, seed):
    """Stage-wise oracle parity of one MXFP4 MLP block's last step on `nrows`
    sampled token rows: each stage from the device's own inputs to it."""
    import numpy as np
    from oracle import mxfp4 as omx
    from oracle import tolerance as tol

    M, I = blk.M, blk.I
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(M, size=min(nrows, M), replace=False))
    rows[-1] = M - 1
    ridx = torch.as_tensor(rows, device="cuda")
    checks = []

    def mx(q, all_rows=False):
        c, s = (q.codes, q.scales) if all_rows else (q.codes.index_select(0, ridx), q.scales.index_select(0, ridx))
        return omx.MXFP4(c.cpu().numpy(), s.cpu().numpy())

    def vals(t, all_rows=False):
        t = t if all_rows else t.index_select(0, ridx)
        b = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def same_mx(name, g, o):
        ok = np.array_equal(g.codes, o.codes) and np.array_equal(g.scales, o.scales)
        checks.append({"stage": name, "kind": "bit-exact", "ok": bool(ok)})

    def same_vals(name, got, want):
        ok = np.array_equal(np.asarray(got, np.float32).view(np.uint32), np.asarray(want, np.float32).view(np.uint32))
        checks.append({"stage": name, "kind": "bit-exact", "ok": bool(ok)})

    def within(name, got, ref, bound):
        n, worst = tol.violations(got, ref, bound)
        checks.append({"stage": name, "kind": "bound", "ok": n == 0, "worst_err_over_bound": round(worst, 4),
                       "elements": int(np.size(ref))})

    x, g = vals(blk.x).astype(np.float32), vals(blk.g, True).astype(np.float32)
    yq, rstd, _ = omx.rmsnorm_quant(x, g, 1e-5)
    same_mx("mx_rmsnorm_quant", mx(blk.yq), yq)
    same_vals("mx_rmsnorm rstd", blk.rstd.index_select(0, ridx).cpu().numpy(), rstd)
    ref, rabs = omx.gemm_nt(mx(blk.yq), mx(blk.w_gu, True))
    within("mx fwd gate/up (stacked)", vals(blk.gu), ref, tol.gemm_bound(ref, rabs))
    gu = vals(blk.gu).astype(np.float32)
    hq, gq, uq, _ = omx.silu_mul_quant(gu[:, :I], gu[:, I:])
    same_mx("mx_silu_mul_quant h", mx(blk.hq), hq)
    same_mx("mx_silu_mul_quant gate copy", mx(blk.gq), gq)
    same_mx("mx_silu_mul_quant up copy", mx(blk.uq), uq)
    ref, rabs = omx.gemm_nt(mx(blk.hq), mx(blk.w_down, True))
    within("mx fwd down", vals(blk.out), ref, tol.gemm_bound(ref, rabs))
    dv = vals(blk.dout)
    same_mx("mx_quantize (output gradient)", mx(blk.doutq), omx.quantize(dv))
    ref, rabs = omx.gemm_nt(mx(blk.doutq), mx(blk.w_down_b, True))
    within("mx dgrad down", vals(blk.dh), ref, tol.gemm_bound(ref, rabs))
    dg, du, dgq, duq = omx.silu_mul_bwd_quant(mx(blk.gq), mx(blk.uq), vals(blk.dh))
    same_vals("mx_silu_mul_bwd dgate", vals(blk.dg).astype(np.float32), dg)
    same_vals("mx_silu_mul_bwd dup", vals(blk.du).astype(np.float32), du)
    same_mx("mx_silu_mul_bwd dgate copy", mx(blk.dgq), dgq)
    same_mx("mx_silu_mul_bwd dup copy", mx(blk.duq), duq)
    # two launches, the second accumulating onto the first's BF16 output: one
    # extra BF16 rounding of the gate partial on top of the GEMM bound
    rg, ag = omx.gemm_nt(mx(blk.dgq), mx(blk.w_gate_b, True))
    ru, au = omx.gemm_nt(mx(blk.duq), mx(blk.w_up_b, True))
    within("mx dgrad gate + up", vals(blk.dy), rg + ru, tol.gemm_bound(rg + ru, ag + au, tol.ulp_bf16(rg)))
    out, outq = omx.rmsnorm_bwd_residual(mx(blk.yq), blk.rstd.index_select(0, ridx).cpu().numpy(),
                                         vals(blk.g, True), vals(blk.dy), dv)
    same_vals("mx_rmsnorm_bwd_residual", vals(blk.dx).astype(np.float32), out)
    same_mx("mx residual-gradient copy", mx(blk.dxq), outq)
    ok = all(c["ok"] for c in checks)
    return {"status": "pass" if ok else "FAIL", "rows_sampled": int(len(rows)), "checks": checks}


def mxfp4_mlp_leg(fw, torch, synth, wl, nblocks, steps, warmup, check=True, nrows=8):
    """The MXFP4 MLP block chain (forward and input-gradient, quantizers fused)
    at the workload's shapes over `nblocks` distinct block instances, timed as
    HIP-graph replays; GEMM TFLOP/s of the chain, its per-launch kernel times
    and the stage-wise parity of the last replay."""
    blocks = [MxMlpBlock(fw, torch, synth, wl, i) for i in range(nblocks)]

    def step():
        for b in blocks:
            b.step()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        graph.replay()
        e1.record()
    torch.cuda.synchronize()
    st = stats([e0.elapsed_time(e1) for e0, e1 in evs])
    flops = sum(b.gemm_flops() for b in blocks)
    res = {"workload": f"{wl.name} MLP block in MXFP4 (rmsnorm+quant, stacked gate/up, silu-mul+quant, down; "
                       f"backward: quantize dOut, down dgrad, silu-mul bwd+quant, gate and up dgrad, "
                       f"rmsnorm bwd+residual+quant)",
           "blocks": nblocks, "gemm_tflops": round(flops / (st["median"] * 1e-3) / 1e12, 1),
           "ms_per_step": round(st["median"], 4), "ms_per_step_min": round(st["min"], 4),
           "gemm_gflop_per_step": round(flops / 1e9, 1), "timed_region": "hip graph replays"}
    del graph
    torch.cuda.synchronize()
    if check:
        res["parity"] = mxfp4_mlp_parity(torch, blocks[0], nrows, 4321 + wl.wid)
    del blocks
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def recipe_leg(fw, torch, synth, wl, n_inst=4, reps=5):
    """The recipe variants at the Llama-3B shapes (M = 4096), over n_inst
    rotating instances: the Q/K/V and gate/up forward and input-gradient GEMMs
    with separate weights versus stacked weights (one GEMM per group, the
    stacked dgrad summing every consumer), and the quantizer's variants on a
    [4096 x 3072] output gradient."""
    M, H, I, KV = wl.tokens, 3072, 8192, 1024
    dev = torch.device("cuda:0")
    bf = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=dev)
    inst = []
    for i in range(n_inst):
        off = 9000 + 100 * i
        d = {"x": fw.quantize(synth.activation_torch(wl, M, H, off))}
        w = {n: synth.normal_torch((rows, H), wl.w_std, wl.wid, off + k)
             for k, (n, rows) in enumerate((("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I)))}
        d["sep"] = {n: fw.weight_layouts(t) for n, t in w.items()}
        d["qkv"] = fw.weight_layouts(torch.cat([w["q"], w["k"], w["v"]], 0).contiguous())
        d["gu"] = fw.weight_layouts(torch.cat([w["gate"], w["up"]], 0).contiguous())
        del w
        dy = {n: synth.normal_torch((M, c), wl.dy_std, wl.wid, off + 10 + k)
              for k, (n, c) in enumerate((("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I)))}
        d["dyq"] = {n: fw.quantize(t) for n, t in dy.items()}
        d["dy_qkv"] = fw.quantize(torch.cat([dy["q"], dy["k"], dy["v"]], 1).contiguous())
        d["dy_gu"] = fw.quantize(torch.cat([dy["gate"], dy["up"]], 1).contiguous())
        del dy
        d["y"] = {n: bf(M, c) for n, c in (("q", H), ("k", KV), ("v", KV), ("gate", I), ("up", I))}
        d["y_qkv"], d["y_gu"], d["dx1"], d["dx2"] = bf(M, H + 2 * KV), bf(M, 2 * I), bf(M, H), bf(M, H)
        inst.append(d)

    def separate():
        for d in inst:
            for n in ("q", "k", "v", "gate", "up"):
                fw.gemm_fwd(d["x"], d["sep"][n][0], out=d["y"][n])
            for k, n in enumerate(("q", "k", "v")):
                fw.gemm_dgrad(d["dyq"][n], d["sep"][n][1], out=d["dx1"], accumulate=k > 0)
            for k, n in enumerate(("gate", "up")):
                fw.gemm_dgrad(d["dyq"][n], d["sep"][n][1], out=d["dx2"], accumulate=k > 0)

    def stacked():
        for d in inst:
            fw.gemm_fwd(d["x"], d["qkv"][0], out=d["y_qkv"])
            fw.gemm_fwd(d["x"], d["gu"][0], out=d["y_gu"])
            fw.gemm_dgrad(d["dy_qkv"], d["qkv"][1], out=d["dx1"])
            fw.gemm_dgrad(d["dy_gu"], d["gu"][1], out=d["dx2"])

    flops = 2.0 * M * H * (H + 2 * KV + 2 * I) * 2          # forward + input gradient
    t_sep, t_cat = timed_best(torch, separate, reps, n_inst), timed_best(torch, stacked, reps, n_inst)
    out = {"stacked_qkv_gate_up": {"separate_tflops": round(flops / (t_sep * 1e-3) / 1e12, 1),
                                   "stacked_tflops": round(flops / (t_cat * 1e-3) / 1e12, 1),
                                   "separate_ms": round(t_sep, 4), "stacked_ms": round(t_cat, 4),
                                   "launches": {"separate": 10, "stacked": 4}}}
    del inst
    # quantizer variants on [M x H]
    xs = [synth.normal_torch((M, H), wl.dy_std, wl.wid, 9900 + i) for i in range(n_inst)]
    qs = [fw.empty_nvfp4(M, H, dev) for _ in range(n_inst)]
    amax = torch.empty((), dtype=torch.float32, device=dev)
    variants = {"default": lambda x, q: fw.quantize(x, out=q),
                "round_up_scales": lambda x, q: fw.quantize_ex(x, round_up=True, out=q),
                "tensor_scale_two_pass": lambda x, q: fw.quantize_ex(x, tensor_scale=True, amax=amax, out=q),
                "fp32_tensor_scale_two_pass": lambda x, q: fw.quantize_ex(x, tensor_scale=True, fp32_scale=True,
                                                                           amax=amax, out=q),
                "fp32_tensor_scale_supplied_amax": lambda x, q: fw.quantize_ex(x, tensor_scale=True,
                                                                                fp32_scale=True, amax=amax,
                                                                                compute_amax=False, out=q)}
    qb = {}
    for name, f in variants.items():
        def fn(f=f):
            for x, q in zip(xs, qs):
                f(x, q)
        best = timed_best(torch, fn, reps, len(xs))
        qb[name] = {"us": round(best * 1e3, 2),
                    "GB/s": round(kernel_bytes(("quant", M, H)) / (best * 1e-3) / 1e9, 1)}
    out["quantizer_4096x3072"] = qb
    del xs, qs
    torch.cuda.synchronize()
    out["fp32_tensor_scale_gemm"] = fp32_scale_gemm_leg(fw, torch, synth, wl, n_inst, reps)
    return out


def fp32_scale_gemm_leg(fw, torch, synth, wl, n_inst=4, reps=5):
    """The stacked gate/up forward GEMM ([4096 x 3072] x [16384 x 3072]^T, LoRA
    rank 32) on operands of the default recipe (power-of-two row scales, fused
    term in the direct-to-LDS kernel) and of the FP32 tensor-scale recipe: the
    plain GEMM (same kernel) and with the term (register-staged kernel,
    PACT_GEMM_ANY_ROW_SCALES)."""
    M, H, I, r = wl.tokens, 3072, 8192, 32
    dev = torch.device("cuda:0")
    inst = []
    for i in range(n_inst):
        off = 9500 + 100 * i
        x = synth.activation_torch(wl, M, H, off)
        w = synth.normal_torch((2 * I, H), wl.w_std, wl.wid, off + 1)
        d = {"x": fw.quantize(x), "w": fw.quantize(w),
             "x32": fw.quantize_ex(x, tensor_scale=True, fp32_scale=True),
             "w32": fw.quantize_ex(w, tensor_scale=True, fp32_scale=True),
             "t": synth.normal_torch((M, r), 0.3, wl.wid, off + 2),
             "b": synth.normal_torch((2 * I, r), 0.01, wl.wid, off + 3),
             "y": torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev)}
        del x, w
        inst.append(d)
    runs = {"default_recipe_with_lora": lambda d: fw.gemm_fwd(d["x"], d["w"], lora_t=d["t"], lora_b=d["b"],
                                                              lora_scale=LORA_SCALE, out=d["y"]),
            "fp32_tensor_scale_no_lora": lambda d: fw.gemm_fwd(d["x32"], d["w32"], out=d["y"]),
            "fp32_tensor_scale_with_lora": lambda d: fw.gemm_fwd(d["x32"], d["w32"], lora_t=d["t"], lora_b=d["b"],
                                                                 lora_scale=LORA_SCALE, out=d["y"],
                                                                 any_row_scales=True)}
    flops = 2.0 * M * H * 2 * I
    res = {}
    for name, f in runs.items():
        def fn(f=f):
            for d in inst:
                f(d)
        t = timed_best(torch, fn, reps, len(inst))
        res[name] = {"us": round(t * 1e3, 1), "tflops": round(flops / (t * 1e-3) / 1e12, 1)}
    del inst
    torch.cuda.synchronize()
    return res


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

        def fn():
            for x, q in zip(xs, qs):
                fw.quantize(x, out=q)
        best = timed_best(torch, fn, reps, len(xs))
        gbs = kernel_bytes(("quant", M, K)) / (best * 1e-3) / 1e9
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
    projections (each with its own launch; the step merges q/k/v and gate/up,
    so this is an upper bound for those)."""
    M, r = wl.tokens, wl.lora_rank
    out, tot, seen = {}, 0.0, {}
    for i, p in enumerate(wl.projections):
        key = (p.d_in, p.d_out)
        if key not in seen:
            x = synth.activation_torch(wl, M, p.d_in, 9800 + i)
            w = synth.normal_torch((p.d_out, p.d_in), wl.w_std, wl.wid, 9810 + i)
            dy = synth.normal_torch((M, p.d_out), wl.dy_std, wl.wid, 9820 + i)
            T = synth.normal_torch((M, r), 0.3, wl.wid, 9830 + i)
            B = synth.normal_torch((p.d_out, r), wl.a_std, wl.wid, 9840 + i)
            A = synth.normal_torch((r, p.d_in), wl.a_std, wl.wid, 9850 + i)
            dT = synth.normal_torch((M, r), 0.01, wl.wid, 9860 + i)
            xq, wf, wb, dyq = fw.quantize(x), fw.quantize(w), fw.quantize(w, transpose=True), fw.quantize(dy)
            y = torch.empty((M, p.d_out), dtype=torch.bfloat16, device="cuda")
            dx = torch.empty((M, p.d_in), dtype=torch.bfloat16, device="cuda")

            def many(fn):
                def run():
                    for _ in range(n):
                        fn()
                return timed_best(torch, run, reps, n) * 1e3
            f0 = many(lambda: fw.gemm_fwd(xq, wf, out=y))
            f1 = many(lambda: fw.gemm_fwd(xq, wf, lora_t=T, lora_b=B, lora_scale=LORA_SCALE, out=y))
            d0 = many(lambda: fw.gemm_dgrad(dyq, wb, out=dx))
            d1 = many(lambda: fw.gemm_dgrad(dyq, wb, out=dx, lora_dt=dT, lora_a=A))
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
    M = wl.tokens
    dev = torch.device("cuda:0")
    inst = []
    for i in range(n_inst):
        off = 12000 + 100 * i
        items = []
        for k, p in enumerate(wl.projections):
            w = synth.normal_torch((p.d_out, p.d_in), wl.w_std, wl.wid, off + k)
            wf, wb = fw.weight_layouts(w)
            del w
            items.append(dict(p=p, wf=wf, wb=wb, sl=fw.SingleLayoutWeight(wf),
                              dyq=fw.quantize(synth.normal_torch((M, p.d_out), wl.dy_std, wl.wid, off + 20 + k)),
                              dx=torch.empty((M, p.d_in), dtype=torch.bfloat16, device=dev)))
        inst.append(items)

    def dual():
        for items in inst:
            for it in items:
                fw.gemm_dgrad(it["dyq"], it["wb"], out=it["dx"])

    def single():
        for items in inst:
            for it in items:
                fw.gemm_dgrad_fwd_layout(it["dyq"], it["sl"], out=it["dx"])

    per = {}
    for j, it0 in enumerate(inst[0]):
        def one(j=j):
            for items in inst:
                fw.gemm_dgrad_fwd_layout(items[j]["dyq"], items[j]["sl"], out=items[j]["dx"])
        per[it0["p"].name] = (timed_best(torch, one, reps, n_inst), 2.0 * M * it0["p"].d_in * it0["p"].d_out)
    flops = sum(2.0 * M * it["p"].d_in * it["p"].d_out for it in inst[0])
    t_dual, t_single = timed_best(torch, dual, reps, n_inst), timed_best(torch, single, reps, n_inst)
    nv = lambda r, c: r * c * 9 // 16 + 4 * r
    bytes_dual = sum(nv(it["p"].d_out, it["p"].d_in) + nv(it["p"].d_in, it["p"].d_out) for it in inst[0])
    bytes_single = sum(nv(it["p"].d_out, it["p"].d_in) + 8 for it in inst[0])
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


# ---------------------------------------------------------------------------
def main():
    global QKV_GRAD_QUANT
    args = parse()
    QKV_GRAD_QUANT = args.qkv_grad_quant
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              f"described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    import frozen_weight_gemms_amd as fw
    import synth

    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[2]
    legs_off = args.step_only

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    progress(f"headline step: {wl.name}, {args.layers} layers")
    head = run_config(fw, torch, synth, wl, args.layers, args.steps, args.warmup, args.instr_steps, args,
                      check=not (args.no_cpu_baseline or legs_off))
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, fp16 MFMA (exact products), fp32 accumulation, bf16 output",
        "data": "synthetic (seeded BF16 device draws: activations N(0,1) with 1% outlier channels x20, "
                "weights N(0,0.02), grads N(0,0.01), LoRA A and B N(0,0.01))",
        "config": {"workload": f"llama3b decoder-layer frozen projections fwd+dgrad + fused quantizers + LoRA r16, "
                               f"M=4096, {head['layers']} distinct layer instances per step, backward chained "
                               f"through BF16 residual gradients",
                   "layers": head["layers"], "resident_gb": head["resident_gb"], "tokens": head["tokens"],
                   "hidden": head["hidden"], "intermediate": head["intermediate"], "kv": head["kv"],
                   "lora_rank": head["lora_rank"], "gemm_gflop_per_step": head["gemm_gflop_per_step"],
                   "parallelism": "single-gpu"},
    }
    for k in ("roofline", "cpu_baseline", "parity", "frac_fp4_peak", "frac_fp16_peak", "ms_per_step_min",
              "ms_per_step_mean", "ms_per_step_wall", "timed_ms", "gemm_only_tflops", "timed_region",
              "schedule_matches_one_stream", "kernel_ms_per_step_by_category", "instr_head_start_ok",
              "bandwidth_kernels", "gemm_kernels"):
        if k in head:
            result[k] = head[k]
    if isinstance(result.get("parity"), dict):
        result["parity_status"] = result["parity"]["status"]
    result["schedule"] = ("stacked q/k/v and gate/up forward GEMMs (stacked LoRA rank <= 128); one "
                          "input-gradient launch each for q/k/v and gate/up; LoRA dT per projection before its "
                          "input gradient; dq, dk, dv quantized " +
                          ("in one nvfp4_quantize_batch launch; " if QKV_GRAD_QUANT == "batched" else
                           "each beside its projection's dT; ") +
                          "per layer two batched dA/dB calls (down/gate/up after the gate/up "
                          "input gradient, o/q/k/v after the q/k/v one), each after T is recomputed from the "
                          "saved NVFP4 input by one stacked lora_down per input; " +
                          ("one stream" if args.sequential else
                           "the dT of gate/up and of q/k/v on 2 side streams, the dA/dB batches on a third, "
                           "joined before the next input-gradient GEMM"))
    if not legs_off and not args.no_configs:
        cfgs = {}
        for wid, nlay, mlp in ((1, 2, False), (3, 2, True), (4, 1, False)):
            w = synth.WORKLOADS[wid]
            progress(f"config {w.name}")
            c = run_config(fw, torch, synth, w, nlay, max(10, min(args.steps, 30)), 3, 3, args, mlp_only=mlp,
                           check=not args.no_cpu_baseline, sample_rows=args.config_sample_rows)
            c["workload"] = w.name
            cfgs[w.name] = c
        result["configs"] = cfgs
    if not legs_off and not args.no_recipes:
        progress("recipe, single-layout, quantizer, LoRA-term and copy legs")
        result["recipe_variants"] = recipe_leg(fw, torch, synth, wl)
        result["single_layout_dgrad"] = single_layout_leg(fw, torch, synth, wl)
        result["quantizer_bandwidth"] = quantizer_leg(fw, torch)
        result["lora_term"] = lora_term_leg(fw, torch, synth, wl)
        sizes = [(n, b["algorithmic_bytes_per_launch"]) for n, b in head["bandwidth_kernels"].items()]
        cp = copy_leg(torch, sizes)
        result["hbm_copy"] = cp
        for n, b in result["bandwidth_kernels"].items():
            if n in cp:
                b["copy_GB/s_same_bytes"] = cp[n]["GB/s"]
                b["frac_of_copy"] = round(b["GB/s"] / cp[n]["GB/s"], 3)
    if not legs_off and not args.no_mxfp4:
        progress("MXFP4 leg")
        result["mxfp4_variant"] = mxfp4_leg(fw, torch, synth, wl, max(1, args.layers), min(args.steps, 30), 3,
                                            eager=args.eager)
        progress("MXFP4 MLP block chain")
        result["mxfp4_mlp_block"] = mxfp4_mlp_leg(fw, torch, synth, synth.WORKLOADS[3], 2, min(args.steps, 30), 3,
                                                  check=not args.no_cpu_baseline)
    if not legs_off:
        # measured MFMA-loop peak beside the published dense peaks (no memory traffic in the loop)
        p16, c16 = fw.mfma_probe(0)
        p4, c4 = fw.mfma_probe(1)
        result["mfma_loop_peak"] = {"fp16_tflops": round(p16, 1), "fp16_clock_ghz": round(c16, 3),
                                    "fp4_tflops": round(p4, 1), "fp4_clock_ghz": round(c4, 3),
                                    "probe": "pact_mfma_probe: 512 workgroups x 4 waves, 16 independent MFMA "
                                             "chains per wave, 4000 iterations; clock from s_memtime / s_memrealtime"}
        result["roofline"]["measured_peak"] = round(p16, 1)
        result["roofline"]["frac_of_measured_peak"] = round(result["roofline"]["achieved"] / p16, 4)
        if "mxfp4_variant" in result:
            mr = result["mxfp4_variant"]["roofline"]
            mr["measured_peak"] = round(p4, 1)
            mr["frac_of_measured_peak"] = round(mr["achieved"] / p4, 4)
    result["device"] = {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__}
    if args.copy_calibration:
        x = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        y = torch.empty_like(x)
        torch.neg(x, out=y)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
