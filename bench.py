"""Benchmark of the block-scaled FP8 linear path on one MI355X.

One step is one pass of the whole path over one batch of seeded synthetic
input already resident in HBM.  For the default workload (the dense MLP
layer-0 shape of DeepSeek-V3: x [8192, 7168], W_up [18432, 7168],
W_down [7168, 18432]) a step is

    act_quant(x) -> fp8 GEMM up with act_quant(H) in its epilogue -> fp8 GEMM down
    -> weight_dequant(W_up)

(--workload dense-mlp-unfused runs act_quant(H) as its own kernel after a bf16 H;
the codes and scales are the same bits either way).

Printed: one JSON line.  `value` is the step's GEMM FLOP divided by the step's
wall time (TFLOP/s); `kernels` gives each kernel's average duration from HIP
events recorded around every launch inside the timed region, with its
algorithmic FLOP or bytes per launch and its fraction of the MI355X peak that
bounds it, and, after the timed region, the same launch timed alone: rounds of
back-to-back launches between one event pair (so the event overhead of one
short launch does not count), median and min per launch over the rounds;
HBM-bound launches are also timed "cold", cycling over copies of their
buffers totalling more than 1 GB so no launch finds its data in the 256 MB
Infinity Cache or in L2.  `roofline` repeats the timed-region figure for the
dominant kernel; `clock` is the GPU's shader clock and socket power sampled
from sysfs during the timed region (and the board power cap); `cpu_baseline`
times the CPU oracle on a bounded, proportional sample of the same step.

Other workloads (parity-test shapes, measured on demand): --workload tiny |
decode | moe-pair (the expert pair, act_quant of H fused into the first GEMM as in the
dense step) | moe-pair-unfused | dense-mlp-unfused | grouped | moe-layer | bf16-branch |
expert-ffn (one expert's gated FFN with the SiLU gate and act_quant fused into the
[w1; w3] GEMM's epilogue) | dense-mlp-ue8m0 (power-of-two scales applied by the MFMA).  moe-layer is the routed
experts of one GPU end to end on the device: moe_dispatch(topk) ->
act_quant_rows(x, row_token) -> grouped GEMM (row buffers sized for T*k rows)
-> moe_combine (weighted sum back to token order).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_scaled_fp8_04_amd as bfp8  # noqa: E402
from block_scaled_fp8_04_amd import synth  # noqa: E402

BLOCK = 128
PEAK_FP8_TFLOPS = 5000.0          # MI355X dense fp8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16 MFMA (no sparsity)

WORKLOADS = {"tiny": 0, "decode": 1, "moe-pair": 2, "moe-pair-unfused": 2, "dense-mlp": 3,
             "grouped": 4, "moe-layer": 4, "bf16-branch": 3, "dense-mlp-unfused": 3, "expert-ffn": 2,
             "dense-mlp-ue8m0": 3}


# ------------------------------------------------------------------ accounting

def gemm_workspace(M, N, K, dev):
    """The fp32 workspace bfp8_gemm uses at this shape (split-K of skinny problems, or the
    split last round of large ones), or None when it uses none."""
    n = bfp8.bfp8_gemm_workspace_size(M, N, K)
    return torch.empty(max(1, n // 4), dtype=torch.float32, device=dev) if n else None


def act_quant_bytes(M, K):
    return 2 * M * K + M * K + 4 * M * (K // BLOCK)


def dequant_bytes(N, K):
    return N * K + 2 * N * K + 4 * (-(-N // BLOCK)) * (-(-K // BLOCK))


def gemm_bytes(M, N, K, G=1):
    return M * K + G * N * K + 2 * M * N + 4 * M * (K // BLOCK) + 4 * G * (-(-N // BLOCK)) * (K // BLOCK)


def dispatch_bytes(T, k, rows, G):
    return 4 * T * k + 4 * T * k + 4 * rows + 4 * (G + 1)


def combine_bytes(T, k, rows, N):
    return 2 * rows * N + 8 * T * k + 2 * T * N


def sha_of(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]


# ------------------------------------------------------------------ the steps

class Launch:
    """One named launch: op(*args), with its algorithmic work and the peak that bounds it.
    Copies of the launch (for cold timing) run the same op on clones of every tensor."""

    def __init__(self, name, op, args, flop, nbytes, bound):
        self.name, self.op, self.args = name, op, tuple(args)
        self.flop, self.bytes, self.bound = flop, nbytes, bound

    def __call__(self):
        self.op(*self.args)

    def footprint(self):
        return sum(a.numel() * a.element_size() for a in self.args if isinstance(a, torch.Tensor))

    def copies(self, n):
        out = []
        for _ in range(n):
            args = tuple(a.clone() if isinstance(a, torch.Tensor) else a for a in self.args)
            out.append(Launch(self.name, self.op, args, self.flop, self.bytes, self.bound))
        return out


class Step:
    """Device buffers and the ordered launches of one step; every launch is named."""

    def __init__(self, wl, dev, kind=None, cold=False):
        self.wl = wl
        self.dev = dev
        t = wl.tensors
        c = wl.config
        if kind in ("moe-layer", "bf16-branch", "dense-mlp", "expert-ffn", "dense-mlp-ue8m0",
                    "moe-pair"):
            c = kind
        self.launches = []            # (name, callable, flops, bytes, bound)
        self.hashes = {}
        for k, v in t.items():
            if k != "token_ids":
                self.hashes[k] = sha_of(v)
        if c in (0, 1):
            M, N, K = wl.meta["M"], wl.meta["N"], wl.meta["K"]
            x = t["x"].to(dev)
            w, s = t["w1"].to(dev), t["s1"].to(dev)
            q = torch.empty(M, K, dtype=torch.uint8, device=dev)
            qs = torch.empty(M, K // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            ws_bytes = bfp8.bfp8_gemm_workspace_size(M, N, K)
            work = torch.empty(max(1, ws_bytes // 4), dtype=torch.float32, device=dev) if ws_bytes else None
            # cold: successive steps read different copies of the weight, more than 512 MB in
            # all, so no step finds its weight in the 256 MB Infinity Cache or in L2
            copies = [(w, s)]
            if cold:
                n_copies = -(-(512 << 20) // (w.numel() + 4 * s.numel()))
                copies = [(w.clone(), s.clone()) for _ in range(n_copies)]
            self.copies, self.turn = copies, 0

            def gemm_step(q, qs, y, work):
                wc, sc = self.copies[self.turn % len(self.copies)]
                self.turn += 1
                bfp8.bfp8_gemm(q, qs, wc, sc, y, work)
            if cold:
                gemm_launch = Launch("fp8_gemm", gemm_step, (q, qs, y, work), 2 * M * N * K,
                                     gemm_bytes(M, N, K), "mfma" if c == 0 else "hbm")
            else:
                gemm_launch = Launch("fp8_gemm", bfp8.bfp8_gemm, (q, qs, w, s, y, work), 2 * M * N * K,
                                     gemm_bytes(M, N, K), "mfma" if c == 0 else "hbm")
            self.launches += [
                Launch("act_quant", bfp8.bfp8_act_quant, (x, q, qs), 0, act_quant_bytes(M, K), "hbm"),
                gemm_launch,
            ]
            self.shape = dict(M=M, N=N, K=K)
            self.dominant, self.dominant_kernel = ["fp8_gemm"], "gemm"
        elif c in (2, 3):
            M, N1, K1, N2, K2 = (wl.meta[k] for k in ("M", "N1", "K1", "N2", "K2"))
            x = t["x"].to(dev)
            w1, s1 = t["w1"].to(dev), t["s1"].to(dev)
            w2, s2 = t["w2"].to(dev), t["s2"].to(dev)
            q = torch.empty(M, K1, dtype=torch.uint8, device=dev)
            qs = torch.empty(M, K1 // BLOCK, dtype=torch.float32, device=dev)
            h = torch.empty(M, N1, dtype=torch.bfloat16, device=dev)
            qh = torch.empty(M, K2, dtype=torch.uint8, device=dev)
            qhs = torch.empty(M, K2 // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
            work1, work2 = gemm_workspace(M, N1, K1, dev), gemm_workspace(M, N2, K2, dev)
            self.launches += [
                Launch("act_quant_x", bfp8.bfp8_act_quant, (x, q, qs), 0, act_quant_bytes(M, K1), "hbm"),
                Launch("fp8_gemm_1", bfp8.bfp8_gemm, (q, qs, w1, s1, h, work1), 2 * M * N1 * K1,
                       gemm_bytes(M, N1, K1), "mfma"),
                Launch("act_quant_h", bfp8.bfp8_act_quant, (h, qh, qhs), 0, act_quant_bytes(M, K2), "hbm"),
                Launch("fp8_gemm_2", bfp8.bfp8_gemm, (qh, qhs, w2, s2, y, work2), 2 * M * N2 * K2,
                       gemm_bytes(M, N2, K2), "mfma"),
            ]
            if c == 3:
                wd = torch.empty(N1, K1, dtype=torch.bfloat16, device=dev)
                self.launches.append(Launch("weight_dequant", bfp8.bfp8_weight_dequant, (w1, s1, wd), 0,
                                            dequant_bytes(N1, K1), "hbm"))
            self.shape = dict(M=M, N1=N1, K1=K1, N2=N2, K2=K2)
            # both GEMMs run the same kernel with the same FLOP count per launch
            self.dominant, self.dominant_kernel = ["fp8_gemm_1", "fp8_gemm_2"], "gemm"
        elif c == 4:
            ids, off = t["token_ids"], t["offsets"]
            T, G, N, K = int(off[-1]), wl.meta["G"], wl.meta["N"], wl.meta["K"]
            xg = t["x"][ids].contiguous().to(dev)          # tokens already gathered in expert order
            self.hashes["x_gathered"] = sha_of(t["x"][ids])
            b, bs = t["w1"].to(dev), t["s1"].to(dev)
            off_d = off.to(dev)
            q = torch.empty(T, K, dtype=torch.uint8, device=dev)
            qs = torch.empty(T, K // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(T, N, dtype=torch.bfloat16, device=dev)
            self.launches += [
                Launch("act_quant", bfp8.bfp8_act_quant, (xg, q, qs), 0, act_quant_bytes(T, K), "hbm"),
                Launch("fp8_gemm_grouped", bfp8.bfp8_gemm_grouped, (q, qs, b, bs, y, off_d),
                       2 * T * N * K, gemm_bytes(T, N, K, G), "hbm"),
            ]
            counts = (off[1:] - off[:-1]).tolist()
            self.shape = dict(T=T, G=G, N=N, K=K, tokens_per_expert_min=min(counts),
                              tokens_per_expert_max=max(counts))
            self.dominant, self.dominant_kernel = ["fp8_gemm_grouped"], "gemm_grouped"
        elif c in ("dense-mlp", "moe-pair"):
            # the chain with act_quant of H fused into the first GEMM's epilogue (bit-identical
            # codes and scales to act_quant of the stored bf16 H); the dense MLP step also
            # dequantizes its up-projection weight
            M, N1, K1, N2, K2 = (wl.meta[k] for k in ("M", "N1", "K1", "N2", "K2"))
            x = t["x"].to(dev)
            w1, s1 = t["w1"].to(dev), t["s1"].to(dev)
            w2, s2 = t["w2"].to(dev), t["s2"].to(dev)
            q = torch.empty(M, K1, dtype=torch.uint8, device=dev)
            qs = torch.empty(M, K1 // BLOCK, dtype=torch.float32, device=dev)
            qh = torch.empty(M, K2, dtype=torch.uint8, device=dev)
            qhs = torch.empty(M, K2 // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
            work2 = gemm_workspace(M, N2, K2, dev)
            self.launches += [
                Launch("act_quant_x", bfp8.bfp8_act_quant, (x, q, qs), 0, act_quant_bytes(M, K1), "hbm"),
                Launch("fp8_gemm_1_quant", bfp8.bfp8_gemm_act_quant, (q, qs, w1, s1, qh, qhs),
                       2 * M * N1 * K1, M * K1 + N1 * K1 + M * N1 + 4 * M * (N1 // BLOCK), "mfma"),
                Launch("fp8_gemm_2", bfp8.bfp8_gemm, (qh, qhs, w2, s2, y, work2), 2 * M * N2 * K2,
                       gemm_bytes(M, N2, K2), "mfma"),
            ]
            if c == "dense-mlp":
                wd = torch.empty(N1, K1, dtype=torch.bfloat16, device=dev)
                self.launches.append(Launch("weight_dequant", bfp8.bfp8_weight_dequant, (w1, s1, wd), 0,
                                            dequant_bytes(N1, K1), "hbm"))
            self.shape = dict(M=M, N1=N1, K1=K1, N2=N2, K2=K2)
            self.dominant, self.dominant_kernel = ["fp8_gemm_1_quant", "fp8_gemm_2"], "gemm"
        elif c == "expert-ffn":
            # one routed expert's gated FFN: act_quant(x) -> [w1; w3] GEMM with silu(g) * u and
            # act_quant in the epilogue -> w2 GEMM
            M, N1, K1, N2, K2 = (wl.meta[k] for k in ("M", "N1", "K1", "N2", "K2"))
            x = t["x"].to(dev)
            w13, s13 = bfp8.interleave_w13(t["w1"], t["s1"], t["w3"], t["s3"])
            w13, s13 = w13.to(dev), s13.to(dev)
            w2, s2 = t["w2"].to(dev), t["s2"].to(dev)
            q = torch.empty(M, K1, dtype=torch.uint8, device=dev)
            qs = torch.empty(M, K1 // BLOCK, dtype=torch.float32, device=dev)
            qh = torch.empty(M, K2, dtype=torch.uint8, device=dev)
            qhs = torch.empty(M, K2 // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
            self.launches += [
                Launch("act_quant_x", bfp8.bfp8_act_quant, (x, q, qs), 0, act_quant_bytes(M, K1), "hbm"),
                Launch("fp8_gemm_w13_swiglu_quant", bfp8.bfp8_gemm_swiglu_act_quant, (q, qs, w13, s13, qh, qhs),
                       2 * M * 2 * N1 * K1, M * K1 + 2 * N1 * K1 + M * N1 + 4 * M * (N1 // BLOCK), "mfma"),
                Launch("fp8_gemm_w2", bfp8.bfp8_gemm, (qh, qhs, w2, s2, y), 2 * M * N2 * K2,
                       gemm_bytes(M, N2, K2), "mfma"),
            ]
            self.shape = dict(M=M, N_gate_up=2 * N1, N_out=N1, K1=K1, N2=N2, K2=K2, activation="silu (stated reading)")
            self.dominant, self.dominant_kernel = ["fp8_gemm_w13_swiglu_quant"], "gemm"
        elif c == "dense-mlp-ue8m0":
            # the dense chain with power-of-two scales (weights re-drawn from the same seeds with
            # their block scales rounded to powers of two), scales applied by the MFMA
            M, N1, K1, N2, K2 = (wl.meta[k] for k in ("M", "N1", "K1", "N2", "K2"))
            w1, s1 = synth.weight(N1, K1, synth.seed_of(3, 1), synth.seed_of(3, 2), pow2=True)
            w2, s2 = synth.weight(N2, K2, synth.seed_of(3, 3), synth.seed_of(3, 4), pow2=True)
            self.hashes.update(w1_pow2=sha_of(w1), s1_pow2=sha_of(s1), w2_pow2=sha_of(w2), s2_pow2=sha_of(s2))
            x = t["x"].to(dev)
            w1, s1, w2, s2 = w1.to(dev), s1.to(dev), w2.to(dev), s2.to(dev)
            q = torch.empty(M, K1, dtype=torch.uint8, device=dev)
            qs = torch.empty(M, K1 // BLOCK, dtype=torch.float32, device=dev)
            h = torch.empty(M, N1, dtype=torch.bfloat16, device=dev)
            qh = torch.empty(M, K2, dtype=torch.uint8, device=dev)
            qhs = torch.empty(M, K2 // BLOCK, dtype=torch.float32, device=dev)
            y = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
            # the down GEMM's half-full last round split over K, as in the fp8 step
            n_ws = bfp8.bfp8_gemm_ue8m0_workspace_size(M, N2, K2)
            ws2 = torch.empty(max(1, n_ws // 4), dtype=torch.float32, device=dev) if n_ws else None
            self.launches += [
                Launch("act_quant_ue8m0_x", bfp8.bfp8_act_quant_ue8m0, (x, q, qs), 0,
                       act_quant_bytes(M, K1), "hbm"),
                Launch("fp8_gemm_ue8m0_1", bfp8.bfp8_gemm_ue8m0, (q, qs, w1, s1, h), 2 * M * N1 * K1,
                       gemm_bytes(M, N1, K1), "mfma"),
                Launch("act_quant_ue8m0_h", bfp8.bfp8_act_quant_ue8m0, (h, qh, qhs), 0,
                       act_quant_bytes(M, K2), "hbm"),
                Launch("fp8_gemm_ue8m0_2", bfp8.bfp8_gemm_ue8m0, (qh, qhs, w2, s2, y, ws2), 2 * M * N2 * K2,
                       gemm_bytes(M, N2, K2), "mfma"),
            ]
            self.shape = dict(M=M, N1=N1, K1=K1, N2=N2, K2=K2, scales="powers of two (e8m0)")
            self.dominant, self.dominant_kernel = ["fp8_gemm_ue8m0_1", "fp8_gemm_ue8m0_2"], "gemm_ue8m0"
        elif c == "bf16-branch":
            M, N1, K1, N2, K2 = (wl.meta[k] for k in ("M", "N1", "K1", "N2", "K2"))
            x = t["x"].to(dev)
            w1, s1 = t["w1"].to(dev), t["s1"].to(dev)
            w2, s2 = t["w2"].to(dev), t["s2"].to(dev)
            w1d = torch.empty(N1, K1, dtype=torch.bfloat16, device=dev)
            w2d = torch.empty(N2, K2, dtype=torch.bfloat16, device=dev)
            h = torch.empty(M, N1, dtype=torch.bfloat16, device=dev)
            y = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
            # the down GEMM's half-full last round split over K, as in the fp8 step
            n_ws = bfp8.bfp8_gemm_bf16_workspace_size(M, N2, K2)
            ws2 = torch.empty(max(1, n_ws // 4), dtype=torch.float32, device=dev) if n_ws else None
            self.launches += [
                Launch("weight_dequant_1", bfp8.bfp8_weight_dequant, (w1, s1, w1d), 0,
                       dequant_bytes(N1, K1), "hbm"),
                Launch("bf16_gemm_1", bfp8.bfp8_gemm_bf16, (x, w1d, h), 2 * M * N1 * K1,
                       2 * M * K1 + 2 * N1 * K1 + 2 * M * N1, "mfma_bf16"),
                Launch("weight_dequant_2", bfp8.bfp8_weight_dequant, (w2, s2, w2d), 0,
                       dequant_bytes(N2, K2), "hbm"),
                Launch("bf16_gemm_2", bfp8.bfp8_gemm_bf16, (h, w2d, y, ws2), 2 * M * N2 * K2,
                       2 * M * K2 + 2 * N2 * K2 + 2 * M * N2, "mfma_bf16"),
            ]
            self.shape = dict(M=M, N1=N1, K1=K1, N2=N2, K2=K2)
            self.dominant, self.dominant_kernel = ["bf16_gemm_1", "bf16_gemm_2"], "gemm_bf16"
        elif c == "moe-layer":
            topk, wts, off = t["topk"], t["weights"], t["offsets"]
            Tt, k = topk.shape
            rows, G, N, K = int(off[-1]), wl.meta["G"], wl.meta["N"], wl.meta["K"]
            cap = Tt * k                                     # worst case: every slot local
            x = t["x"].to(dev)
            topk_d, w_d = topk.to(dev), wts.to(dev)
            b, bs = t["w1"].to(dev), t["s1"].to(dev)
            off_d = torch.empty(G + 1, dtype=torch.int32, device=dev)
            row_token = torch.empty(cap, dtype=torch.int32, device=dev)
            slot_row = torch.empty(Tt, k, dtype=torch.int32, device=dev)
            ws = torch.empty(max(1, bfp8.bfp8_moe_dispatch_workspace_size(Tt, k, G) // 4),
                             dtype=torch.int32, device=dev)
            q = torch.empty(cap, K, dtype=torch.uint8, device=dev)
            qs = torch.empty(cap, K // BLOCK, dtype=torch.float32, device=dev)
            h = torch.empty(cap, N, dtype=torch.bfloat16, device=dev)
            y = torch.empty(Tt, N, dtype=torch.bfloat16, device=dev)
            nrows = off_d[G:]
            self.launches += [
                Launch("moe_dispatch", lambda topk_d, off_d, rt, sr, ws: bfp8.bfp8_moe_dispatch(topk_d, 0, off_d, rt, sr, ws),
                       (topk_d, off_d, row_token, slot_row, ws), 0, dispatch_bytes(Tt, k, rows, G), "hbm"),
                Launch("act_quant_rows", bfp8.bfp8_act_quant_rows, (x, row_token, nrows, q, qs),
                       0, act_quant_bytes(rows, K) + 4 * rows, "hbm"),
                Launch("fp8_gemm_grouped", bfp8.bfp8_gemm_grouped, (q, qs, b, bs, h, off_d),
                       2 * rows * N * K, gemm_bytes(rows, N, K, G), "hbm"),
                Launch("moe_combine", bfp8.bfp8_moe_combine, (h, slot_row, w_d, y),
                       0, combine_bytes(Tt, k, rows, N), "hbm"),
            ]
            counts = (off[1:] - off[:-1]).tolist()
            self.shape = dict(tokens=Tt, top_k=k, local_experts=G, rows=rows, row_capacity=cap,
                              N=N, K=K, tokens_per_expert_min=min(counts),
                              tokens_per_expert_max=max(counts))
            self.dominant, self.dominant_kernel = ["fp8_gemm_grouped"], "gemm_grouped"
        else:
            raise ValueError(c)

    def run(self, events=None):
        for i, launch in enumerate(self.launches):
            if events is not None:
                events[i].record()
            launch()
        if events is not None:
            events[len(self.launches)].record()


# ------------------------------------------------------------------ CPU oracle leg

def cpu_baseline(wl, target_s=12.0, kind=None):
    """Time the CPU oracle on a proportional sample of one step: a fraction f of the
    rows of every stage (activation rows, and weight rows for dequant)."""
    import oracle

    threads = min(oracle.default_threads(), int(os.environ.get("OMP_NUM_THREADS", "1024")))
    t = wl.tensors
    c = wl.config
    x_bits = t["x"].contiguous().view(torch.int16).numpy().view(np.uint16)

    def run(rows):
        done = 0.0
        t0 = time.perf_counter()
        if kind == "bf16-branch":
            # the weights are dequantized whole (a fixed cost), the GEMMs on the sampled rows
            w1d = oracle.weight_dequant(t["w1"].numpy(), t["s1"].numpy())
            h = oracle.gemm_bf16(x_bits, w1d, rows=np.arange(rows), threads=threads)
            hb = oracle.f32_to_bf16(h.astype(np.float32))
            w2d = oracle.weight_dequant(t["w2"].numpy(), t["s2"].numpy())
            oracle.gemm_bf16(hb, w2d, threads=threads)
            done = 2.0 * rows * (wl.meta["N1"] * wl.meta["K1"] + wl.meta["N2"] * wl.meta["K2"])
        elif c in (0, 1):
            q, s = oracle.act_quant(x_bits[:rows])
            oracle.gemm(q, s, t["w1"].numpy(), t["s1"].numpy(), threads=threads)
            done = 2.0 * rows * wl.meta["N"] * wl.meta["K"]
        elif c in (2, 3):
            q, s = oracle.act_quant(x_bits[:rows])
            h = oracle.gemm(q, s, t["w1"].numpy(), t["s1"].numpy(), threads=threads)
            hb = oracle.f32_to_bf16(h.astype(np.float32))
            qh, sh = oracle.act_quant(hb)
            oracle.gemm(qh, sh, t["w2"].numpy(), t["s2"].numpy(), threads=threads)
            done = 2.0 * rows * (wl.meta["N1"] * wl.meta["K1"] + wl.meta["N2"] * wl.meta["K2"])
            if c == 3:
                wrows = max(1, int(round(t["w1"].shape[0] * rows / wl.meta["M"])))
                oracle.weight_dequant(t["w1"].numpy()[:wrows], t["s1"].numpy()[:-(-wrows // BLOCK)])
        elif kind == "moe-layer":
            # rows = sampled tokens: dispatch of the whole batch, then every later stage
            # for the sampled tokens' local slots only
            G = wl.meta["G"]
            off, rt, sr = oracle.moe_dispatch(t["topk"].numpy(), 0, G)
            mine = np.unique(sr[:rows][sr[:rows] >= 0])
            q, s = oracle.act_quant(x_bits[rt[mine]])
            grp = np.searchsorted(off, mine, side="right") - 1
            c_off = np.concatenate([[0], np.cumsum(np.bincount(grp, minlength=G))]).astype(np.int32)
            h = oracle.gemm_grouped(q, s, t["w1"].numpy(), t["s1"].numpy(), c_off, threads=threads)
            pos = np.full(int(off[-1]), -1, np.int64)
            pos[mine] = np.arange(mine.size)
            sub = np.where(sr[:rows] >= 0, pos[np.maximum(sr[:rows], 0)], -1).astype(np.int32)
            oracle.moe_combine(oracle.f32_to_bf16(h.astype(np.float32)), sub, t["weights"].numpy()[:rows])
            done = 2.0 * mine.size * wl.meta["N"] * wl.meta["K"]
        else:
            ids, off = t["token_ids"].numpy(), t["offsets"].numpy()
            xg = x_bits[ids[:rows]]
            q, s = oracle.act_quant(xg)
            full_q = np.zeros((int(off[-1]), q.shape[1]), np.uint8)
            full_s = np.ones((int(off[-1]), s.shape[1]), np.float32)
            full_q[:rows], full_s[:rows] = q, s
            oracle.gemm_grouped(full_q, full_s, t["w1"].numpy(), t["s1"].numpy(), off,
                                rows=np.arange(rows), threads=threads)
            done = 2.0 * rows * wl.meta["N"] * wl.meta["K"]
        return time.perf_counter() - t0, done

    M = wl.meta["tokens"] if kind == "moe-layer" else wl.meta.get("M", wl.meta.get("T"))
    probe = min(M, max(1, threads))
    dt, _ = run(probe)
    rows = int(min(M, max(probe, probe * target_s / max(dt, 1e-6))))
    dt, flop = run(rows)
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{rows} of {M} {'tokens' if kind == 'moe-layer' else 'rows'} of every stage "
                       f"of one step ({dt:.1f} s of CPU work)")}


# ------------------------------------------------------------------ traffic

def read_traffic(kernel_name, workload):
    """HBM bytes per launch measured by rocprofv3 counters on this workload, if the kernel
    source is unchanged since (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("workload") != workload:
        return None
    src = os.path.join(ROOT, "block_scaled_fp8_04_amd", "csrc", kv.get("source", "gemm.hip"))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv.get("source_sha256"):
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ clock and power

class ClockSampler:
    """Samples the GPU's shader clock and socket power from sysfs every few ms while
    active: the level marked current in pp_dpm_sclk (as the driver reports it), and hwmon
    power1_average (else power1_input); the board power cap from hwmon power1_cap.
    Reading sysfs costs the GPU nothing; fields are None where a file is absent."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        self.sclk_path = self.power_path = self.cap_path = None
        for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
            if os.path.exists(os.path.join(dev_dir, "pp_dpm_sclk")):
                self.sclk_path = os.path.join(dev_dir, "pp_dpm_sclk")
                for name in ("power1_average", "power1_input"):
                    hits = sorted(glob.glob(os.path.join(dev_dir, "hwmon", "hwmon*", name)))
                    if hits:
                        self.power_path = hits[0]
                        break
                caps = sorted(glob.glob(os.path.join(dev_dir, "hwmon", "hwmon*", "power1_cap")))
                self.cap_path = caps[0] if caps else None
                break
        self.period = period_s
        self.sclk, self.power = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def _sample(self):
        text = self._read(self.sclk_path) if self.sclk_path else None
        if text:
            for line in text.splitlines():
                if line.rstrip().endswith("*"):
                    digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                    if digits:
                        self.sclk.append(int(digits))
        text = self._read(self.power_path) if self.power_path else None
        if text and text.strip().isdigit():
            self.power.append(int(text.strip()) / 1e6)

    def _loop(self):
        while not self._stop.is_set():
            self._sample()
            self._stop.wait(self.period)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join()
        cap = self._read(self.cap_path) if self.cap_path else None
        return {"sclk_mhz_median": float(np.median(self.sclk)) if self.sclk else None,
                "sclk_mhz_range": [min(self.sclk), max(self.sclk)] if self.sclk else None,
                "socket_power_w_median": float(np.median(self.power)) if self.power else None,
                "power_cap_w": int(cap.strip()) / 1e6 if cap and cap.strip().isdigit() else None,
                "samples": len(self.sclk), "source": "sysfs pp_dpm_sclk (current level), hwmon power1",
                "window": "warmup, timed steps and the isolated per-kernel timing"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ------------------------------------------------------------------ isolated timing

def time_isolated(launches, est_us, rounds=5, min_round_ms=2.0):
    """Per-launch duration of `launches` (copies of one launch, called in turn), timed as
    `rounds` rounds of back-to-back calls between one event pair; returns the median and
    min over the rounds of the mean duration per call, in us."""
    n = len(launches)
    reps = max(n, int(np.ceil(min_round_ms * 1e3 / max(est_us, 1.0))))
    reps = -(-reps // n) * n
    per_call = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            launches[r % n]()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / reps)
    return {"median_us": float(np.median(per_call)), "min_us": float(min(per_call)),
            "rounds": rounds, "launches_per_round": reps}


def rates(entry, us):
    """TFLOP/s, GB/s and roofline fraction of a launch that takes `us`."""
    out = {"gbs": entry["bytes"] / (us * 1e-6) / 1e9}
    if entry["flop"]:
        out["tflops"] = entry["flop"] / (us * 1e-6) / 1e12
    if entry["bound"] == "mfma":
        out["frac"] = out["tflops"] / PEAK_FP8_TFLOPS
    elif entry["bound"] == "mfma_bf16":
        out["frac"] = out["tflops"] / PEAK_BF16_TFLOPS
    else:
        out["frac"] = out["gbs"] / PEAK_HBM_GBS
    return out


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="dense-mlp")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as replays of one captured HIP graph (launch-bound shapes); "
                         "the per-kernel table still comes from an eager pass with events")
    ap.add_argument("--cold", action="store_true",
                    help="decode: rotate over weight copies totalling > 512 MB so every step "
                         "reads its weight from HBM (eager launches only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stream-calibration", action="store_true",
                    help="only time plain device copies of 1 GiB (read + write, cycling over three buffer "
                         "pairs, so no copy finds its data in the Infinity Cache) and exit: the streaming "
                         "rate this box reaches, the practical ceiling of the HBM-bound kernels")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the per-kernel isolated (warm / cold) timing after the timed region "
                         "(profiler runs: every launch then belongs to the timed steps)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy three times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X "
              "(sharding across GPUs is described, not measured). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.cold and (args.workload != "decode" or args.graph):
        sys.exit("--cold applies to the decode workload with eager launches")
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 512 * 1024 * 1024
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3, "copy_ms": ms,
                          "copy_gbs": 2 * n / (ms * 1e-3) / 1e9}), flush=True)
        return
    if args.stream_calibration:
        n = 1 << 30
        pairs = [(torch.full((n,), i + 1, dtype=torch.uint8, device=dev),
                  torch.empty(n, dtype=torch.uint8, device=dev)) for i in range(3)]
        for i in range(3):
            pairs[i][1].copy_(pairs[i][0])
        torch.cuda.synchronize()
        times = []
        for r in range(9):
            src, dst = pairs[r % 3]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        print(json.dumps({"stream_calibration": "torch copy of 1 GiB, 3 rotating buffer pairs",
                          "bytes_moved": 2 * n, "copy_ms_median": ms,
                          "copy_gbs_median": 2 * n / (ms * 1e-3) / 1e9,
                          "copy_gbs_best": 2 * n / (min(times) * 1e-3) / 1e9}), flush=True)
        return
    bfp8.library()

    t0 = time.time()
    wl = synth.make(WORKLOADS[args.workload])
    step = Step(wl, dev, args.workload, cold=args.cold)
    gen_s = time.time() - t0
    print(f"# workload {wl.name}: inputs built in {gen_s:.1f}s; launches "
          f"{[l.name for l in step.launches]}", file=sys.stderr, flush=True)

    nl = len(step.launches)
    sampler = ClockSampler().start()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step.run(events[k])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps

    kernels = {}
    for i, launch in enumerate(step.launches):
        per = [events[k][i].elapsed_time(events[k][i + 1]) * 1e3 for k in range(args.steps)]
        entry = {"avg_us": float(np.mean(per)), "median_us": float(np.median(per)),
                 "min_us": float(min(per)), "flop": launch.flop, "bytes": launch.bytes,
                 "bound": launch.bound}
        entry.update(rates(entry, entry["avg_us"]))
        kernels[launch.name] = entry

    # each launch alone, after the timed region: back-to-back rounds on the same buffers
    # (warm), and for the HBM-bound ones over copies of their buffers totalling > 1 GB
    # (cold: no launch finds its data in the Infinity Cache or L2)
    if not args.cold and not args.no_isolated:
        for launch in step.launches:
            entry = kernels[launch.name]
            iso = time_isolated([launch], entry["avg_us"])
            iso.update({k: v for k, v in rates(entry, iso["median_us"]).items()})
            entry["isolated_warm"] = iso
            if launch.bound == "hbm" and launch.footprint() > 0:
                n_copies = int(min(16, max(2, -(-(1 << 30) // launch.footprint()))))
                copies = launch.copies(n_copies)
                torch.cuda.synchronize()
                iso = time_isolated(copies, entry["avg_us"])
                iso.update({k: v for k, v in rates(entry, iso["median_us"]).items()})
                iso["buffer_copies"] = n_copies
                entry["isolated_cold"] = iso
                del copies
                torch.cuda.empty_cache()
    clock = sampler.stop()

    launch_mode = "eager"
    if args.graph:
        # the K timed steps captured into one graph (the library only enqueues
        # kernels on the current stream, with no allocation or memset), so the
        # host's cost of a replay is not paid per step; warmup replays the same
        # graph, then one timed replay runs exactly K steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step.run()
        for _ in range(max(1, -(-args.warmup // args.steps))):
            graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
        launch_mode = f"hip-graph replay ({args.steps} steps in one graph)"

    gemm_flop = sum(l.flop for l in step.launches)
    value = gemm_flop / (ms_per_step * 1e-3) / 1e12

    # dominant kernel: the launches of the kernel that takes most of the step
    dom = step.dominant
    avg_us = float(np.mean([kernels[n]["avg_us"] for n in dom]))
    d = kernels[dom[0]]
    traffic = read_traffic(step.dominant_kernel, args.workload)
    if d["bound"] in ("mfma", "mfma_bf16"):
        peak = PEAK_FP8_TFLOPS if d["bound"] == "mfma" else PEAK_BF16_TFLOPS
        ach = d["flop"] / (avg_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "traffic": traffic, "kernel": step.dominant_kernel,
                "launches": dom, "avg_us": avg_us}
    else:
        nbytes = float(np.mean([kernels[n]["bytes"] for n in dom]))
        ach = nbytes / (avg_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "kernel": step.dominant_kernel,
                "launches": dom, "avg_us": avg_us}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, args.workload)

    wl_name = (f"{args.workload}-{wl.name}"
               if args.workload in ("moe-layer", "bf16-branch", "dense-mlp-unfused", "expert-ffn",
                                    "dense-mlp-ue8m0", "moe-pair-unfused") else wl.name)
    config = {"workload": wl_name, "shape": step.shape,
              "step": " -> ".join(l.name for l in step.launches),
              "value_definition": "GEMM FLOP per step / wall time per step",
              "input_sha256_16": step.hashes, "seeds": "1000*config+tensor_id",
              "parallelism": "single-gpu", "launch": launch_mode,
              "caches": "cold (weight copies > 512 MB rotated)" if args.cold else "no flush between steps"}
    dtype = ("bf16 (fp32 accumulate, bf16 out; fp8_e4m3 weights dequantized)"
             if args.workload == "bf16-branch" else "fp8_e4m3 (fp32 accumulate, bf16 out)")
    out = {"metric": "block-FP8 GEMM TFLOP/s & % of fp8 MFMA peak; act_quant/dequant HBM GB/s",
           "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic (seeded; DeepSeek-V3 projection shapes, random-init)",
           "config": config, "kernels": kernels, "roofline": roof, "clock": clock,
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
