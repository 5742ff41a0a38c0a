"""The library's calls inside a captured HIP graph: the decode-shaped linear (act_quant and
the split-K GEMM over a caller workspace, and the same as one bfp8_linear_fp8 call) and the
MoE chain are captured once and replayed
several times, with eager work and synchronizations in between; every replay must equal the
eager result bit for bit (the kernels are deterministic and enqueue no memset or allocation).
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_04_amd as bfp8
from gpu_helpers import announce, dev, workload

pytestmark = pytest.mark.gpu


def test_decode_linear_graph_replays():
    wl = workload(1)
    x = wl.tensors["x"].to(dev())
    w, s = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    M, K = x.shape
    N = w.shape[0]
    ws = torch.empty(max(1, bfp8.bfp8_gemm_workspace_size(M, N, K) // 4), dtype=torch.float32, device=dev())
    q = torch.empty(M, K, dtype=torch.uint8, device=dev())
    qs = torch.empty(M, K // 128, dtype=torch.float32, device=dev())
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev())

    def step():
        bfp8.bfp8_act_quant(x, q, qs)
        bfp8.bfp8_gemm(q, qs, w, s, y, ws)

    step()
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        y.zero_()
        ws.fill_(float("nan"))                     # stale workspace must not leak into the result
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        announce(f"decode graph replay {r}")
        assert torch.equal(y, ref), f"replay {r} differs from the eager result"
        _ = (x.float() * 2).sum()                  # eager work between replays
        torch.cuda.synchronize()


def test_linear_fp8_graph_replays():
    """bfp8_linear_fp8 (act_quant into its workspace, then the split-K GEMM) captured once."""
    wl = workload(1)
    x = wl.tensors["x"].to(dev())
    w, s = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    M, K = x.shape
    N = w.shape[0]
    work = bfp8.linear_workspace(M, N, K, dev())
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    bfp8.bfp8_linear_fp8(x, w, s, y, work)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bfp8.bfp8_linear_fp8(x, w, s, y, work)
    for r in range(4):
        y.zero_()
        work.fill_(0xFF)                           # stale workspace must not leak into the result
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        announce(f"linear_fp8 graph replay {r}")
        assert torch.equal(y, ref), f"replay {r} differs from the eager result"
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()


def test_moe_chain_graph_replays():
    wl = workload(4, 0.25)
    x, topk, wts = wl.tensors["x"].to(dev()), wl.tensors["topk"].to(dev()), wl.tensors["weights"].to(dev())
    W, S = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    T, k = topk.shape
    G, N, K = W.shape
    cap = T * k
    off = torch.empty(G + 1, dtype=torch.int32, device=dev())
    row_token = torch.empty(cap, dtype=torch.int32, device=dev())
    slot_row = torch.empty(T, k, dtype=torch.int32, device=dev())
    dws = torch.empty(max(1, bfp8.bfp8_moe_dispatch_workspace_size(T, k, G) // 4), dtype=torch.int32, device=dev())
    q = torch.empty(cap, K, dtype=torch.uint8, device=dev())
    qs = torch.empty(cap, K // 128, dtype=torch.float32, device=dev())
    h = torch.empty(cap, N, dtype=torch.bfloat16, device=dev())
    y = torch.empty(T, N, dtype=torch.bfloat16, device=dev())

    def step():
        bfp8.bfp8_moe_dispatch(topk, 0, off, row_token, slot_row, dws)
        bfp8.bfp8_act_quant_rows(x, row_token, off[G:], q, qs)
        bfp8.bfp8_gemm_grouped(q, qs, W, S, h, off)
        bfp8.bfp8_moe_combine(h, slot_row, wts, y)

    step()
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        y.zero_()
        off.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        announce(f"moe graph replay {r}")
        assert torch.equal(y, ref), f"replay {r} differs from the eager result"


def test_split_last_round_graph_replays():
    """The three GEMM forms with a split last round (main tiles, the two K halves of the
    tail columns into the workspace, the ordered reduction) captured once; each replay equals
    the eager result bit for bit, the workspace filled with NaN between replays."""
    from block_scaled_fp8_04_amd import synth
    M, N, K = 2048, 8448, 10368
    g = torch.Generator().manual_seed(91)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    q, qs = bfp8.act_quant(x)
    qe, qes = bfp8.act_quant_ue8m0(x)
    w, ws = synth.weight(N, K, 92, 93)
    wp, wps = synth.weight(N, K, 94, 95, pow2=True)
    w, ws, wp, wps = w.to(dev()), ws.to(dev()), wp.to(dev()), wps.to(dev())
    wd = bfp8.weight_dequant(w, ws)
    need = max(bfp8.bfp8_gemm_workspace_size(M, N, K), bfp8.bfp8_gemm_ue8m0_workspace_size(M, N, K),
               bfp8.bfp8_gemm_bf16_workspace_size(M, N, K))
    assert need > 0
    work = torch.empty(need // 4, dtype=torch.float32, device=dev())
    y1 = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    y2 = torch.empty_like(y1)
    y3 = torch.empty_like(y1)

    def step():
        bfp8.bfp8_gemm(q, qs, w, ws, y1, work)
        bfp8.bfp8_gemm_ue8m0(qe, qes, wp, wps, y2, work)
        bfp8.bfp8_gemm_bf16(x, wd, y3, work)

    step()
    torch.cuda.synchronize()
    refs = [y1.clone(), y2.clone(), y3.clone()]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for r in range(3):
        for y in (y1, y2, y3):
            y.zero_()
        work.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        announce(f"split last round graph replay {r}")
        for name, y, ref in zip(("fp8", "e8m0", "bf16"), (y1, y2, y3), refs):
            assert torch.equal(y, ref), f"replay {r}: the {name} GEMM differs from the eager result"
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()


def test_split_schedule_graph_replays():
    """The 256 x 256 tile's split load schedule (whole M tiles, even K-block count) captured
    once: the bf16 GEMM, the GEMM with act_quant fused, and a GEMM whose split last round
    runs the schedule on both launches of tiles; every replay equals the eager result."""
    from block_scaled_fp8_04_amd import synth
    g = torch.Generator().manual_seed(97)
    M, N, K = 2048, 5120, 7168
    M2, N2, K2 = 2048, 10240, 10240
    x = torch.randn(M2, max(K, K2), generator=g).to(torch.bfloat16).to(dev())
    q, qs = bfp8.act_quant(x[:, :K].contiguous())
    q2, qs2 = bfp8.act_quant(x[:, :K2].contiguous())
    w, ws = (t.to(dev()) for t in synth.weight(N, K, 98, 99))
    w2, ws2 = (t.to(dev()) for t in synth.weight(N2, K2, 100, 101))
    need = bfp8.bfp8_gemm_workspace_size(M2, N2, K2)
    assert need > 0
    work = torch.empty(need // 4, dtype=torch.float32, device=dev())
    y1 = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    y2 = torch.empty(M2, N2, dtype=torch.bfloat16, device=dev())
    yq = torch.empty(M, N, dtype=torch.uint8, device=dev())
    yqs = torch.empty(M, N // 128, dtype=torch.float32, device=dev())

    def step():
        bfp8.bfp8_gemm(q[:M], qs[:M], w, ws, y1, None)
        bfp8.bfp8_gemm_act_quant(q[:M], qs[:M], w, ws, yq, yqs)
        bfp8.bfp8_gemm(q2, qs2, w2, ws2, y2, work)

    step()
    torch.cuda.synchronize()
    refs = [y1.clone(), y2.clone(), yq.clone(), yqs.clone()]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for r in range(3):
        y1.zero_(); y2.zero_(); yq.zero_(); yqs.zero_()
        work.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        announce(f"split schedule graph replay {r}")
        for name, t, ref in zip(("bf16", "split last round", "codes", "scales"), (y1, y2, yq, yqs), refs):
            assert torch.equal(t, ref), f"replay {r}: {name} differ from the eager result"
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()
