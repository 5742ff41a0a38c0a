"""GPU parity of the fp8 GEMM with act_quant fused into its epilogue.

Three checks per case:
  * consistency: the fused kernel's codes and scales equal bfp8_act_quant of
    bfp8_gemm's bf16 output, bit for bit (both on the GPU; the fused epilogue
    rounds to bf16 first exactly as the stored output is rounded);
  * stage-wise parity: the oracle's act_quant of the GPU's own bf16 GEMM
    output equals the fused codes and scales bit for bit, on every checked
    row (the chain's act_quant of the first GEMM's output is exact given that
    output);
  * parity with the oracle on sampled rows: the dequantized codes
    deq(q) * s approximate the oracle's fp64 product C within the GEMM
    tolerance plus what the bf16 rounding and the e4m3 quantization may add:
        |deq - C| <= tol_gemm + 2^-8 |C| + 2^-4 (|C| + tol_gemm) + 2^-10 s,
    (half an e4m3 ulp is at most 2^-4 of a normal value and 2^-10 s in the
    subnormal range), and the scales match max(amax, 1e-4) / 448 of the
    oracle's row blocks within the same GEMM tolerance on the block maximum.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import GEMM_REL, GEMM_RMS, announce, bits16, dev, gemm_check, sample_rows, u8, workload

pytestmark = pytest.mark.gpu
BLOCK = 128


def _e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _check(q, qs, ref, what):
    """q uint8 [r, N], qs [r, N/128] (numpy) against the oracle's fp64 rows ref [r, N]."""
    vals = _e4m3_values()
    deq = vals[q] * np.repeat(qs.astype(np.float64), BLOCK, axis=1)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    tol = GEMM_REL * np.abs(ref) + GEMM_RMS * rms
    s_col = np.repeat(qs.astype(np.float64), BLOCK, axis=1)
    bound = tol + 2.0 ** -8 * np.abs(ref) + 2.0 ** -4 * (np.abs(ref) + tol) + 2.0 ** -10 * s_col
    err = np.abs(deq - ref)
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements outside the bound"
    amax = np.abs(ref).reshape(ref.shape[0], -1, BLOCK).max(axis=2)
    tol_a = (GEMM_REL + 2.0 ** -8) * amax + GEMM_RMS * rms
    s_ref = np.maximum(amax, 1e-4) / 448.0
    assert np.all(np.abs(qs - s_ref) <= tol_a / 448.0 + 1e-12), f"{what}: scales outside tolerance"
    announce(f"{what}: worst err/bound {float(np.max(err / bound)):.3f}")


def _case(q_a, s_a, w, s_w, what, rows=None):
    M, N = q_a.shape[0], w.shape[0]
    announce(f"gemm_act_quant {what} M={M} N={N} K={q_a.shape[1]} via {bfp8.bfp8_gemm_kernel_name(M, N, q_a.shape[1])}")
    q = torch.full((M, N), 0x33, dtype=torch.uint8, device=dev())
    qs = torch.full((M, N // BLOCK), -1.0, dtype=torch.float32, device=dev())
    bfp8.bfp8_gemm_act_quant(q_a, s_a, w, s_w, q, qs)
    c = bfp8.gemm(q_a, s_a, w, s_w)
    q2, qs2 = bfp8.act_quant(c)
    torch.cuda.synchronize()
    assert torch.equal(q, q2), f"{what}: codes differ from act_quant(gemm)"
    assert torch.equal(qs, qs2), f"{what}: scales differ from act_quant(gemm)"
    r = np.arange(M) if rows is None else rows
    rt = torch.from_numpy(np.asarray(r)).to(dev())
    # stage-wise: the oracle's act_quant of the GPU's own bf16 output, row by row
    qo, so = oracle.act_quant(bits16(c[rt]))
    assert np.array_equal(qo, u8(q[rt])), f"{what}: codes differ from the oracle's act_quant of C"
    assert np.array_equal(so, qs[rt].cpu().numpy()), f"{what}: scales differ from the oracle's act_quant of C"
    ref = oracle.gemm(u8(q_a), s_a.cpu().numpy(), u8(w), s_w.cpu().numpy(), rows=r)
    _check(u8(q[rt]), qs[rt].cpu().numpy(), ref, what)
    return q, qs


def test_fused_quant_shapes():
    g = torch.Generator().manual_seed(61)
    for i, (M, N, K) in enumerate([(16, 256, 256), (1, 128, 128), (130, 384, 384), (300, 1280, 256),
                                    (2000, 4096, 256), (4100, 8192, 128), (257, 640, 512)]):
        x = (torch.randn(M, K, generator=g) * (1 + i)).to(torch.bfloat16).to(dev())
        q_a, s_a = bfp8.act_quant(x)
        w, s_w = synth.weight(N, K, 620 + i, 640 + i)
        rows = None if M <= 300 else sample_rows(M, 16, 660 + i)
        _case(q_a, s_a, w.to(dev()), s_w.to(dev()), f"shape {i}", rows)


def test_fused_quant_zero_rows():
    """A zero activation row gives a zero output row: codes 0 and the floor scale."""
    K, N = 256, 512
    x = torch.randn(64, K).to(torch.bfloat16)
    x[5] = 0
    q_a, s_a = bfp8.act_quant(x.to(dev()))
    w, s_w = synth.weight(N, K, 670, 671)
    q, qs = bfp8.gemm_act_quant(q_a, s_a, w.to(dev()), s_w.to(dev()))
    torch.cuda.synchronize()
    assert torch.all(q[5] == 0)
    assert torch.all(qs[5] == torch.tensor(1e-4, dtype=torch.float32) / 448.0)


def test_fused_quant_dense_chain_full_size():
    """The dense MLP up projection with H quantized in the epilogue, then the down GEMM on it.

    Rows: the first and last of every 128-row block plus seeded ones.  The down GEMM
    8192 x 7168 x 18432 runs on the fused codes and scales, and its output is held to
    the GEMM tolerance against the oracle's fp64 product of those same codes."""
    wl = workload(3)
    x = wl.tensors["x"].to(dev())
    w1, s1 = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    w2, s2 = wl.tensors["w2"].to(dev()), wl.tensors["s2"].to(dev())
    q_a, s_a = bfp8.act_quant(x)
    rows = sample_rows(8192, 16, 680)
    qh, qhs = _case(q_a, s_a, w1, s1, "dense-mlp up 8192x18432x7168", rows)
    M, N2, K2 = 8192, w2.shape[0], w2.shape[1]
    need = bfp8.bfp8_gemm_workspace_size(M, N2, K2)
    work = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev()) if need else None
    y = bfp8.gemm(qh, qhs, w2, s2, workspace=work)
    torch.cuda.synchronize()
    rt = torch.from_numpy(rows).to(dev())
    ref = oracle.gemm(u8(qh[rt]), qhs[rt].cpu().numpy(), u8(w2), s2.cpu().numpy())
    worst = gemm_check(y[rt], ref, "dense-mlp down on the fused codes")
    announce(f"dense-mlp down 8192x7168x18432 on the fused codes: worst err/bound {worst:.3f}")


def test_fused_quant_expert_pair_full_size():
    """The expert pair's first GEMM, 4096 x 2048 x 7168 (256 x 128 tiles), with H quantized in
    its epilogue, on the first and last row of every 128-row block plus seeded rows."""
    wl = workload(2)
    x = wl.tensors["x"].to(dev())
    w1, s1 = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    q_a, s_a = bfp8.act_quant(x)
    _case(q_a, s_a, w1, s1, "expert pair up 4096x2048x7168", sample_rows(4096, 16, 690))


# ------------------------------------------------------------------- gated FFN

def _swiglu_case(M, N, K, seed, what, rows=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    q_a, s_a = bfp8.act_quant(x)
    w1, s1 = synth.weight(N, K, seed + 1, seed + 2)
    w3, s3 = synth.weight(N, K, seed + 3, seed + 4)
    w13, s13 = bfp8.interleave_w13(w1, s1, w3, s3)
    announce(f"gemm_swiglu_act_quant {what} M={M} N={N} K={K}")
    q = torch.full((M, N), 0x33, dtype=torch.uint8, device=dev())
    qs = torch.full((M, N // BLOCK), -1.0, dtype=torch.float32, device=dev())
    bfp8.bfp8_gemm_swiglu_act_quant(q_a, s_a, w13.to(dev()), s13.to(dev()), q, qs)
    torch.cuda.synchronize()
    r = np.arange(M) if rows is None else rows
    qa, sa = u8(q_a), s_a.cpu().numpy()
    c1 = oracle.gemm(qa, sa, w1.numpy(), s1.numpy(), rows=r)
    c3 = oracle.gemm(qa, sa, w3.numpy(), s3.numpy(), rows=r)
    h = oracle.bf16_to_f32(oracle.swiglu_bf16(c1, c3)).astype(np.float64)
    # bound: the GEMM tolerance of g and u carried through silu(g) * u (|silu'| < 1.1),
    # three bf16 roundings, then the e4m3 quantization of the block
    tol1 = GEMM_REL * np.abs(c1) + GEMM_RMS * float(np.sqrt(np.mean(c1 ** 2)))
    tol3 = GEMM_REL * np.abs(c3) + GEMM_RMS * float(np.sqrt(np.mean(c3 ** 2)))
    silu = c1 / (1.0 + np.exp(-c1))
    bh = 1.1 * np.abs(c3) * tol1 + np.abs(silu) * tol3 + 2.0 ** -6 * np.abs(h) + 1e-30
    rt = torch.from_numpy(np.asarray(r)).to(dev())
    qn, qsn = u8(q[rt]), qs[rt].cpu().numpy()
    s_col = np.repeat(qsn.astype(np.float64), BLOCK, axis=1)
    deq = _e4m3_values()[qn] * s_col
    bound = bh + 2.0 ** -4 * (np.abs(h) + bh) + 2.0 ** -10 * s_col
    err = np.abs(deq - h)
    assert np.all(err <= bound), f"{what}: {int((err > bound).sum())} elements outside the bound"
    amax = np.abs(h).reshape(len(r), -1, BLOCK).max(axis=2)
    bmax = bh.reshape(len(r), -1, BLOCK).max(axis=2)
    s_ref = np.maximum(amax, 1e-4) / 448.0
    assert np.all(np.abs(qsn - s_ref) <= bmax / 448.0 + 1e-12), f"{what}: scales outside tolerance"
    announce(f"{what}: worst err/bound {float(np.max(err / bound)):.3f}")


def test_swiglu_quant_shapes():
    _swiglu_case(256, 256, 256, 1200, "one tile")
    _swiglu_case(300, 640, 512, 1210, "ragged M, five tiles")
    _swiglu_case(1, 128, 128, 1220, "single row")


def test_swiglu_quant_expert_shape():
    """One routed expert's gated FFN input projection at its real shape: 4096 x (2 x 2048) x 7168."""
    _swiglu_case(4096, 2048, 7168, 1230, "expert 4096x2048x7168", rows=sample_rows(4096, 12, 1231))
