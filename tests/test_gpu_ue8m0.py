"""GPU parity of the power-of-two-scale path (the e8m0 reading of scale_fmt).

act_quant_ue8m0 is bit-exact against the oracle; the hardware-scaled GEMM is
within the path's GEMM tolerance of the oracle's fp64 product on the same
codes and (power-of-two) scales.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import announce, bits16, dev, gemm_check, sample_rows, u8, workload

pytestmark = pytest.mark.gpu


def _aq_case(x, what):
    announce(f"act_quant_ue8m0 {what} {tuple(x.shape)}")
    q, s = bfp8.act_quant_ue8m0(x.to(dev()))
    torch.cuda.synchronize()
    rq, rs = oracle.act_quant_pow2(bits16(x))
    assert np.array_equal(u8(q), rq), f"{what}: codes differ"
    assert np.array_equal(s.cpu().numpy(), rs), f"{what}: scales differ"
    m, _ = np.frexp(rs.astype(np.float64))
    assert np.all(m == 0.5), f"{what}: a scale is not a power of two"


def test_act_quant_ue8m0_workloads():
    for cfg in (0, 1):
        _aq_case(workload(cfg).tensors["x"], f"config {cfg}")
    _aq_case(workload(3).tensors["x"][:1024], "dense x, first 1024 rows")


def test_act_quant_ue8m0_edge_cases():
    K = 128 * 6
    x = torch.randn(8, K, generator=torch.Generator().manual_seed(5)).float()
    x[0] = 0.0                                     # zero row: floor scale
    x[1] = 1e-7                                    # below the floor
    x[2, :128] = 448.0 * 2.0 ** -3                 # block max a power of two times 448
    x[2, 128:256] = 448.0 * 2.0 ** -3 * (1 + 2 ** -7)   # just above it: next octave
    x[3] *= 2.0 ** 40                              # large
    x[4] *= 2.0 ** -60                             # tiny (below the floor)
    x[5, 7] = -3.0e38                              # near the bf16 maximum
    x[6] = -0.0
    x[7, ::2] = 1.0
    _aq_case(x.to(torch.bfloat16), "edge cases")


def _gemm_case(M, N, K, seed, what, rows=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    q, s = bfp8.act_quant_ue8m0(x)
    w, ws = synth.weight(N, K, seed + 1, seed + 2, pow2=True)
    wd, wsd = w.to(dev()), ws.to(dev())
    announce(f"gemm_ue8m0 {what} M={M} N={N} K={K} via {bfp8.bfp8_gemm_kernel_name(M, N, K)}")
    c = bfp8.gemm_ue8m0(q, s, wd, wsd)
    c_fold = bfp8.gemm(q, s, wd, wsd)
    torch.cuda.synchronize()
    r = np.arange(M) if rows is None else rows
    ref = oracle.gemm(u8(q), s.cpu().numpy(), u8(w), ws.numpy(), rows=r)
    rt = torch.from_numpy(np.asarray(r)).to(dev())
    worst = gemm_check(c[rt], ref, what)
    gemm_check(c_fold[rt], ref, what + " (fold path)")
    announce(f"gemm_ue8m0 {what}: worst err/bound {worst:.3f}")


def test_gemm_ue8m0_shapes():
    for i, (M, N, K) in enumerate([(16, 256, 256), (130, 300, 384), (300, 1000, 640),
                                    (2000, 4096, 256), (4096, 8192, 256)]):
        rows = None if M <= 300 else sample_rows(M, 16, 900 + i)
        _gemm_case(M, N, K, 910 + 10 * i, f"shape {i}", rows)


def test_gemm_ue8m0_dense_full_size():
    """Rows: the first and last of every 128-row block plus seeded ones."""
    _gemm_case(8192, 18432, 7168, 990, "dense-mlp up", rows=sample_rows(8192, 16, 991))


def test_gemm_ue8m0_split_last_round():
    """With a workspace, shapes whose last round of 256 x 256 tiles is at most half full run
    that round as two K halves into the workspace: within tolerance of the oracle on sampled
    rows, independent of what the workspace held, a too-small workspace refused; the dense
    down projection among them."""
    for i, (M, N, K) in enumerate([(2048, 8448, 10368), (8192, 7168, 18432)]):
        need = bfp8.bfp8_gemm_ue8m0_workspace_size(M, N, K)
        assert need > 0, (M, N, K)
        g = torch.Generator().manual_seed(1700 + i)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant_ue8m0(x)
        w, ws = synth.weight(N, K, 1710 + i, 1720 + i, pow2=True)
        wd, wsd = w.to(dev()), ws.to(dev())
        work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
        announce(f"gemm_ue8m0 split last round M={M} N={N} K={K}, workspace {need} B")
        c1 = bfp8.gemm_ue8m0(q, s, wd, wsd, workspace=work)
        work.fill_(1e30)
        c2 = bfp8.gemm_ue8m0(q, s, wd, wsd, workspace=work)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2), "the result depends on the workspace contents"
        rows = sample_rows(M, 8, 1730 + i)
        ref = oracle.gemm(u8(q), s.cpu().numpy(), u8(w), ws.numpy(), rows=rows)
        worst = gemm_check(c1[torch.from_numpy(rows).to(dev())], ref, f"split last round {i}")
        announce(f"gemm_ue8m0 split last round {i}: worst err/bound {worst:.3f}")
        with pytest.raises(bfp8.Bfp8Error):
            bfp8.bfp8_gemm_ue8m0(q, s, wd, wsd, torch.empty_like(c1), work[: need // 4 - 4])


def test_gemm_ue8m0_split_last_round_random_shapes():
    """Seeded large shapes with a split last round (8 or 16 M-tiles, one or two tail columns,
    K from 80 to 96 blocks): the e8m0 GEMM with a workspace within tolerance of the oracle
    on sampled rows."""
    rng = np.random.default_rng(1750)
    for mt, rem_cols in ((8, 1), (16, 2)):
        M, N = mt * 256, (256 // mt + rem_cols) * 256
        K = int(rng.integers(80, 96)) * 128
        need = bfp8.bfp8_gemm_ue8m0_workspace_size(M, N, K)
        assert need > 0, (M, N, K)
        g = torch.Generator().manual_seed(1751 + mt)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant_ue8m0(x)
        w, ws = synth.weight(N, K, 1760 + mt, 1770 + mt, pow2=True)
        wd, wsd = w.to(dev()), ws.to(dev())
        work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
        announce(f"gemm_ue8m0 random split last round M={M} N={N} K={K}")
        c = bfp8.gemm_ue8m0(q, s, wd, wsd, workspace=work)
        torch.cuda.synchronize()
        rows = sample_rows(M, 8, 1780 + mt)
        ref = oracle.gemm(u8(q), s.cpu().numpy(), u8(w), ws.numpy(), rows=rows)
        gemm_check(c[torch.from_numpy(rows).to(dev())], ref, f"ue8m0 random split [{M},{N},{K}]")
