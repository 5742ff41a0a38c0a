"""GPU parity of the BF16 branch of linear(): weight_dequant then the bf16 MFMA GEMM.

Expected values come from the CPU oracle on the same seeded inputs: the GEMM
within the path's tolerance |err| <= 2^-7 |ref| + 1e-3 rms(ref) of the fp64
sum of bf16 products (fp32 accumulation of exact bf16 products, one bf16
rounding); identity and small-integer operands are exact.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import announce, bits16, canary_intact, dev, gemm_check, sample_rows, u8, with_canary, workload

pytestmark = pytest.mark.gpu


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _case(a, b, label, rows=None):
    M, K = a.shape
    N = b.shape[0]
    announce(f"gemm_bf16 {label} M={M} N={N} K={K}")
    raw, c, pad = with_canary((M, N), torch.bfloat16)
    bfp8.bfp8_gemm_bf16(a.to(dev()), b.to(dev()), c)
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), f"{label}: wrote outside the output"
    ref = oracle.gemm_bf16(bits16(a), bits16(b), rows=rows)
    got = c if rows is None else c[torch.from_numpy(rows).to(dev())]
    worst = gemm_check(got, ref, label)
    announce(f"gemm_bf16 {label}: worst err/bound {worst:.3f}")
    return c


def test_gemm_bf16_ragged_shapes():
    shapes = [(16, 256, 256), (1, 1, 64), (17, 100, 192), (64, 257, 128), (300, 520, 640),
              (129, 1000, 64), (513, 384, 1024), (700, 2100, 256)]
    for i, (M, N, K) in enumerate(shapes):
        _case(_bf16((M, K), 500 + i), _bf16((N, K), 600 + i, 0.05), f"shape {i}")


def test_gemm_bf16_tile_configs_exercised():
    # 256x256 needs >= 2 tiles per CU; 256x128 >= half a tile per CU
    cases = [(2048, 8192, 256, "256x256"), (1024, 2048, 320, "256x128"), (96, 160, 192, "64x64")]
    for i, (M, N, K, want) in enumerate(cases):
        c = _case(_bf16((M, K), 700 + i), _bf16((N, K), 710 + i, 0.05), want,
                  rows=sample_rows(M, 24, 720 + i))
        del c


def test_linear_bf16_dense_full_size():
    """x [8192,7168] through the BF16 branch with W_up [18432,7168]: weight_dequant then
    the bf16 GEMM; the first and last row of every 128-row block (plus seeded rows)
    against the oracle's dequant and bf16 GEMM."""
    wl = workload(3)
    x, w, s = wl.tensors["x"], wl.tensors["w1"], wl.tensors["s1"]
    wd = bfp8.weight_dequant(w.to(dev()), s.to(dev()))
    c = bfp8.gemm_bf16(x.to(dev()), wd)
    torch.cuda.synchronize()
    ref_wd = oracle.weight_dequant(u8(w), s.numpy())
    assert np.array_equal(bits16(wd), ref_wd)
    rows = sample_rows(8192, 16, 820)
    ref = oracle.gemm_bf16(bits16(x), ref_wd, rows=rows)
    worst = gemm_check(c[torch.from_numpy(rows).to(dev())], ref, "linear_bf16 dense")
    announce(f"linear_bf16 dense-mlp up: worst err/bound {worst:.3f}")


def test_gemm_bf16_identity_and_integers_exact():
    a = _bf16((300, 256), 800)
    eye = torch.eye(256, dtype=torch.bfloat16)
    c = bfp8.gemm_bf16(a.to(dev()), eye.to(dev()))
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), a)
    g = torch.Generator().manual_seed(801)
    ai = torch.randint(-16, 16, (260, 512), generator=g).to(torch.bfloat16)
    bi = torch.randint(-16, 16, (300, 512), generator=g).to(torch.bfloat16)
    c = bfp8.gemm_bf16(ai.to(dev()), bi.to(dev()))
    torch.cuda.synchronize()
    exact = ai.long() @ bi.long().T                      # |sum| < 2^17: exact in fp32
    ref = exact.to(torch.float32).to(torch.bfloat16)     # one rounding, as the kernel
    assert torch.equal(c.cpu(), ref)


def test_gemm_bf16_deterministic():
    a, b = _bf16((1024, 512), 810), _bf16((2048, 512), 811)
    c1 = bfp8.gemm_bf16(a.to(dev()), b.to(dev()))
    c2 = bfp8.gemm_bf16(a.to(dev()), b.to(dev()))
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def test_gemm_bf16_split_last_round():
    """With a workspace, a shape whose last round of 256 x 256 tiles is at most half full
    runs it as two K halves (K = 10304 = 161 steps of 64, an odd count) into the workspace:
    within tolerance of the oracle on sampled rows, independent of the workspace contents,
    a short workspace refused."""
    M, N, K = 2048, 8448, 10304
    need = bfp8.bfp8_gemm_bf16_workspace_size(M, N, K)
    assert need > 0
    a, b = _bf16((M, K), 830), _bf16((N, K), 831, 0.05)
    ad, bd = a.to(dev()), b.to(dev())
    work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
    announce(f"gemm_bf16 split last round M={M} N={N} K={K}, workspace {need} B")
    raw, c1, pad = with_canary((M, N), torch.bfloat16)
    bfp8.bfp8_gemm_bf16(ad, bd, c1, work)
    work.fill_(1e30)
    c2 = bfp8.gemm_bf16(ad, bd, workspace=work)
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), "wrote outside the output"
    assert torch.equal(c1, c2), "the result depends on the workspace contents"
    rows = sample_rows(M, 8, 832)
    ref = oracle.gemm_bf16(bits16(a), bits16(b), rows=rows)
    worst = gemm_check(c1[torch.from_numpy(rows).to(dev())], ref, "bf16 split last round")
    announce(f"gemm_bf16 split last round: worst err/bound {worst:.3f}")
    with pytest.raises(bfp8.Bfp8Error):
        bfp8.bfp8_gemm_bf16(ad, bd, torch.empty_like(c1), work[: need // 4 - 4])


def test_gemm_bf16_split_last_round_random_shapes():
    """Seeded large shapes whose last round of 256 x 256 tiles is whole tile columns and at
    most half full (8 or 16 M-tiles, one or two tail columns, K from 80 to 96 blocks of 128
    in steps of 64): with a workspace, within tolerance of the oracle on sampled rows."""
    rng = np.random.default_rng(840)
    for mt, rem_cols in ((8, 1), (16, 2)):
        M, N = mt * 256, (256 // mt + rem_cols) * 256
        K = int(rng.integers(160, 192)) * 64
        need = bfp8.bfp8_gemm_bf16_workspace_size(M, N, K)
        assert need > 0, (M, N, K)
        a, b = _bf16((M, K), 841 + mt), _bf16((N, K), 842 + mt, 0.05)
        work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
        announce(f"gemm_bf16 random split last round M={M} N={N} K={K}")
        c = bfp8.gemm_bf16(a.to(dev()), b.to(dev()), workspace=work)
        torch.cuda.synchronize()
        rows = sample_rows(M, 8, 843 + mt)
        ref = oracle.gemm_bf16(bits16(a), bits16(b), rows=rows)
        gemm_check(c[torch.from_numpy(rows).to(dev())], ref, f"bf16 random split [{M},{N},{K}]")
