"""GPU edge cases at the ends of the size range.

* Empty problems (a zero dimension, or groups that hold no rows) return OK, launch
  nothing and leave every output byte untouched (canary-filled buffers).
* K at its stated maximum (2^22 - 128): the tile path addresses rows with 32-bit byte
  offsets up to ~2^29 there, and the split-K path runs thousands of splits; both are
  checked against the oracle on sampled rows within the GEMM tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from gpu_helpers import announce, canary_intact, dev, gemm_check, u8, with_canary

pytestmark = pytest.mark.gpu
BLOCK = 128
K_MAX = (1 << 22) - BLOCK


def _codes(rows, cols, seed):
    """Random finite e4m3 codes (magnitude codes below 0x78, random sign), built on the host."""
    g = torch.Generator().manual_seed(seed)
    mag = torch.randint(0, 0x78, (rows, cols), generator=g, dtype=torch.uint8)
    sign = torch.randint(0, 2, (rows, cols), generator=g, dtype=torch.uint8) << 7
    return mag | sign


def _scales(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.exp2(torch.empty(shape).uniform_(-12.0, -6.0, generator=g)).to(torch.float32)


def test_empty_problems_touch_nothing():
    K = 256
    raw_q, q, pq = with_canary((4, K), torch.uint8)
    raw_s, s, ps = with_canary((4, K // BLOCK), torch.float32)
    raw_y, y, py = with_canary((4, 256), torch.bfloat16)
    x = torch.randn(4, K, device=dev()).to(torch.bfloat16)
    w = torch.zeros(256, K, dtype=torch.uint8, device=dev())
    ws = torch.ones(2, K // BLOCK, dtype=torch.float32, device=dev())
    P = lambda t: t.data_ptr()
    lib = bfp8.library()
    stream = torch.cuda.current_stream().cuda_stream
    announce("empty problems: act_quant M=0, dequant N=0, gemm M=0 / N=0, bf16 gemm M=0, linear M=0")
    assert lib.bfp8_act_quant(P(x), P(q), P(s), 0, K, stream) == 0
    assert lib.bfp8_weight_dequant(P(w), P(ws), P(y), 0, K, stream) == 0
    assert lib.bfp8_gemm(P(q), P(s), P(w), P(ws), P(y), 0, 256, K, None, 0, stream) == 0
    assert lib.bfp8_gemm(P(q), P(s), P(w), P(ws), P(y), 4, 0, K, None, 0, stream) == 0
    assert lib.bfp8_gemm_bf16(P(x), P(x), P(y), 0, 4, K, None, 0, stream) == 0
    work = torch.zeros(1 << 16, dtype=torch.uint8, device=dev())
    assert lib.bfp8_linear_fp8(P(x), P(w), P(ws), P(y), 0, 256, K, P(work), work.numel(), stream) == 0
    # grouped: two groups, neither holds a row
    off = torch.zeros(3, dtype=torch.int32, device=dev())
    w2 = torch.zeros(2, 256, K, dtype=torch.uint8, device=dev())
    ws2 = torch.ones(2, 2, K // BLOCK, dtype=torch.float32, device=dev())
    assert lib.bfp8_gemm_grouped(P(q), P(s), P(w2), P(ws2), P(y), P(off), 2, 4, 256, K, stream) == 0
    torch.cuda.synchronize()
    for raw, pad, view, fill in ((raw_q, pq, q, 0xA5), (raw_s, ps, s, 0xA5), (raw_y, py, y, 0xA5)):
        assert canary_intact(raw, pad), "wrote outside the buffer"
        assert bool((raw[pad:-pad] == fill).all()), "an empty problem wrote into its output"


def _max_k_case(M, N, rows, seed, workspace):
    K = K_MAX
    announce(f"gemm at the K limit: M={M} N={N} K={K} via "
             f"{'split-K' if workspace else bfp8.bfp8_gemm_kernel_name(M, N, K)}; building inputs")
    a = _codes(M, K, seed)
    b = _codes(N, K, seed + 1)
    sa = _scales((M, K // BLOCK), seed + 2)
    sb = _scales((-(-N // BLOCK), K // BLOCK), seed + 3)
    a_d, b_d, sa_d, sb_d = a.to(dev()), b.to(dev()), sa.to(dev()), sb.to(dev())
    work = None
    if workspace:
        need = bfp8.bfp8_gemm_workspace_size(M, N, K)
        assert need > 0
        work = torch.empty(need // 4, dtype=torch.float32, device=dev())
    raw, c, pad = with_canary((M, N), torch.bfloat16)
    bfp8.bfp8_gemm(a_d, sa_d, b_d, sb_d, c, work)
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), "wrote outside the output"
    ref = oracle.gemm(u8(a), sa.numpy(), u8(b), sb.numpy(), rows=rows)
    worst = gemm_check(c[torch.from_numpy(rows).to(dev())], ref, f"K limit [{M},{N},{K}]")
    announce(f"gemm at the K limit [{M},{N}]: worst err/bound {worst:.3f}")


def test_gemm_at_k_limit_tile_path():
    # 256 x 256 runs on 128 x 128 tiles: row offsets up to 127 * K (~2^29)
    _max_k_case(256, 256, np.array([0, 1, 127, 128, 200, 255]), seed=71, workspace=False)


def test_gemm_at_k_limit_split_k_path():
    _max_k_case(3, 130, np.arange(3), seed=81, workspace=True)
