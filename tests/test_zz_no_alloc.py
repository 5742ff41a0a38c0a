"""GPU checks of bfp8_gemm_noalloc, the GEMM entry point that allocates nothing.

It runs bfp8_gemm's kernels with their workspace in the library's fixed per-GPU
scratch array.  Two calls in a row, the second on a smaller problem, each compared
bit for bit with bfp8_gemm given a caller workspace of bfp8_gemm_workspace_size bytes
(which runs the same plan and kernels): a large problem whose split last round keeps
32 MiB of partial sums in the scratch array, then the decode-shaped skinny problem
whose split-K partials reuse the start of it.  A problem that needs no scratch and
one checked against the oracle within the GEMM tolerance complete the sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import announce, bits16, canary_intact, dev, gemm_check, u8, with_canary

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    w, w_s = synth.weight(N, K, 1300 + seed, 1400 + seed)
    q, s = bfp8.act_quant(x)
    return q, s, w.to(dev()), w_s.to(dev())


def _compare(M, N, K, seed, oracle_rows=None):
    q, s, w, w_s = _operands(M, N, K, seed)
    need = bfp8.bfp8_gemm_workspace_size(M, N, K)
    announce(f"gemm_noalloc M={M} N={N} K={K} seed={seed} scratch need={need} B")
    assert need <= bfp8.NOALLOC_SCRATCH_BYTES
    raw, c, pad = with_canary((M, N), torch.bfloat16)
    bfp8.bfp8_gemm_noalloc(q, s, w, w_s, c)
    work = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=dev()) if need else None
    ref = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    bfp8.bfp8_gemm(q, s, w, w_s, ref, work)
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), "wrote outside the output"
    diff = int((bits16(c) != bits16(ref)).sum())
    assert diff == 0, f"[{M},{N},{K}]: {diff} outputs differ from bfp8_gemm with a workspace"
    if oracle_rows is not None:
        r = oracle.gemm(u8(q), s.cpu().numpy(), u8(w), w_s.cpu().numpy(), rows=oracle_rows)
        worst = gemm_check(c[torch.from_numpy(oracle_rows).to(dev())], r, f"noalloc[{M},{N},{K}]")
        announce(f"gemm_noalloc [{M},{N},{K}] oracle worst err/bound {worst:.3f}")
    announce(f"gemm_noalloc [{M},{N},{K}] bit-identical to bfp8_gemm with a workspace")
    return need


def test_noalloc_two_calls_larger_then_smaller():
    # 2048 x 10240 x 10240: 320 tiles of 256 x 256, the last 64 split over K (32 MiB of partials)
    big = _compare(2048, 10240, 10240, seed=1, oracle_rows=np.array([0, 127, 1000, 2047], np.int64))
    assert big == 32 << 20
    # then the decode-shaped projection 64 x 1536 x 7168 (split-K, 2.75 MiB of partials)
    small = _compare(64, 1536, 7168, seed=2, oracle_rows=np.arange(64, dtype=np.int64))
    assert 0 < small < big


def test_noalloc_without_scratch_and_repeat():
    # a problem with no split (no scratch), then the split one again: same bits each time
    assert _compare(300, 384, 512, seed=3, oracle_rows=np.arange(300, dtype=np.int64)) == 0
    q, s, w, w_s = _operands(64, 1536, 7168, 2)
    outs = []
    for _ in range(2):
        c = torch.empty(64, 1536, dtype=torch.bfloat16, device=dev())
        bfp8.bfp8_gemm_noalloc(q, s, w, w_s, c)
        outs.append(c)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_noalloc_rejects_over_the_maximum():
    M, N, K = 64, 12288, 128 * 1000
    assert bfp8.bfp8_gemm_workspace_size(M, N, K) > bfp8.NOALLOC_SCRATCH_BYTES
    a = torch.zeros(M, K, dtype=torch.uint8, device=dev())
    b = torch.zeros(N, K, dtype=torch.uint8, device=dev())
    sa = torch.ones(M, K // 128, dtype=torch.float32, device=dev())
    sb = torch.ones(N // 128, K // 128, dtype=torch.float32, device=dev())
    c = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    with pytest.raises(bfp8.Bfp8Error) as e:
        bfp8.bfp8_gemm_noalloc(a, sa, b, sb, c)
    assert e.value.status == 8
