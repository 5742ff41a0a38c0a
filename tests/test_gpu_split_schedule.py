"""GPU checks of the 256 x 256 tile's split load schedule.

Whole M tiles with an even K-block count run the schedule in which waves 0..3 load
the next block's A rows and waves 4..7 load the weight rows two blocks ahead; other
shapes run every wave through one schedule.  Both fold the same block products in the
same order, so the bits must agree: a problem whose M is a multiple of 256 is compared
with the same rows inside a problem one row taller (whose last tile is ragged and takes
the other schedule), for the bf16 GEMM, the GEMM with act_quant in its epilogue and the
GEMM whose last round is split over K; and the oracle checks sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import announce, bits16, dev, gemm_check, sample_rows, u8

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    w, w_s = synth.weight(N, K, 2100 + seed, 2200 + seed)
    q, s = bfp8.act_quant(x)
    return q, s, w.to(dev()), w_s.to(dev())


# (the last two have a partial last column of tiles: rows of the weight past N read as
# zeros; N = 2602 also leaves the 8-byte stores for element stores)
@pytest.mark.parametrize("M,N,K", [(2048, 5120, 2048), (4096, 3072, 4096), (2048, 7168, 7168),
                                   (4096, 2600, 2048), (4096, 2602, 4096)])
def test_split_schedule_bf16_matches_other_schedule(M, N, K):
    assert bfp8.bfp8_gemm_kernel_name(M, N, K).startswith("lds-direct 256x256")
    assert (K // 128) % 2 == 0
    q, s, w, w_s = _operands(M + 1, N, K, seed=M // 256)
    announce(f"split schedule bf16 [{M},{N},{K}] against [{M + 1},{N},{K}]")
    c_split = bfp8.gemm(q[:M], s[:M], w, w_s)
    c_other = bfp8.gemm(q, s, w, w_s)
    torch.cuda.synchronize()
    diff = int((bits16(c_split) != bits16(c_other[:M])).sum())
    assert diff == 0, f"{diff} outputs differ between the two schedules"
    rows = sample_rows(M, 8, M)
    ref = oracle.gemm(u8(q[:M]), s[:M].cpu().numpy(), u8(w), w_s.cpu().numpy(), rows=rows)
    worst = gemm_check(c_split[torch.from_numpy(rows).to(dev())], ref, f"split [{M},{N},{K}]")
    announce(f"split schedule bf16 [{M},{N},{K}] bit-identical; oracle worst err/bound {worst:.3f}")


def test_split_schedule_fused_act_quant_matches_other_schedule():
    M, N, K = 2048, 5120, 7168
    assert bfp8.bfp8_gemm_kernel_name(M, N, K).startswith("lds-direct 256x256")
    q, s, w, w_s = _operands(M + 1, N, K, seed=7)
    announce(f"split schedule fused act_quant [{M},{N},{K}] against [{M + 1},{N},{K}]")
    qa, sa = bfp8.gemm_act_quant(q[:M], s[:M], w, w_s)
    qb, sb = bfp8.gemm_act_quant(q, s, w, w_s)
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.uint8), qb[:M].view(torch.uint8)), "codes differ"
    assert torch.equal(sa, sb[:M]), "scales differ"
    # and stage-wise against the oracle: its act_quant of the other schedule's bf16 output
    c = bfp8.gemm(q[:M], s[:M], w, w_s)
    rows = sample_rows(M, 8, 71)
    cq, cs = oracle.act_quant(bits16(c[torch.from_numpy(rows).to(dev())]))
    assert np.array_equal(cq, u8(qa[torch.from_numpy(rows).to(dev())]))
    assert np.array_equal(cs, sa[torch.from_numpy(rows).to(dev())].cpu().numpy())
    announce("split schedule fused act_quant bit-identical")


def test_split_schedule_with_split_last_round():
    # 2048 x 10240 x 10240: 320 tiles, the last 64 columns of tiles split over K; the
    # whole rounds run the split schedule (80 K blocks, even)
    M, N, K = 2048, 10240, 10240
    q, s, w, w_s = _operands(M + 1, N, K, seed=9)
    need = bfp8.bfp8_gemm_workspace_size(M, N, K)
    assert need > 0
    work = torch.empty(need // 4, dtype=torch.float32, device=dev())
    announce(f"split schedule + split last round [{M},{N},{K}], workspace {need} B")
    c_split = bfp8.gemm(q[:M], s[:M], w, w_s, work)
    c_plain = bfp8.gemm(q[:M], s[:M], w, w_s)         # no workspace: every tile whole
    c_other = bfp8.gemm(q, s, w, w_s)                  # ragged M: the other schedule
    torch.cuda.synchronize()
    assert int((bits16(c_plain) != bits16(c_other[:M])).sum()) == 0
    rows = sample_rows(M, 8, 91)
    ref = oracle.gemm(u8(q[:M]), s[:M].cpu().numpy(), u8(w), w_s.cpu().numpy(), rows=rows)
    worst = gemm_check(c_split[torch.from_numpy(rows).to(dev())], ref, "split last round")
    announce(f"split schedule + split last round: oracle worst err/bound {worst:.3f}")


def test_split_schedule_random_shapes():
    # seeded shapes that take the split schedule: whole M tiles, an even K-block count and
    # enough 256 x 256 tiles for that tile; N anywhere (partial last columns included)
    rng = np.random.default_rng(2027)
    done = 0
    while done < 6:
        M = 256 * int(rng.integers(4, 33))
        N = 8 * int(rng.integers(128, 1537))
        K = 128 * 2 * int(rng.integers(4, 41))
        if not bfp8.bfp8_gemm_kernel_name(M, N, K).startswith("lds-direct 256x256"):
            continue
        done += 1
        q, s, w, w_s = _operands(M + 1, N, K, seed=300 + done)
        announce(f"split schedule random [{M},{N},{K}]")
        c_split = bfp8.gemm(q[:M], s[:M], w, w_s)
        c_other = bfp8.gemm(q, s, w, w_s)
        torch.cuda.synchronize()
        diff = int((bits16(c_split) != bits16(c_other[:M])).sum())
        assert diff == 0, f"[{M},{N},{K}]: {diff} outputs differ between the two schedules"
        rows = sample_rows(M, 4, 400 + done)
        ref = oracle.gemm(u8(q[:M]), s[:M].cpu().numpy(), u8(w), w_s.cpu().numpy(), rows=rows)
        gemm_check(c_split[torch.from_numpy(rows).to(dev())], ref, f"random [{M},{N},{K}]")
