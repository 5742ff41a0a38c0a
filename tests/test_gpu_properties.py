"""Properties of the GPU GEMM that hold at any size, checked on every output element at the
dense MLP layer's full size (the oracle comparisons there sample rows).

Each output element is sum_kb P_kb * (a_s * b_s) folded in K-block order in fp32, with P_kb
the fp8 MFMA block product; nothing in that arithmetic depends on where the element sits in
its tile, on which tile configuration runs it, or on the other rows and columns (when no
workspace plan splits K).  Hence, bit for bit:

* row equivariance: permuting the rows of A (codes and scales) permutes the rows of C;
* weight-block equivariance: permuting the weight's 128-row blocks (codes and scale rows)
  permutes C's 128-column blocks;
* power-of-two homogeneity: doubling every weight scale doubles C (every term and partial sum
  scales by 2 exactly, and so does bf16 rounding, away from overflow and subnormals);
* tile-configuration independence: the first rows of a GEMM equal the GEMM of those rows
  alone, which runs on other tiles (256 x 256, 256 x 128, or 128 x 128 two per CU, with
  partial tiles);
* the fused act_quant epilogue is row-equivariant too (quantization is row-local);
* the grouped GEMM's rows equal the plain GEMM of each group's rows with its expert's
  weight, and reversing the group order reverses its output's row blocks;
* the BF16 branch's GEMM and the power-of-two-scale GEMM are row-equivariant and give the
  same bits for leading rows run alone.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_04_amd as bfp8
from gpu_helpers import announce, dev, workload

pytestmark = pytest.mark.gpu
BLOCK = 128


@pytest.fixture(scope="module")
def dense():
    wl = workload(3)
    x = wl.tensors["x"].to(dev())
    q, s = bfp8.act_quant(x)
    w, ws = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    c = bfp8.gemm(q, s, w, ws)
    torch.cuda.synchronize()
    return q, s, w, ws, c


def test_row_permutation_full_size(dense):
    q, s, w, ws, c = dense
    g = torch.Generator(device=dev()).manual_seed(41)
    perm = torch.randperm(q.shape[0], generator=g, device=dev())
    announce(f"row permutation: {q.shape[0]} x {w.shape[0]} x {q.shape[1]}")
    cp = bfp8.gemm(q[perm].contiguous(), s[perm].contiguous(), w, ws)
    torch.cuda.synchronize()
    assert torch.equal(cp, c[perm]), "C of permuted rows differs from the permuted C"


def test_weight_block_permutation_full_size(dense):
    q, s, w, ws, c = dense
    N, K = w.shape
    nb = N // BLOCK
    g = torch.Generator(device=dev()).manual_seed(42)
    bperm = torch.randperm(nb, generator=g, device=dev())
    cols = (bperm[:, None] * BLOCK + torch.arange(BLOCK, device=dev())[None, :]).reshape(-1)
    announce(f"weight block permutation: {nb} blocks of {BLOCK} rows")
    wp = w.view(nb, BLOCK, K)[bperm].reshape(N, K).contiguous()
    cp = bfp8.gemm(q, s, wp, ws[bperm].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(cp, c[:, cols]), "C of permuted weight blocks differs from permuted C columns"


def test_weight_scale_doubling_full_size(dense):
    q, s, w, ws, c = dense
    announce("weight scales doubled")
    c2 = bfp8.gemm(q, s, w, ws * 2.0)
    torch.cuda.synchronize()
    finite = torch.isfinite(c.float()).all().item()
    assert finite
    assert torch.equal(c2.float(), c.float() * 2.0), "doubling the weight scales did not double C"


@pytest.mark.parametrize("rows", [4096, 3000, 1000, 257, 100, 64])
def test_leading_rows_alone(dense, rows):
    q, s, w, ws, c = dense
    announce(f"first {rows} rows alone via {bfp8.bfp8_gemm_kernel_name(rows, w.shape[0], q.shape[1])}")
    cr = bfp8.gemm(q[:rows].contiguous(), s[:rows].contiguous(), w, ws)
    torch.cuda.synchronize()
    assert torch.equal(cr, c[:rows]), f"the first {rows} rows differ when run alone"


def test_fused_quant_row_permutation(dense):
    q, s, w, ws, c = dense
    M = 2048
    g = torch.Generator(device=dev()).manual_seed(43)
    perm = torch.randperm(M, generator=g, device=dev())
    announce(f"fused act_quant, row permutation of {M} rows")
    q1, s1 = bfp8.gemm_act_quant(q[:M].contiguous(), s[:M].contiguous(), w, ws)
    q2, s2 = bfp8.gemm_act_quant(q[:M][perm].contiguous(), s[:M][perm].contiguous(), w, ws)
    torch.cuda.synchronize()
    assert torch.equal(q2, q1[perm]) and torch.equal(s2, s1[perm])


# ------------------------------------------------------------------ grouped GEMM

@pytest.fixture(scope="module")
def routed():
    wl = workload(4)
    ids, off = wl.tensors["token_ids"], wl.tensors["offsets"]
    xg = wl.tensors["x"][ids].contiguous().to(dev())
    q, s = bfp8.act_quant(xg)
    b, bs = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    c = bfp8.gemm_grouped(q, s, b, bs, off.to(dev()))
    torch.cuda.synchronize()
    return q, s, b, bs, off, c


def test_grouped_equals_per_group_gemm_full_size(routed):
    """Every row of the grouped GEMM (32 experts, 8195 routed rows, each group's remainder
    rows riding in its last tile) equals the plain GEMM of that group's rows with its
    expert's weight, bit for bit."""
    q, s, b, bs, off, c = routed
    announce(f"grouped vs per-group GEMM: {len(off) - 1} groups, {int(off[-1])} rows")
    for g in range(len(off) - 1):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        cg = bfp8.gemm(q[lo:hi].contiguous(), s[lo:hi].contiguous(), b[g], bs[g])
        torch.cuda.synchronize()
        assert torch.equal(cg, c[lo:hi]), f"group {g} ({hi - lo} rows) differs"


def test_grouped_group_permutation_full_size(routed):
    """Reversing the order of the groups (their rows and their weights) reverses the
    output's row blocks, bit for bit."""
    q, s, b, bs, off, c = routed
    G = len(off) - 1
    counts = (off[1:] - off[:-1]).tolist()
    order = list(range(G))[::-1]
    rows = torch.cat([torch.arange(int(off[g]), int(off[g + 1])) for g in order]).to(dev())
    off2 = torch.tensor([0] + list(np.cumsum([counts[g] for g in order])), dtype=torch.int32)
    announce(f"grouped GEMM with the {G} groups in reverse order")
    c2 = bfp8.gemm_grouped(q[rows].contiguous(), s[rows].contiguous(), b.flip(0).contiguous(),
                           bs.flip(0).contiguous(), off2.to(dev()))
    torch.cuda.synchronize()
    assert torch.equal(c2, c[rows])


# ------------------------------------------------------------- BF16 branch and e8m0

def test_bf16_gemm_row_permutation_and_leading_rows():
    """The BF16 branch's GEMM (dense MLP up projection on the dequantized weight): permuting
    the rows of x permutes the rows of the output, and leading rows alone (other tiles)
    give the same bits."""
    wl = workload(3)
    x = wl.tensors["x"].to(dev())
    wd = bfp8.weight_dequant(wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev()))
    c = bfp8.gemm_bf16(x, wd)
    g = torch.Generator(device=dev()).manual_seed(44)
    perm = torch.randperm(x.shape[0], generator=g, device=dev())
    announce("bf16 GEMM row permutation")
    cp = bfp8.gemm_bf16(x[perm].contiguous(), wd)
    torch.cuda.synchronize()
    assert torch.equal(cp, c[perm])
    for rows in (3000, 200):
        cr = bfp8.gemm_bf16(x[:rows].contiguous(), wd)
        torch.cuda.synchronize()
        assert torch.equal(cr, c[:rows]), f"bf16 GEMM: the first {rows} rows differ when run alone"


def test_ue8m0_gemm_row_permutation_and_leading_rows():
    """The power-of-two-scale GEMM at the dense MLP up shape: row equivariance and leading
    rows alone (256 x 256 tiles, then 128 x 128 tiles two per CU)."""
    wl = workload(3)
    x = wl.tensors["x"].to(dev())
    q, s = bfp8.act_quant_ue8m0(x)
    from block_scaled_fp8_04_amd import synth
    w, ws = synth.weight(18432, 7168, 4401, 4402, pow2=True)
    w, ws = w.to(dev()), ws.to(dev())
    c = bfp8.gemm_ue8m0(q, s, w, ws)
    g = torch.Generator(device=dev()).manual_seed(45)
    perm = torch.randperm(q.shape[0], generator=g, device=dev())
    announce("e8m0 GEMM row permutation")
    cp = bfp8.gemm_ue8m0(q[perm].contiguous(), s[perm].contiguous(), w, ws)
    torch.cuda.synchronize()
    assert torch.equal(cp, c[perm])
    for rows in (3000, 300):
        cr = bfp8.gemm_ue8m0(q[:rows].contiguous(), s[:rows].contiguous(), w, ws)
        torch.cuda.synchronize()
        assert torch.equal(cr, c[:rows]), f"e8m0 GEMM: the first {rows} rows differ when run alone"
