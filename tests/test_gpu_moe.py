"""GPU parity of the MoE dispatch / gathered act_quant / grouped GEMM / combine chain.

Every call goes through the C ABI (the ctypes binding), and every expected
value comes from the CPU oracle fed the same seeded inputs:
  * dispatch (offsets, row of each token, row of each slot) is integer work:
    bit-exact;
  * act_quant of gathered rows: bit-exact codes and scales;
  * grouped GEMM: the path's tolerance |err| <= 2^-7 |ref| + 1e-3 rms(ref);
  * combine: fp32 fused multiply-adds then one bf16 rounding.  With u = 2^-8
    (bf16 unit roundoff) and k slots, |y - ref| <= u |ref| + (k + 1) 2^-23
    sum_j |w_j out_j|, where ref is the exact (fp64) weighted sum.
"""
import numpy as np
import pytest
import torch

import oracle
import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import synth
from gpu_helpers import (BLOCK, GEMM_REL, GEMM_RMS, announce, bits16, canary_intact, dev,
                         gemm_check, u8, with_canary, workload)

pytestmark = pytest.mark.gpu


def _topk(T, k, E, seed, distinct=True):
    rng = np.random.default_rng(seed)
    if distinct:
        return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    return rng.integers(-3, E + 3, size=(T, k)).astype(np.int32)


def _dispatch_case(topk, lo, G, label):
    T, k = topk.shape
    announce(f"moe_dispatch {label} T={T} k={k} lo={lo} G={G}")
    t = torch.from_numpy(topk).to(dev())
    off = torch.full((G + 1,), -7, dtype=torch.int32, device=dev())
    raw_rt, row_token, pad = with_canary((max(1, T * k),), torch.int32)
    row_token.fill_(-5)
    slot_row = torch.full((T, k), -9, dtype=torch.int32, device=dev())
    ws_bytes = bfp8.bfp8_moe_dispatch_workspace_size(T, k, G)
    ws = torch.empty(max(1, ws_bytes // 4), dtype=torch.int32, device=dev())
    bfp8.bfp8_moe_dispatch(t, lo, off, row_token, slot_row, ws)
    torch.cuda.synchronize()
    assert canary_intact(raw_rt, pad), f"{label}: row_token written out of bounds"
    r_off, r_rt, r_sr = oracle.moe_dispatch(topk, lo, G)
    got_off = off.cpu().numpy()
    assert np.array_equal(got_off, r_off), f"{label}: offsets differ"
    n = int(r_off[-1])
    got_rt = row_token.cpu().numpy()
    assert np.array_equal(got_rt[:n], r_rt), f"{label}: row_token differs"
    assert np.all(got_rt[n:] == -5), f"{label}: row_token written past offsets[G]"
    assert np.array_equal(slot_row.cpu().numpy(), r_sr), f"{label}: slot_row differs"
    return off, row_token, slot_row


def test_dispatch_golden_and_random():
    _dispatch_case(np.array([[3, 0], [1, 3], [0, 2], [3, 1]], np.int32), 0, 3, "hand example")
    _dispatch_case(np.array([[3, 0], [1, 3], [0, 2], [3, 1]], np.int32), 1, 3, "hand example lo=1")
    cases = [
        (300, 8, 64, 16, 24, True),      # several workgroups, ragged tail (2400 entries)
        (97, 6, 40, 0, 40, True),        # every expert local
        (1000, 4, 10, 3, 5, False),      # duplicates and out-of-range / negative ids
        (50, 8, 256, 200, 56, True),     # range at the top of the id space
        (33, 3, 8, 8, 4, True),          # no local expert at all
        (1, 1, 4, 2, 1, True),           # one token, one slot, one group
        (4096, 8, 256, 0, 1, True),      # single local expert
        (700, 8, 2048, 0, 1024, True),   # the largest group count
        (257, 64, 96, 0, 96, True),      # 64 slots per token
        # G * nblk^2 (count-table entries read by the fused scan-and-place
        # kernel over all workgroups, nblk = 256 here) at its limit of 2^22,
        # then just above it (the separate single-workgroup scan)
        (8192, 8, 256, 0, 64, True),
        (8192, 8, 256, 0, 65, True),
    ]
    for i, (T, k, E, lo, G, distinct) in enumerate(cases):
        _dispatch_case(_topk(T, k, E, 2000 + i, distinct), lo, G, f"case {i}")


def test_dispatch_empty_batch():
    G = 7
    off = torch.full((G + 1,), 99, dtype=torch.int32, device=dev())
    t = torch.empty((0, 8), dtype=torch.int32, device=dev())
    e = torch.empty(1, dtype=torch.int32, device=dev())
    bfp8.bfp8_moe_dispatch(t, 0, off, e, torch.empty((0, 8), dtype=torch.int32, device=dev()),
                           None)
    torch.cuda.synchronize()
    assert np.all(off.cpu().numpy() == 0)


def test_dispatch_full_size_routing():
    wl = workload(4)
    topk = wl.tensors["topk"].numpy()
    off, _, _ = _dispatch_case(topk, 0, synth.LOCAL_EXPERTS, wl.name)
    # the offsets agree with the workload's own per-expert token lists
    assert np.array_equal(off.cpu().numpy(), wl.tensors["offsets"].numpy())


def test_dispatch_deterministic():
    topk = _topk(5000, 8, 256, 2100)
    a = _dispatch_case(topk, 64, 32, "run 1")
    b = _dispatch_case(topk, 64, 32, "run 2")
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# --------------------------------------------------------------- gathered act_quant

def _rows_case(x, row_token, num_rows, M, label):
    T, K = x.shape
    announce(f"act_quant_rows {label} T={T} M={M} K={K}")
    xd = x.to(dev())
    rt = torch.from_numpy(row_token.astype(np.int32)).to(dev())
    nr = None if num_rows is None else torch.tensor([num_rows], dtype=torch.int32, device=dev())
    q = torch.full((M, K), 0x5A, dtype=torch.uint8, device=dev())
    s = torch.full((M, K // BLOCK), -3.0, dtype=torch.float32, device=dev())
    bfp8.bfp8_act_quant_rows(xd, rt, nr, q, s)
    torch.cuda.synchronize()
    rows = M if num_rows is None else max(0, min(num_rows, M))
    valid = np.array([0 <= row_token[r] < T for r in range(rows)], bool)
    xb = x.contiguous().view(torch.int16).numpy().view(np.uint16)
    gq, gs = u8(q), s.cpu().numpy()
    written = np.nonzero(valid)[0]
    if written.size:
        rq, rs = oracle.act_quant(xb[row_token[written]])
        assert np.array_equal(gq[written], rq), f"{label}: codes differ"
        assert np.array_equal(gs[written], rs), f"{label}: scales differ"
    untouched = np.setdiff1d(np.arange(M), written)
    assert np.all(gq[untouched] == 0x5A) and np.all(gs[untouched] == -3.0), \
        f"{label}: wrote a row it must skip"


def test_act_quant_rows_cases():
    g = torch.Generator().manual_seed(77)
    x = (torch.randn(300, 7168, generator=g) * 3).to(torch.bfloat16)
    rng = np.random.default_rng(78)
    rt = rng.integers(0, 300, size=900)
    _rows_case(x, rt, None, 900, "all rows")
    _rows_case(x, rt, 517, 900, "num_rows below capacity")
    _rows_case(x, rt, 5000, 900, "num_rows above capacity")
    _rows_case(x, rt, 0, 900, "no rows")
    bad = rt.copy()
    bad[[0, 5, 899]] = [-1, 300, 10 ** 6]
    _rows_case(x, bad, None, 900, "invalid tokens skipped")
    x2 = (torch.randn(5, 256, generator=g)).to(torch.bfloat16)
    _rows_case(x2, np.array([4, 4, 0, 2, 1, 3, 0]), 7, 7, "tiny K=256")


def test_act_quant_rows_equals_act_quant_of_gather():
    wl = workload(4)
    x = wl.tensors["x"]
    ids = wl.tensors["token_ids"].numpy()
    xd = x.to(dev())
    M = ids.size
    rt = torch.from_numpy(ids.astype(np.int32)).to(dev())
    q1 = torch.empty((M, x.shape[1]), dtype=torch.uint8, device=dev())
    s1 = torch.empty((M, x.shape[1] // BLOCK), dtype=torch.float32, device=dev())
    bfp8.bfp8_act_quant_rows(xd, rt, None, q1, s1)
    q2, s2 = bfp8.act_quant(xd[torch.from_numpy(ids).to(dev())].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


# ------------------------------------------------------------ grouped GEMM with capacity

def test_grouped_capacity_and_clamped_offsets():
    """off[G] < total_M leaves the tail untouched; offsets past total_M are clamped."""
    g = torch.Generator().manual_seed(90)
    K, N, cap = 256, 384, 700
    x = torch.randn(cap, K, generator=g).to(torch.bfloat16).to(dev())
    q, s = bfp8.act_quant(x)
    ws = [synth.weight(N, K, 910 + i, 920 + i) for i in range(3)]
    b = torch.stack([w for w, _ in ws]).to(dev())
    b_s = torch.stack([sc for _, sc in ws]).to(dev())
    for off_list, label in (([0, 200, 210, 450], "tail 450..700 unused"),
                            ([0, 300, 650, 10 ** 6], "last offset past capacity"),
                            ([-40, 150, 120, 120], "negative start, decreasing offsets")):
        announce(f"gemm_grouped capacity case: {label}")
        raw, c, pad = with_canary((cap, N), torch.bfloat16, fill_byte=0x3C)
        off = torch.tensor(off_list, dtype=torch.int32, device=dev())
        bfp8.bfp8_gemm_grouped(q, s, b, b_s, c, off)
        torch.cuda.synchronize()
        assert canary_intact(raw, pad, 0x3C), f"{label}: wrote outside the output"
        # expected: the oracle with the offsets clamped as the header states
        lo_hi = []
        for gi in range(3):
            a0 = min(max(off_list[gi], 0), cap)
            b0 = min(max(off_list[gi + 1], a0), cap)
            lo_hi.append((a0, b0))
        got = bits16(c)
        for gi, (a0, b0) in enumerate(lo_hi):
            if b0 <= a0:
                continue
            ref = oracle.gemm(u8(q[a0:b0]), s[a0:b0].cpu().numpy(), u8(b[gi]), b_s[gi].cpu().numpy())
            gemm_check(c[a0:b0], ref, f"{label} group {gi}")
        covered = np.zeros(cap, bool)
        for a0, b0 in lo_hi:
            covered[a0:b0] = True
        assert np.all(got[~covered] == 0x3C3C), f"{label}: wrote rows outside every group"


# ------------------------------------------------------------------------ combine

def _combine_bound(out_bits, slot_row, w, ref):
    k = slot_row.shape[1]
    absb = out_bits & np.uint16(0x7FFF)
    sabs = oracle.moe_combine(absb, slot_row, np.abs(w))
    return 2.0 ** -8 * np.abs(ref) + (k + 1) * 2.0 ** -23 * sabs


def _combine_case(T, k, E, lo, G, N, seed, label, y_offset=0):
    topk = _topk(T, k, E, seed)
    r_off, r_rt, r_sr = oracle.moe_dispatch(topk, lo, G)
    rows = int(r_off[-1])
    rng = np.random.default_rng(seed + 1)
    out_f = (rng.standard_normal((max(rows, 1), N)) * np.exp2(rng.integers(-4, 5, (max(rows, 1), 1))))
    out = torch.from_numpy(out_f.astype(np.float32)).to(torch.bfloat16)[:rows]
    w = rng.random((T, k)).astype(np.float32)
    announce(f"moe_combine {label} T={T} k={k} rows={rows} N={N}")
    yb = torch.full((T * N + y_offset + 8,), 0x7777, dtype=torch.int16, device=dev())
    y = yb[y_offset:y_offset + T * N].view(torch.bfloat16).view(T, N)
    bfp8.bfp8_moe_combine(out.to(dev()).contiguous(), torch.from_numpy(r_sr).to(dev()),
                          torch.from_numpy(w).to(dev()), y)
    torch.cuda.synchronize()
    tail = yb[y_offset + T * N:].cpu().numpy()
    assert np.all(tail == 0x7777) and (y_offset == 0 or np.all(yb[:y_offset].cpu().numpy() == 0x7777))
    ob = out.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.moe_combine(ob, r_sr, w)
    got = y.float().cpu().numpy().astype(np.float64)
    bound = _combine_bound(ob, r_sr, w, ref)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{label}: {int((err > bound).sum())} elements outside the bound"
    none_local = np.all(r_sr < 0, axis=1)
    assert np.all(got[none_local] == 0.0)


def test_combine_vector_and_scalar_paths():
    _combine_case(200, 8, 64, 0, 16, 2048, 3000, "vector N=2048")
    _combine_case(64, 8, 64, 8, 24, 7168, 3010, "vector N=7168 (ragged chunk)")
    _combine_case(90, 6, 32, 4, 12, 100, 3020, "scalar N=100")
    _combine_case(50, 4, 16, 0, 16, 2048, 3030, "scalar (unaligned y)", y_offset=1)
    _combine_case(70, 8, 256, 250, 6, 256, 3040, "mostly empty tokens")
    _combine_case(100, 12, 32, 0, 32, 2048, 3050, "vector k=12 (every slot local, two slot groups)")


def test_combine_skips_rows_past_capacity():
    T, k, N = 40, 4, 512
    rng = np.random.default_rng(3100)
    rows = 60
    sr = rng.integers(-1, rows + 20, size=(T, k)).astype(np.int32)
    out = torch.from_numpy(rng.standard_normal((rows, N)).astype(np.float32)).to(torch.bfloat16)
    w = rng.random((T, k)).astype(np.float32)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev())
    bfp8.bfp8_moe_combine(out.to(dev()), torch.from_numpy(sr).to(dev()), torch.from_numpy(w).to(dev()), y)
    torch.cuda.synchronize()
    sr_valid = np.where(sr < rows, sr, -1).astype(np.int32)
    ob = out.view(torch.int16).numpy().view(np.uint16)
    ref = oracle.moe_combine(ob, sr_valid, w)
    err = np.abs(y.float().cpu().numpy() - ref)
    assert np.all(err <= _combine_bound(ob, sr_valid, w, ref))


# ------------------------------------------------------------------ whole chain

def test_moe_chain_full_size():
    """dispatch -> gathered act_quant -> grouped GEMM -> combine at 8192 tokens, top-8,
    32 local experts of 256, K=7168, N=2048, row buffers sized for T*k rows."""
    wl = workload(4)
    x, topk, w = wl.tensors["x"], wl.tensors["topk"], wl.tensors["weights"]
    W, S = wl.tensors["w1"], wl.tensors["s1"]
    T, K = x.shape
    k = topk.shape[1]
    G, N, _ = W.shape
    announce(f"moe chain {wl.name}: T={T} k={k} G={G} N={N} K={K}")
    xd, Wd, Sd = x.to(dev()), W.to(dev()), S.to(dev())
    y = bfp8.moe_experts_fp8(xd, topk.to(dev()), w.to(dev()), Wd, Sd, 0)
    # the intermediate steps, through the same entry points, to check each one
    off, row_token, slot_row = bfp8.moe_dispatch(topk.to(dev()), 0, G)
    torch.cuda.synchronize()
    r_off, r_rt, r_sr = oracle.moe_dispatch(topk.numpy(), 0, G)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(row_token.cpu().numpy()[:int(r_off[-1])], r_rt)
    assert np.array_equal(slot_row.cpu().numpy(), r_sr)

    # sampled tokens: the oracle's own chain on exactly their rows
    rng = np.random.default_rng(4040)
    toks = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, 40)]))
    sel_rows = np.unique(r_sr[toks][r_sr[toks] >= 0])
    xb = x.view(torch.int16).numpy().view(np.uint16)
    aq, asc = oracle.act_quant(xb[r_rt[sel_rows]])
    # grouped rows through the oracle: a compact A holding only the sampled rows, grouped
    # by the expert each row belongs to
    grp = np.searchsorted(r_off, sel_rows, side="right") - 1
    counts = np.bincount(grp, minlength=G)
    c_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    o_ref = oracle.gemm_grouped(aq, asc, u8(W), S.numpy(), c_off)
    o_bf = oracle.f32_to_bf16(o_ref.astype(np.float32))
    pos = {int(r): i for i, r in enumerate(sel_rows)}
    sr_sub = np.array([[pos.get(int(r), -1) if r >= 0 else -1 for r in row] for row in r_sr[toks]],
                      np.int32)
    y_ref = oracle.moe_combine(o_bf, sr_sub, w.numpy()[toks])
    # bound: each GPU expert row is within the GEMM tolerance of the exact product, the
    # reference row is that product rounded to bf16 (2^-8 relative); both carry through
    # the weights ("carried").  The combine then adds one bf16 rounding of the sum and the
    # fp32 accumulation error (k + 1) 2^-23 sum |w o|.
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    e_rows = (GEMM_REL + 2.0 ** -8) * np.abs(o_ref) + GEMM_RMS * rms
    wsub = w.numpy()[toks].astype(np.float64)
    carried = np.zeros((toks.size, N))
    sabs = np.zeros((toks.size, N))
    for ti in range(toks.size):
        for j in range(k):
            r = sr_sub[ti, j]
            if r >= 0:
                carried[ti] += wsub[ti, j] * e_rows[r]
                sabs[ti] += wsub[ti, j] * np.abs(o_ref[r])
    bound = ((1 + 2.0 ** -8) * carried + 2.0 ** -8 * np.abs(y_ref)
             + (k + 1) * 2.0 ** -22 * (sabs + carried) + 1e-30)
    got = y[torch.from_numpy(toks).to(dev())].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - y_ref)
    worst = float(np.max(err / bound))
    announce(f"moe chain: {toks.size} tokens checked, worst err/bound {worst:.3f}")
    assert np.all(err <= bound)
