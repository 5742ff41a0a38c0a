"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: act_quant codes and scales bit-exact; weight_dequant bit-exact; GEMM within
|c - ref| <= 2^-7 |ref| + 1e-3 rms(ref) of the oracle's fp64 reference on the same
fp8 inputs (rms over every entry compared); the closed-form GEMM cases (identity,
one-hot, integer-valued, 2^k scaling) bit-exact.  Full-size GEMMs are compared on
sampled rows (the first and last row of every 128-row tile plus random rows), in
the same launch configuration the benchmark times.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import block_scaled_fp8_04_amd as bfp8
import oracle
from gpu_helpers import (BLOCK, announce, bits16, canary_intact, dev, gemm_check, sample_rows,
                         u8, with_canary, workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bfp8.library()               # loud failure if the HIP library is missing
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ encoder

def _oracle_encode_parallel(v, threads=16):
    out = np.empty(v.size, np.uint8)
    parts = np.array_split(np.arange(v.size), threads)

    def work(idx):
        out[idx[0]:idx[-1] + 1] = oracle.e4m3_encode(v[idx[0]:idx[-1] + 1])

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, [p for p in parts if p.size]))
    return out


@pytest.mark.parametrize("variant", [0, 1], ids=["act_quant_encoder", "alternative_encoder"])
def test_encoder_exhaustive(variant):
    """Q5: the device encoder equals the oracle on all 2^32 fp32 patterns (NaNs excluded)."""
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.uint8, device=dev())
    mismatches = 0
    first_bad = None
    for c in range(1 << 4):
        first = c * chunk
        announce(f"encode_range variant={variant} chunk {c}/16 first=0x{first:08x}")
        bfp8.bfp8_e4m3_encode_range(first, chunk, out, variant)
        got = out.cpu().numpy()
        bits = np.arange(first, first + chunk, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
        want = _oracle_encode_parallel(v)
        keep = (bits & 0x7FFFFFFF) <= 0x7F800000
        bad = np.flatnonzero((got != want) & keep)
        mismatches += bad.size
        if bad.size and first_bad is None:
            first_bad = [(hex(int(bits[i])), float(v[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    assert mismatches == 0, f"{mismatches} mismatches, first {first_bad}"


# ---------------------------------------------------------------- act_quant

def _act_quant_case(x_cpu_bf16, label):
    M, K = x_cpu_bf16.shape
    announce(f"act_quant {label} M={M} K={K}")
    x = x_cpu_bf16.to(dev())
    raw_q, q, pq = with_canary((M, K), torch.uint8)
    raw_s, s, ps = with_canary((M, K // BLOCK), torch.float32)
    bfp8.bfp8_act_quant(x, q, s)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.act_quant(bits16(x_cpu_bf16))
    q_got, s_got = u8(q), s.cpu().numpy()
    bad = np.flatnonzero(q_got.ravel() != q_ref.ravel())
    assert bad.size == 0, f"{label}: {bad.size} codes differ, first at {bad[:5]}"
    assert np.array_equal(s_got.view(np.uint32), s_ref.view(np.uint32)), f"{label}: scales differ"
    assert canary_intact(raw_q, pq) and canary_intact(raw_s, ps), f"{label}: wrote outside outputs"
    return q, s


@pytest.mark.parametrize("config,key", [(0, "x"), (1, "x"), (2, "x"), (3, "x")])
def test_act_quant_configs(config, key):
    wl = workload(config)
    _act_quant_case(wl.tensors[key], f"{wl.name}:{key}")


def test_act_quant_hidden_shapes():
    """The intermediate activations of the expert pair and the dense MLP: [4096,2048], [8192,18432]."""
    g = torch.Generator().manual_seed(2000 + 7)
    _act_quant_case(torch.randn(4096, 2048, generator=g).to(torch.bfloat16), "H[4096,2048]")
    g = torch.Generator().manual_seed(3000 + 7)
    _act_quant_case((torch.randn(8192, 18432, generator=g) * 0.5).to(torch.bfloat16), "H[8192,18432]")


def test_act_quant_edge_cases():
    g = torch.Generator().manual_seed(99)
    x = torch.randn(37, 384, generator=g)
    x[0, :128] = 0.0                                   # all-zero block -> floor scale
    x[1, :128] = -0.0                                  # negative zeros keep their sign
    x[2, :128] = 3.0                                   # constant block -> all +448 codes
    x[3, 128:256] *= 1e-30                             # tiny values, below the floor
    x[4, 256:] *= 1e30                                 # huge values
    x[5, :] = torch.linspace(-1, 1, 384)               # many exact bf16 values
    x[6, :128] = torch.tensor([2.0 ** -k for k in range(128)])  # a wide dynamic range
    _act_quant_case(x.to(torch.bfloat16), "edges[37,384]")
    _act_quant_case(torch.randn(1, 128, generator=g).to(torch.bfloat16), "single block")
    _act_quant_case(torch.randn(3, 128 * 61, generator=g).to(torch.bfloat16), "odd block count")
    # every bf16 bit pattern that is finite, in blocks
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (allbits.astype(np.uint32) << 16).view(np.float32)
    finite = allbits[np.isfinite(f)]
    pad = (-finite.size) % 128
    xb = np.concatenate([finite, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    _act_quant_case(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).clone(), "all bf16 patterns")


def test_act_quant_directed_near_ties():
    """Blocks built from values whose quotient sits next to an e4m3 rounding midpoint."""
    allx = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allx = allx[np.isfinite(allx)]
    blocks = []
    for amax in (3.0, 0.7265625, 11.5, 97.0, 1.0078125, 250.0):
        s = np.float32(np.float32(amax) / np.float32(448.0))
        xs = allx[np.abs(allx) <= amax]
        y = (xs / s).astype(np.float32)
        low = (y.view(np.uint32) & 0xFFFFF).astype(np.int64)
        near = xs[np.abs(low - 0x80000) <= 64]
        for i in range(0, near.size, 127):
            blk = np.zeros(128, np.float32)
            blk[0] = amax
            part = near[i:i + 127]
            blk[1:1 + part.size] = part
            blocks.append(blk)
    x = torch.from_numpy(np.stack(blocks)).to(torch.bfloat16)
    _act_quant_case(x, f"near-ties[{x.shape[0]},128]")


def test_act_quant_deterministic():
    wl = workload(1)
    x = wl.tensors["x"].to(dev())
    q1, s1 = bfp8.act_quant(x)
    q2, s2 = bfp8.act_quant(x)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


# ------------------------------------------------------------ weight_dequant

def _dequant_case(w_cpu, s_cpu, label, offset=0):
    N, K = w_cpu.shape
    announce(f"weight_dequant {label} N={N} K={K} offset={offset}")
    if offset:
        wbig = torch.empty(N * K + offset, dtype=torch.uint8, device=dev())
        w = wbig[offset:].view(N, K)
        w.copy_(w_cpu.to(dev()))
    else:
        w = w_cpu.to(dev())
    raw, out, pad = with_canary((N, K), torch.bfloat16)
    bfp8.bfp8_weight_dequant(w, s_cpu.to(dev()), out)
    torch.cuda.synchronize()
    ref = oracle.weight_dequant(u8(w_cpu), s_cpu.numpy())
    got = bits16(out)
    bad = np.flatnonzero(got.ravel() != ref.ravel())
    assert bad.size == 0, f"{label}: {bad.size} elements differ, first {bad[:5]}"
    assert canary_intact(raw, pad), f"{label}: wrote outside the output"


@pytest.mark.parametrize("config,key", [(0, "w1"), (1, "w1"), (2, "w1"), (2, "w2"), (3, "w1")])
def test_weight_dequant_configs(config, key):
    wl = workload(config)
    _dequant_case(wl.tensors[key], wl.tensors["s" + key[1]], f"{wl.name}:{key}")


def test_weight_dequant_ragged_and_unaligned():
    from block_scaled_fp8_04_amd import synth
    for (N, K, off) in ((300, 200, 0), (129, 144, 0), (1, 16, 0), (257, 384, 1), (130, 272, 3),
                        (128, 136, 0), (1000, 1024, 0), (8, 128, 0)):
        w, s = synth.weight(N, K, 500 + N, 600 + K)
        _dequant_case(w, s, f"ragged[{N},{K}]", offset=off)
    # every code with unit and power-of-two scales
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    codes[0x7F] = 0; codes[0xFF] = 0
    w = codes.repeat(256, 1).contiguous()
    _dequant_case(w, torch.tensor([[1.0, 2.0 ** -7], [2.0 ** 5, 0.3]], dtype=torch.float32), "all codes")


# ---------------------------------------------------------------------- GEMM

def _gemm_case(a_q, a_s, w, w_s, label, rows=None, workspace=None):
    M, K = a_q.shape
    N = w.shape[0]
    announce(f"gemm {label} M={M} N={N} K={K} rows={'all' if rows is None else len(rows)}")
    raw, c, pad = with_canary((M, N), torch.bfloat16)
    bfp8.bfp8_gemm(a_q, a_s, w, w_s, c, workspace)
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), f"{label}: wrote outside the output"
    a_np, as_np, w_np, ws_np = u8(a_q), a_s.cpu().numpy(), u8(w), w_s.cpu().numpy()
    ref = oracle.gemm(a_np, as_np, w_np, ws_np, rows=rows)
    got = c if rows is None else c[torch.from_numpy(rows).to(dev())]
    worst = gemm_check(got, ref, label)
    announce(f"gemm {label}: worst err/bound {worst:.3f}")
    return c


def _quantized_x(wl, key="x"):
    x = wl.tensors[key].to(dev())
    return bfp8.act_quant(x)


def test_gemm_tiny_config():
    wl = workload(0)
    q, s = _quantized_x(wl)
    _gemm_case(q, s, wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev()), wl.name)


def test_gemm_decode_config():
    wl = workload(1)
    q, s = _quantized_x(wl)
    w, ws = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    _gemm_case(q, s, w, ws, wl.name)
    size = bfp8.bfp8_gemm_workspace_size(*q.shape[:1], w.shape[0], q.shape[1])
    if size:
        work = torch.empty(size // 4, dtype=torch.float32, device=dev())
        _gemm_case(q, s, w, ws, wl.name + "+workspace", workspace=work)


@pytest.mark.parametrize("config", [2, 3])
def test_gemm_chain_full_size(config):
    """x -> act_quant -> GEMM1 -> H -> act_quant(H) -> GEMM2, checked stage-wise on sampled rows."""
    wl = workload(config)
    q, s = _quantized_x(wl)
    w1, s1 = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    w2, s2 = wl.tensors["w2"].to(dev()), wl.tensors["s2"].to(dev())
    rows = sample_rows(q.shape[0], seed=config)
    h = _gemm_case(q, s, w1, s1, f"{wl.name}:gemm1", rows=rows)
    qh, sh = _act_quant_case(h.cpu(), f"{wl.name}:act_quant(H)")
    _gemm_case(qh, sh, w2, s2, f"{wl.name}:gemm2", rows=rows)
    need = bfp8.bfp8_gemm_workspace_size(qh.shape[0], w2.shape[0], qh.shape[1])
    if need:
        # with a workspace (as the benchmark runs it) the last round of tiles is split over K
        work = torch.empty(need // 4, dtype=torch.float32, device=dev())
        _gemm_case(qh, sh, w2, s2, f"{wl.name}:gemm2+workspace", rows=rows, workspace=work)


def test_gemm_ragged_shapes():
    from block_scaled_fp8_04_amd import synth
    g = torch.Generator().manual_seed(5)
    seen = set()
    for (M, N, K) in ((1, 1, 128), (37, 300, 384), (130, 129, 256), (64, 257, 640), (200, 64, 128),
                      (129, 1000, 1152), (65, 130, 128), (2000, 4001, 384), (4000, 8100, 256),
                      (4096, 8192, 128)):
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        w, ws = synth.weight(N, K, 700 + M, 800 + N)
        name = bfp8.bfp8_gemm_kernel_name(M, N, K)
        seen.add(name)
        rows = None if M <= 256 else sample_rows(M, seed=M)
        _gemm_case(q, s, w.to(dev()), ws.to(dev()), f"ragged[{M},{N},{K}] via {name}", rows=rows)
    assert len(seen) >= 3, f"every kernel configuration should be exercised, saw {seen}"


def test_gemm_split_k_workspace():
    """Skinny shapes with a workspace take the split-K path; same tolerance, and the
    result does not depend on what the workspace held before."""
    from block_scaled_fp8_04_amd import synth
    g = torch.Generator().manual_seed(6)
    for (M, N, K) in ((64, 1536, 7168), (37, 300, 1152), (1, 3000, 1024), (64, 7168, 2048),
                      (50, 129, 640), (128, 2048, 7168), (256, 1536, 7168), (193, 1000, 2304),
                      (100, 4096, 1152)):
        need = bfp8.bfp8_gemm_workspace_size(M, N, K)
        assert need > 0, (M, N, K)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        w, ws = synth.weight(N, K, 900 + M, 950 + N)
        w, ws = w.to(dev()), ws.to(dev())
        work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
        c1 = _gemm_case(q, s, w, ws, f"split-k[{M},{N},{K}]", workspace=work)
        work.fill_(1e30)
        c2 = bfp8.gemm(q, s, w, ws, workspace=work)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2), "split-K result depends on the workspace contents"
        with pytest.raises(bfp8.Bfp8Error):
            bfp8.bfp8_gemm(q, s, w, ws, torch.empty_like(c1), work[: need // 4 - 4])


def test_gemm_tail_split_workspace():
    """Large shapes whose last round of 256 x 256 tiles is at most half full and whole
    columns of tiles run those columns as two K halves into the workspace: same tolerance,
    canaries intact, independent of what the workspace held, too small a workspace refused."""
    from block_scaled_fp8_04_amd import synth
    g = torch.Generator().manual_seed(8)
    # (M, N, K): 4 x 65 tiles (4 in the tail), 8 x 33 tiles (8, odd K blocks), 16 x 18 tiles
    # (32 in two tail columns), all with the at least 80 K blocks the split tail needs
    for (M, N, K) in ((1024, 16640, 10240), (2048, 8448, 10368), (4096, 4608, 10240)):
        need = bfp8.bfp8_gemm_workspace_size(M, N, K)
        assert need > 0, (M, N, K)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        w, ws = synth.weight(N, K, 1100 + M, 1200 + N)
        w, ws = w.to(dev()), ws.to(dev())
        rows = sample_rows(M, seed=M)
        work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
        c1 = _gemm_case(q, s, w, ws, f"tail-split[{M},{N},{K}]", rows=rows, workspace=work)
        work.fill_(1e30)
        c2 = bfp8.gemm(q, s, w, ws, workspace=work)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2), "tail-split result depends on the workspace contents"
        with pytest.raises(bfp8.Bfp8Error):
            bfp8.bfp8_gemm(q, s, w, ws, torch.empty_like(c1), work[: need // 4 - 4])


def test_gemm_workspace_paths_random_shapes():
    """Seeded random shapes through both workspace paths: skinny problems (M <= 64, and
    64 < M <= 256 with at most 32 tiles of 128 x 128; deep or shallow split-K, whichever the
    plan picks) and large ones whose last round of tiles is split over
    K.  Each runs with and without the workspace; both within tolerance of the oracle on
    sampled rows, canaries intact."""
    from block_scaled_fp8_04_amd import synth
    rng = np.random.default_rng(11)
    g = torch.Generator().manual_seed(12)
    shapes = []
    for _ in range(8):                                   # skinny: M <= 64
        M = int(rng.integers(1, 65))
        N = int(rng.integers(1, 40)) * 64 + int(rng.integers(0, 64))
        K = int(rng.integers(9, 40)) * 128
        shapes.append((M, N, K))
    for mt, rem_cols in ((8, 1), (16, 2), (32, 1)):      # large: whole rounds + a short tail
        nt = 256 // mt + rem_cols
        K = int(rng.integers(80, 96)) * 128
        shapes.append((mt * 256, nt * 256, K))
    for _ in range(4):                                   # skinny: 64 < M <= 256, <= 32 tiles
        M = int(rng.integers(65, 257))
        mt = (M + 127) // 128
        N = int(rng.integers(1, 32 // mt)) * 128 + int(rng.integers(0, 128))
        K = int(rng.integers(9, 60)) * 128
        shapes.append((M, N, K))
    for (M, N, K) in shapes:
        need = bfp8.bfp8_gemm_workspace_size(M, N, K)
        x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        w, ws = synth.weight(N, K, 1300 + M, 1400 + N)
        w, ws = w.to(dev()), ws.to(dev())
        rows = None if M <= 256 else sample_rows(M, extra=8, seed=M)
        _gemm_case(q, s, w, ws, f"random[{M},{N},{K}] no workspace", rows=rows)
        if need:
            work = torch.full((need // 4,), float("nan"), dtype=torch.float32, device=dev())
            _gemm_case(q, s, w, ws, f"random[{M},{N},{K}] workspace {need} B", rows=rows,
                       workspace=work)
    ws_size = bfp8.bfp8_gemm_workspace_size
    assert sum(1 for (M, N, K) in shapes if M > 256 and ws_size(M, N, K)) == 3
    assert sum(1 for (M, N, K) in shapes if 64 < M <= 256 and ws_size(M, N, K)) == 4


def test_gemm_identity_bit_exact():
    """G3: W = I (code 0x38, scale 1) gives bf16(fl32(dec(q) * s)) exactly."""
    wl = workload(0)
    q, s = _quantized_x(wl)
    K = q.shape[1]
    eye = torch.zeros(K, K, dtype=torch.uint8)
    eye.fill_diagonal_(0x38)
    c = bfp8.gemm(q, s, eye.to(dev()), torch.ones(K // BLOCK, K // BLOCK, device=dev()))
    torch.cuda.synchronize()
    val = oracle.e4m3_decode(u8(q)) * np.repeat(s.cpu().numpy(), BLOCK, axis=1)   # float32 product
    want = oracle.f32_to_bf16(val.astype(np.float32))
    got = bits16(c)
    zero = lambda b: np.where((b & 0x7FFF) == 0, 0, b)     # +0 and -0 compare equal
    assert np.array_equal(zero(got), zero(want))


def test_gemm_one_hot_bit_exact():
    """G4: row n of W is 1.0 at pi(n); scales 2^k -> bf16(fl32(dec(q[m,pi(n)]) * s) * 2^k)."""
    g = torch.Generator().manual_seed(17)
    M, N, K = 64, 256, 384
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev())
    q, s = bfp8.act_quant(x)
    perm = torch.randperm(K, generator=g)[:N].numpy()
    w = torch.zeros(N, K, dtype=torch.uint8)
    w[torch.arange(N), torch.from_numpy(perm)] = 0x38
    k = torch.randint(-4, 5, (2, 3), generator=g).to(torch.float32)
    ws = torch.exp2(k)
    c = bfp8.gemm(q, s, w.to(dev()), ws.to(dev()))
    torch.cuda.synchronize()
    qv = oracle.e4m3_decode(u8(q))[:, perm]
    sv = s.cpu().numpy()[:, perm // BLOCK]
    prod = (qv * sv).astype(np.float32) * ws.numpy()[np.arange(N)[None, :] // BLOCK, perm[None, :] // BLOCK]
    want = oracle.f32_to_bf16(prod.astype(np.float32))
    got = bits16(c)
    zero = lambda b: np.where((b & 0x7FFF) == 0, 0, b)     # +0 and -0 compare equal
    assert np.array_equal(zero(got), zero(want))


def test_gemm_integer_exact():
    """G5: integer codes (|v| <= 4), unit scales, K = 18432: fp32 accumulation is exact."""
    vals = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    small = np.array([c for c in range(256) if np.isfinite(vals[c]) and vals[c] == np.round(vals[c])
                      and abs(vals[c]) <= 4], np.uint8)
    rng = np.random.default_rng(18)
    M, N, K = 96, 300, 18432
    a = small[rng.integers(0, small.size, (M, K))]
    b = small[rng.integers(0, small.size, (N, K))]
    a_s = torch.ones(M, K // BLOCK, device=dev())
    b_s = torch.ones(-(-N // BLOCK), K // BLOCK, device=dev())
    c = bfp8.gemm(torch.from_numpy(a).to(dev()), a_s, torch.from_numpy(b).to(dev()), b_s)
    torch.cuda.synchronize()
    exact = vals[a].astype(np.int64) @ vals[b].astype(np.int64).T
    want = oracle.f32_to_bf16(exact.astype(np.float32))
    assert np.array_equal(bits16(c), want)


def test_gemm_scale_power_of_two():
    """G6: weight scales times 2^k -> output times 2^k, bit for bit; and run-twice determinism."""
    wl = workload(1)
    q, s = _quantized_x(wl)
    w, ws = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    c0 = bfp8.gemm(q, s, w, ws)
    c1 = bfp8.gemm(q, s, w, ws * 8.0)
    c2 = bfp8.gemm(q, s, w, ws)
    torch.cuda.synchronize()
    assert torch.equal(c0, c2)
    assert torch.equal((c0.float() * 8.0).to(torch.bfloat16), c1)


# ------------------------------------------------------------- grouped GEMM

def _grouped_case(a_q, a_s, b, b_s, off, label, rows=None):
    T, K = a_q.shape
    G, N, _ = b.shape
    announce(f"gemm_grouped {label} T={T} G={G} N={N} K={K}")
    raw, c, pad = with_canary((T, N), torch.bfloat16)
    bfp8.bfp8_gemm_grouped(a_q, a_s, b, b_s, c, off.to(dev()))
    torch.cuda.synchronize()
    assert canary_intact(raw, pad), f"{label}: wrote outside the output"
    ref = oracle.gemm_grouped(u8(a_q), a_s.cpu().numpy(), u8(b), b_s.cpu().numpy(),
                              off.numpy(), rows=rows)
    got = c if rows is None else c[torch.from_numpy(rows).to(dev())]
    worst = gemm_check(got, ref, label)
    announce(f"gemm_grouped {label}: worst err/bound {worst:.3f}")
    return c


def test_grouped_routed_experts_full_size():
    wl = workload(4)
    x = wl.tensors["x"]
    ids, off = wl.tensors["token_ids"], wl.tensors["offsets"]
    xg = x[ids].contiguous().to(dev())             # tokens gathered in expert order
    q, s = bfp8.act_quant(xg)
    counts = (off[1:] - off[:-1]).numpy()
    announce(f"routing: T={int(off[-1])} tokens-per-expert min {counts.min()} max {counts.max()}")
    rows = []
    for g in range(len(counts)):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            rows += [lo, hi - 1, (lo + hi) // 2]
    rows = np.array(sorted(set(rows)), np.int64)
    _grouped_case(q, s, wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev()), off,
                  wl.name, rows=rows)


def test_grouped_small_cases():
    from block_scaled_fp8_04_amd import synth
    g = torch.Generator().manual_seed(41)
    K, N = 256, 300
    # a group's last tile takes a remainder of up to 64 rows past a full 256 (tiles of 257 ..
    # 288 and 289 .. 320 rows are separate code paths); a larger remainder, or a group below
    # 256 rows, takes a partial tile; N = 300 leaves a ragged last N-tile
    for counts in ([3, 0, 5, 1, 0, 4], [0, 0, 130], [129], [1] * 9, [0, 257, 0, 0, 64, 1],
                   [63, 100, 326, 191], [256, 288, 289, 320, 321, 512, 575, 576, 577, 0, 65, 1],
                   [304, 214, 287, 2, 800]):
        counts = np.array(counts)
        G = len(counts)
        off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
        T = int(off[-1])
        x = torch.randn(T, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        ws = [synth.weight(N, K, 900 + i, 950 + i) for i in range(G)]
        b = torch.stack([w for w, _ in ws]).to(dev())
        b_s = torch.stack([sc for _, sc in ws]).to(dev())
        _grouped_case(q, s, b, b_s, off, f"counts={counts.tolist()}")


def test_grouped_random_offsets():
    """Seeded random group sizes, including runs of empty groups, more than 64 groups (the
    tile lookup scans the offsets 64 groups at a time) and groups past 320 rows (several
    tiles, the last one partial or tall), against the oracle on every row."""
    from block_scaled_fp8_04_amd import synth
    rng = np.random.default_rng(71)
    g = torch.Generator().manual_seed(72)
    for G, hi, K, N in ((130, 70, 256, 320), (70, 600, 384, 256), (65, 2, 128, 130)):
        counts = rng.integers(0, hi + 1, size=G)
        counts[rng.random(G) < 0.25] = 0
        off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
        T = int(off[-1])
        assert T > 0
        x = torch.randn(T, K, generator=g).to(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        ws = [synth.weight(N, K, 1500 + i, 1600 + i) for i in range(G)]
        b = torch.stack([w for w, _ in ws]).to(dev())
        b_s = torch.stack([sc for _, sc in ws]).to(dev())
        _grouped_case(q, s, b, b_s, off, f"random G={G} T={T} K={K} N={N}")


def test_grouped_single_group_equals_gemm():
    wl = workload(0)
    q, s = _quantized_x(wl)
    w, ws = wl.tensors["w1"].to(dev()), wl.tensors["s1"].to(dev())
    off = torch.tensor([0, q.shape[0]], dtype=torch.int32, device=dev())
    c1 = bfp8.gemm(q, s, w, ws)
    c2 = bfp8.gemm_grouped(q, s, w[None].contiguous(), ws[None].contiguous(), off)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


# ------------------------------------------------------- exhaustive sweeps

def _oracle_bf16_parallel(v, threads=16):
    out = np.empty(v.size, np.uint16)
    bounds = np.linspace(0, v.size, threads + 1).astype(np.int64)

    def work(i):
        out[bounds[i]:bounds[i + 1]] = oracle.f32_to_bf16(v[bounds[i]:bounds[i + 1]])

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))
    return out


@pytest.mark.parametrize("variant", [0, 1], ids=["native_conversion", "bit_rule"])
def test_bf16_rounding_exhaustive(variant):
    """The device bf16 rounding used by dequant and the GEMM epilogue equals the oracle
    on all 2^32 fp32 patterns (NaNs excluded)."""
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int16, device=dev())
    mismatches, first_bad = 0, None
    for c in range(1 << 4):
        first = c * chunk
        announce(f"bf16_round_range variant={variant} chunk {c}/16 first=0x{first:08x}")
        bfp8.bfp8_bf16_round_range(first, chunk, out, variant)
        got = out.cpu().numpy().view(np.uint16)
        bits = np.arange(first, first + chunk, dtype=np.uint64).astype(np.uint32)
        want = _oracle_bf16_parallel(bits.view(np.float32))
        keep = (bits & 0x7FFFFFFF) <= 0x7F800000
        bad = np.flatnonzero((got != want) & keep)
        mismatches += bad.size
        if bad.size and first_bad is None:
            first_bad = [(hex(int(bits[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:5]]
    assert mismatches == 0, f"{mismatches} mismatches, first {first_bad}"


def _pair_blocks(v_lo, v_hi):
    """Blocks [amax, x...] covering, for every bf16 bit pattern v in [v_lo, v_hi) taken as
    the block maximum, every bf16 x with |x| <= v (both signs), 127 per block."""
    vs = np.arange(v_lo, v_hi, dtype=np.int64)
    counts = 2 * (vs + 1)
    nblk = -(-counts // 127)
    lengths = nblk * 127
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    p = np.arange(int(lengths.sum()), dtype=np.int64) - np.repeat(starts, lengths)
    v_rep = np.repeat(vs, lengths)
    x = np.where(p <= v_rep, p, np.where(p <= 2 * v_rep + 1, 0x8000 + p - v_rep - 1, 0))
    blocks = np.zeros((int(nblk.sum()), 128), np.uint16)
    blocks[:, 0] = np.repeat(vs, nblk).astype(np.uint16)
    blocks[:, 1:] = x.astype(np.uint16).reshape(-1, 127)
    return blocks


def _oracle_act_quant_parallel(xb, threads=16):
    q = np.empty(xb.shape, np.uint8)
    s = np.empty((xb.shape[0], xb.shape[1] // BLOCK), np.float32)
    bounds = np.linspace(0, xb.shape[0], threads + 1).astype(np.int64)

    def work(i):
        lo, hi = bounds[i], bounds[i + 1]
        if hi > lo:
            q[lo:hi], s[lo:hi] = oracle.act_quant(xb[lo:hi])

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))
    return q, s


def test_act_quant_exhaustive_max_element_pairs():
    """act_quant equals the oracle for every (block max, element) pair of bf16 values:
    each finite positive bf16 value as a block's max, with every bf16 value of no
    larger magnitude (both signs) as an element of that block."""
    v_end = 0x7F80                                   # positive finite bf16 patterns 1 .. 0x7F7F
    edges = [1]
    target = 1 << 27                                 # elements per chunk
    while edges[-1] < v_end:
        v = edges[-1]
        nxt = int(np.sqrt(v * v + target)) + 1
        edges.append(min(v_end, max(nxt, v + 1)))
    total = 0
    for lo, hi in zip(edges[:-1], edges[1:]):
        xb = _pair_blocks(lo, hi)
        announce(f"act_quant pairs amax bits [0x{lo:04x}, 0x{hi:04x}): {xb.shape[0]} blocks")
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev())
        q, s = bfp8.act_quant(x)
        torch.cuda.synchronize()
        q_ref, s_ref = _oracle_act_quant_parallel(xb)
        q_got = u8(q)
        bad = np.flatnonzero(q_got.ravel() != q_ref.ravel())
        assert bad.size == 0, (f"amax bits [{lo:#x},{hi:#x}): {bad.size} codes differ; first "
                               f"(block, pos) {[(int(i) // 128, int(i) % 128) for i in bad[:5]]}")
        assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        total += xb.size
        del x, q, s
    announce(f"act_quant pairs: {total} elements checked")
