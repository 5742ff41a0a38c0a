"""Checks that pin the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with a fact that the pages, the e4m3 / bf16 format
definitions or plain mathematics fix: hand-derived closed forms (the golden
files), brute force, torch's own e4m3 and bf16 casts, exact rational
arithmetic, and invariants of the method.  The same functions are run against
deliberately broken builds of the oracle to show that each plausible mistake
fails at least one pin.

Sources: "Data flow - deepseek-ai/DeepSeek-V3" (codevetter), FP8 quantization
bullet (128-element activation blocks, fp32 scales, fp32 accumulation, a
.scale on each 1-byte weight); pyshine "DeepSeek-V3" tour, "FP8 with per-block
scales" (block max clamped and divided by 448, the e4m3 ceiling; weight scale
grid; dequantize-then-BF16-matmul is the other branch of linear());
"Behavior traces" (codevetter), fp8->bf16 trace bullet (dequant multiplies by
the stored scale).
"""
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BLOCK = 128


# ------------------------------------------------------------ independent helpers

def torch_e4m3_values() -> np.ndarray:
    """All 256 e4m3 code values as float64, decoded by torch (a library, not the oracle)."""
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def torch_e4m3_cast(v: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn cast (nearest-even, NOT saturating)."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def torch_bf16(v: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def brute_encode(v: np.ndarray) -> np.ndarray:
    """Nearest of the 127 finite e4m3 magnitudes, ties to the even code, sign kept.

    Brute force over the code table that torch decodes; +-inf saturate.
    """
    v = np.asarray(v, np.float32).ravel()
    mags = torch_e4m3_values()[:0x7F]             # codes 0x00..0x7E, increasing
    even = (np.arange(0x7F) % 2) == 0
    out = np.empty(v.size, np.uint8)
    step = 1 << 15
    for i in range(0, v.size, step):
        a = np.abs(v[i:i + step].astype(np.float64))
        # beyond 1000 the nearest magnitude is 448 for every a; clamping keeps the
        # distances below exact in float64 (and maps +-inf in)
        a = np.minimum(a, 1000.0)
        d = np.abs(a[:, None] - mags[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        two = cand.sum(axis=1) > 1
        pick = np.where(two, np.argmax(cand & even[None, :], axis=1), np.argmax(cand, axis=1))
        out[i:i + step] = pick.astype(np.uint8)
    sign = np.signbit(v)
    return np.where(sign, out | 0x80, out).astype(np.uint8)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def finite_f32_bit_sets(seed=7, n_random=1 << 18):
    """float32 inputs for the codec pins: every bf16 pattern, midpoints +-ulps, random."""
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf)]
    mags = torch_e4m3_values()[:0x7F]
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)      # exact in f32
    near = [mids]
    for k in (1, 2):
        up = mids.copy(); dn = mids.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf)); dn = np.nextafter(dn, np.float32(0))
        near += [up, dn]
    near = np.concatenate(near)
    near = np.concatenate([near, -near, np.float32([464.0, 463.99997, 448.0, 447.99997, 480.0])])
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, n_random, dtype=np.uint32) << 31
    expo = rng.integers(127 - 14, 127 + 11, n_random, dtype=np.uint32) << 23
    mant = rng.integers(0, 1 << 23, n_random, dtype=np.uint32)
    rnd = (sign | expo | mant).view(np.float32)
    return np.concatenate([allbf, near, rnd]).astype(np.float32)


# ---------------------------------------------------------------- codec pins

def pin_decode_table(orc):
    """Q1: all 256 codes decode as torch decodes them; 0x7E is the 448 ceiling."""
    ours = orc.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    ref = torch_e4m3_values()
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert np.array_equal(nan_o, nan_r), "NaN codes differ"
    assert set(np.flatnonzero(nan_o)) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan_o], ref[~nan_r]), "decoded values differ from torch"
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert np.nanmax(ours) == 448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def pin_encode_golden(orc):
    """Hand-derived codes (tests/golden/e4m3_hand_examples.txt)."""
    rows = read_golden("e4m3_hand_examples.txt")
    vals = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    got = orc.e4m3_encode(vals)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"golden codes differ at {[(rows[i][0], hex(got[i])) for i in bad]}"


def pin_encode_brute_force(orc):
    """Q2: encode equals brute-force nearest-even over the 127 magnitudes."""
    v = finite_f32_bit_sets()
    got = orc.e4m3_encode(v)
    want = brute_encode(v)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} -> {got[bad[:5]]} want {want[bad[:5]]}"


def pin_encode_vs_torch(orc):
    """Q3: encode equals torch's cast wherever that cast cannot overflow (|v| < 464)."""
    v = finite_f32_bit_sets(seed=11)
    v = v[np.abs(v) < 464.0]
    assert np.array_equal(orc.e4m3_encode(v), torch_e4m3_cast(v))


def pin_roundtrip(orc):
    """Q4: encode(decode(c)) == c for every non-NaN code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)


def pin_bf16_round(orc):
    """f32 -> bf16 nearest-even equals torch's cast (random patterns and exact ties)."""
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, 4096, dtype=np.uint32) << 16) | np.uint32(0x8000)
    v = np.concatenate([bits, ties]).view(np.float32)
    v = v[np.isfinite(v)]
    v = v[np.abs(v) < 3.0e38]                 # keep clear of rounding up to inf
    assert np.array_equal(orc.f32_to_bf16(v), torch_bf16(v))


# ------------------------------------------------------------ act_quant pins

def _rand_bf16(M, K, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(M, K, generator=g) * scale).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16).copy()


def pin_act_quant_golden(orc):
    """Hand-worked blocks (tests/golden/act_quant_hand_block.txt): scale 1 and scale 2."""
    rows = read_golden("act_quant_hand_block.txt")
    x = np.zeros(256, np.float32)
    want_q = np.zeros(256, np.uint8)
    want_s = {}
    for r in rows:
        if r[0] == "scale":
            want_s[int(r[1])] = float(r[2])
            continue
        blk, pos = int(r[0]), int(r[1])
        x[blk * BLOCK + pos] = float(r[2])
        want_q[blk * BLOCK + pos] = int(r[3], 16)
    xb = torch_bf16(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x), "golden inputs must be exact in bf16"
    q, s = orc.act_quant(xb[None, :])
    assert s[0, 0] == want_s[0] and s[0, 1] == want_s[1], f"scales {s}"
    bad = np.flatnonzero(q[0] != want_q)
    assert bad.size == 0, f"codes differ at {bad}: {q[0][bad]} want {want_q[bad]}"


def pin_act_quant_ceiling_hit(orc):
    """A1: every block whose max is above the floor holds a +-448 code (0x7E / 0xFE)."""
    x = _rand_bf16(64, 1024, 21)
    q, s = orc.act_quant(x)
    blocks = (q & 0x7F).reshape(64, -1, BLOCK)
    assert np.all((blocks == 0x7E).any(axis=2))


def ulp_e4m3(v):
    """Spacing of e4m3 values around |v| (2^-9 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -40)))
    return np.exp2(np.maximum(e, -6) - 3)


def pin_act_quant_error_bound(orc):
    """A2: |dec(q)*s - x| <= s * (ulp/2 at x/s + 2^-23 * |x|/s) for every element."""
    x = _rand_bf16(32, 2048, 22)
    x[5, 100:228] = torch_bf16(np.full(128, 1e-3, np.float32) * np.linspace(-1, 1, 128))
    q, s = orc.act_quant(x)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    sf = np.repeat(s.astype(np.float64), BLOCK, axis=1)
    deq = torch_e4m3_values()[q] * sf
    ratio = np.abs(xf) / sf
    bound = sf * (0.5 * ulp_e4m3(ratio) + 2.0 ** -23 * ratio)
    assert np.all(np.abs(deq - xf) <= bound * (1 + 1e-12))


def pin_act_quant_scale_value(orc):
    """Each scale is the fp32 quotient of the block max |x| and 448 (numpy float32)."""
    x = _rand_bf16(16, 1024, 23, scale=3.0)
    _, s = orc.act_quant(x)
    amax = np.abs(bf16_bits_to_f32(x)).reshape(16, -1, BLOCK).max(axis=2)
    assert np.array_equal(s, (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32))


def pin_act_quant_constant_block(orc):
    """A3: a constant block c gives all codes +-448 and scale |c|/448."""
    for c in (1.0, -3.5, 0.15625, 1000.0, -2.0 ** -6):
        x = torch_bf16(np.full((1, 128), c, np.float32))
        q, s = orc.act_quant(x)
        assert np.all(q == (0xFE if c < 0 else 0x7E)), (c, q[0, :4])
        assert s[0, 0] == np.float32(abs(c)) / np.float32(448.0)


def pin_act_quant_power_of_two(orc):
    """A4: x * 2^k gives the same codes and the scale times 2^k, exactly."""
    x = _rand_bf16(8, 512, 24)
    q0, s0 = orc.act_quant(x)
    for k in (-5, 3, 7):
        xk = torch_bf16(bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        qk, sk = orc.act_quant(xk)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk, (s0 * np.float32(2.0 ** k)).astype(np.float32))


def pin_act_quant_negation(orc):
    """A5: -x flips every code's sign bit and keeps the scales."""
    x = _rand_bf16(8, 512, 25)
    q0, s0 = orc.act_quant(x)
    q1, s1 = orc.act_quant(x ^ np.uint16(0x8000))
    assert np.array_equal(q1, q0 ^ np.uint8(0x80)) and np.array_equal(s1, s0)


def pin_act_quant_row_gather(orc):
    """A6: quantizing gathered rows equals gathering quantized rows."""
    x = _rand_bf16(32, 384, 26)
    idx = np.array([5, 0, 31, 5, 17, 2, 2, 9])
    q, s = orc.act_quant(x)
    qg, sg = orc.act_quant(x[idx])
    assert np.array_equal(qg, q[idx]) and np.array_equal(sg, s[idx])


def pin_act_quant_zero_block(orc):
    """A7: an all-zero block gives zero codes and scale floor/448 (floor value unpinned)."""
    x = np.zeros((2, 256), np.uint16)
    x[1, 128:] = 0x8000                                     # -0.0
    q, s = orc.act_quant(x)
    assert np.all(q[:, :128] == 0) and np.all(q[0, 128:] == 0) and np.all(q[1, 128:] == 0x80)
    floor = np.float32(orc.amax_floor())
    assert floor > 0 and np.all(s == floor / np.float32(448.0))


def pin_act_quant_directed_quotients(orc):
    """The codes come from the IEEE fp32 quotient x/s, not from x * (1/s).

    For several block maxima, every bf16 value of the block's range is tried;
    where the two quotient forms round to different codes, those values are
    packed into blocks (with the maximum in position 0) and the expected codes
    come from numpy's float32 division plus torch's cast.
    """
    allx = bf16_bits_to_f32(np.arange(1 << 16, dtype=np.uint16))
    allx = allx[np.isfinite(allx)]
    found = 0
    for amax in (np.float32(3.0), np.float32(0.7265625), np.float32(11.5), np.float32(97.0)):
        s = np.float32(amax / np.float32(448.0))
        xs = allx[np.abs(allx) <= amax]
        q_div = (xs / s).astype(np.float32)
        q_rcp = (xs * (np.float32(1.0) / s)).astype(np.float32)
        diff = xs[torch_e4m3_cast(np.clip(q_div, -448, 448)) != torch_e4m3_cast(np.clip(q_rcp, -448, 448))]
        if diff.size == 0:
            continue
        found += diff.size
        n = -(-diff.size // 127)
        blocks = np.zeros((n, 128), np.float32)
        blocks[:, 0] = amax
        flat = blocks[:, 1:].reshape(-1)
        flat[:diff.size] = diff
        blocks[:, 1:] = flat.reshape(n, 127)
        xb = torch_bf16(blocks)
        q, sc = orc.act_quant(xb)
        assert np.all(sc == s)
        want = torch_e4m3_cast(np.clip((blocks / s).astype(np.float32), -448, 448))
        assert np.array_equal(q, want), "codes do not follow the fp32 quotient x/s"
    assert found > 0, "no directed near-tie cases found"


# ------------------------------------------------------- weight_dequant pins

def _rand_codes(shape, seed, maxmag=0x7E):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, maxmag + 1, size=shape, dtype=np.int32).astype(np.uint8)
    sign = rng.integers(0, 2, size=shape).astype(np.uint8) << 7
    return c | sign


def _expand(S, N, K):
    return np.repeat(np.repeat(S, BLOCK, axis=0), BLOCK, axis=1)[:N, :K]


def pin_dequant_unit_and_pow2(orc):
    """D1: with S = 1 the output is the code's value in bf16; S = 2^k scales exactly."""
    w = _rand_codes((256, 384), 31)
    vals = torch_e4m3_values()[w].astype(np.float32)
    one = np.ones((2, 3), np.float32)
    assert np.array_equal(orc.weight_dequant(w, one), torch_bf16(vals))
    S = np.float32([[2.0 ** -3, 2.0 ** 5, 1.0], [0.5, 2.0 ** -10, 4.0]])
    assert np.array_equal(orc.weight_dequant(w, S), torch_bf16(vals * _expand(S, 256, 384)))


def pin_dequant_vs_torch(orc):
    """D2: equals torch (code value * expanded scale in fp32, then bf16), ragged edges too."""
    for (N, K, seed) in ((256, 256, 32), (300, 200, 33), (1, 129, 34), (129, 1, 35)):
        w = _rand_codes((N, K), seed)
        rng = np.random.default_rng(seed)
        S = np.exp2(rng.uniform(-10, -2, size=(-(-N // BLOCK), -(-K // BLOCK)))).astype(np.float32)
        vals = torch_e4m3_values()[w].astype(np.float32)
        want = torch_bf16((vals * _expand(S, N, K)).astype(np.float32))
        assert np.array_equal(orc.weight_dequant(w, S), want), (N, K)


# ------------------------------------------------------------------ GEMM pins

def _rand_scales(shape, seed, lo=-8, hi=-2):
    rng = np.random.default_rng(seed)
    return np.exp2(rng.uniform(lo, hi, size=shape)).astype(np.float32)


def _terms_abs(a, sa, b, sb):
    """sum_k |a_k * sa * b_k * sb| in fp64: the natural scale for rounding errors."""
    av = np.abs(torch_e4m3_values()[a]) * np.repeat(sa, BLOCK, axis=1)
    bv = np.abs(torch_e4m3_values()[b]) * np.repeat(np.repeat(sb, BLOCK, axis=0)[:b.shape[0]], BLOCK, axis=1)
    return av @ bv.T


def pin_gemm_fraction_exact(orc):
    """G1: equals an exact rational computation on tiny shapes."""
    vals = torch_e4m3_values()
    cases = ((2, 3, 128, 41, None), (4, 4, 256, 42, None), (3, 130, 128, 43, (0, 1, 127, 128, 129)))
    for (M, N, K, seed, cols) in cases:
        a = _rand_codes((M, K), seed); b = _rand_codes((N, K), seed + 100)
        sa = _rand_scales((M, K // BLOCK), seed + 200)
        sb = _rand_scales((-(-N // BLOCK), K // BLOCK), seed + 300)
        got = orc.gemm(a, sa, b, sb)
        bound = _terms_abs(a, sa, b, sb)
        for m in range(M):
            for n in (cols if cols is not None else range(N)):
                total = Fraction(0)
                for kb in range(K // BLOCK):
                    blk = sum(Fraction(float(vals[a[m, k]])) * Fraction(float(vals[b[n, k]]))
                              for k in range(kb * BLOCK, (kb + 1) * BLOCK))
                    total += blk * Fraction(float(sa[m, kb])) * Fraction(float(sb[n // BLOCK, kb]))
                err = abs(Fraction(float(got[m, n])) - total)
                assert err <= Fraction(1e-14) * Fraction(float(bound[m, n])), (M, N, K, m, n)


def pin_gemm_vs_torch_f64(orc):
    """G2: equals torch float64 (dec(a)*sa) @ (dec(b)*sb)^T, the scales factored into operands."""
    vals = torch.from_numpy(torch_e4m3_values())
    for (M, N, K, seed) in ((16, 256, 256, 51), (37, 300, 384, 52), (5, 1, 128, 53)):
        a = _rand_codes((M, K), seed); b = _rand_codes((N, K), seed + 1)
        sa = _rand_scales((M, K // BLOCK), seed + 2); sb = _rand_scales((-(-N // BLOCK), K // BLOCK), seed + 3)
        A = vals[torch.from_numpy(a).long()] * torch.from_numpy(np.repeat(sa, BLOCK, 1)).double()
        Bs = np.repeat(np.repeat(sb, BLOCK, 0)[:N], BLOCK, 1)
        B = vals[torch.from_numpy(b).long()] * torch.from_numpy(Bs).double()
        ref = (A @ B.T).numpy()
        got = orc.gemm(a, sa, b, sb)
        assert np.all(np.abs(got - ref) <= 1e-12 * _terms_abs(a, sa, b, sb) + 1e-300), (M, N, K)


def pin_gemm_identity(orc):
    """G3: W = identity (code 0x38 = 1.0, S = 1) reproduces dec(q_a) * s_a exactly."""
    K = 256
    a = _rand_codes((16, K), 61); sa = _rand_scales((16, 2), 62)
    b = np.zeros((K, K), np.uint8); np.fill_diagonal(b, 0x38)
    got = orc.gemm(a, sa, b, np.ones((2, 2), np.float32))
    want = torch_e4m3_values()[a] * np.repeat(sa.astype(np.float64), BLOCK, axis=1)
    assert np.array_equal(got, want)


def pin_gemm_one_hot(orc):
    """G4: row n of W is 1.0 at column pi(n); scales 2^k -> dec(q_a[m, pi(n)]) * s_a * 2^k."""
    K, N = 384, 256
    rng = np.random.default_rng(63)
    perm = rng.permutation(K)[:N]
    a = _rand_codes((8, K), 64); sa = _rand_scales((8, 3), 65)
    b = np.zeros((N, K), np.uint8); b[np.arange(N), perm] = 0x38
    ksb = rng.integers(-4, 5, size=(2, 3))
    sb = np.exp2(ksb).astype(np.float32)
    got = orc.gemm(a, sa, b, sb)
    want = torch_e4m3_values()[a[:, perm]] * sa.astype(np.float64)[:, perm // BLOCK] \
        * sb.astype(np.float64)[np.arange(N)[None, :] // BLOCK, perm[None, :] // BLOCK]
    assert np.array_equal(got, want)


def pin_gemm_integer_exact(orc):
    """G5: integer-valued codes with unit scales give the exact integer product."""
    vals = torch_e4m3_values()
    small = np.array([c for c in range(256) if c not in (0x7F, 0xFF)
                      and vals[c] == np.round(vals[c]) and abs(vals[c]) <= 4], np.uint8)
    rng = np.random.default_rng(66)
    M, N, K = 12, 140, 1024
    a = small[rng.integers(0, small.size, (M, K))]; b = small[rng.integers(0, small.size, (N, K))]
    got = orc.gemm(a, np.ones((M, K // BLOCK), np.float32), b,
                   np.ones((2, K // BLOCK), np.float32))
    want = vals[a].astype(np.int64) @ vals[b].astype(np.int64).T
    assert np.array_equal(got, want.astype(np.float64))


def pin_gemm_scale_pow2(orc):
    """G6: multiplying the weight scales by 2^k multiplies the result by 2^k exactly."""
    a = _rand_codes((6, 256), 67); b = _rand_codes((200, 256), 68)
    sa = _rand_scales((6, 2), 69); sb = _rand_scales((2, 2), 70)
    r0 = orc.gemm(a, sa, b, sb)
    r1 = orc.gemm(a, sa, b, (sb * np.float32(2.0 ** 6)).astype(np.float32))
    assert np.array_equal(r1, r0 * 2.0 ** 6)


def pin_fp8_vs_bf16_branch(orc):
    """G7: the FP8 branch (act_quant then gemm) and the exact linear map x * (dec(W) S)^T
    differ by at most the activation-quantization error sum_k |x_k - dec(q_k) s| |w_k S|."""
    M, N, K = 8, 256, 512
    x = _rand_bf16(M, K, 71)
    w = _rand_codes((N, K), 72)
    S = _rand_scales((2, 4), 73)
    q, s = orc.act_quant(x)
    got = orc.gemm(q, s, w, S)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    wf = torch_e4m3_values()[w] * _expand(S, N, K).astype(np.float64)
    exact = xf @ wf.T
    sf = np.repeat(s.astype(np.float64), BLOCK, 1)
    ratio = np.abs(xf) / sf
    per_elem = sf * (0.5 * ulp_e4m3(ratio) + 2.0 ** -23 * ratio)
    bound = per_elem @ np.abs(wf).T
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9) + 1e-12 * (np.abs(xf) @ np.abs(wf).T))


def pin_gemm_brute_force(orc):
    """G8: plain loops in fp64 over random tiny shapes (ragged N)."""
    vals = torch_e4m3_values()
    rng = np.random.default_rng(81)
    for t in range(4):
        M = int(rng.integers(1, 5))
        N = int(rng.integers(1, 9)) + 125 * (t % 2)
        K = 128 * int(rng.integers(1, 4))
        a = _rand_codes((M, K), 82 + t); b = _rand_codes((N, K), 92 + t)
        sa = _rand_scales((M, K // BLOCK), 102 + t)
        sb = _rand_scales((-(-N // BLOCK), K // BLOCK), 112 + t)
        got = orc.gemm(a, sa, b, sb)
        bound = 1e-13 * _terms_abs(a, sa, b, sb)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for kb in range(K // BLOCK):
                    blk = 0.0
                    for k in range(kb * BLOCK, kb * BLOCK + BLOCK):
                        blk += vals[a[m, k]] * vals[b[n, k]]
                    acc += blk * float(sa[m, kb]) * float(sb[n // BLOCK, kb])
                assert abs(got[m, n] - acc) <= bound[m, n], (M, N, K, m, n)


def pin_gemm_row_subset(orc):
    """Computing a subset of rows gives exactly those rows of the full result."""
    a = _rand_codes((20, 256), 121); b = _rand_codes((130, 256), 122)
    sa = _rand_scales((20, 2), 123); sb = _rand_scales((2, 2), 124)
    full = orc.gemm(a, sa, b, sb)
    rows = np.array([19, 0, 7, 7])
    assert np.array_equal(orc.gemm(a, sa, b, sb, rows=rows), full[rows])


# --------------------------------------------------------------- grouped pins

def pin_grouped_reduces_to_gemm(orc):
    """R1: grouped == per-group plain GEMMs (torch f64 cross-check); G=1 == gemm; empty groups."""
    K, N = 256, 200
    counts = [3, 0, 5, 1, 0, 4]
    G = len(counts)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    a = _rand_codes((T, K), 131); sa = _rand_scales((T, 2), 132)
    b = _rand_codes((G, N, K), 133); sb = _rand_scales((G, 2, 2), 134)
    got = orc.gemm_grouped(a, sa, b, sb, off)
    vals = torch.from_numpy(torch_e4m3_values())
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        if hi == lo:
            continue
        A = vals[torch.from_numpy(a[lo:hi]).long()] * torch.from_numpy(np.repeat(sa[lo:hi], BLOCK, 1)).double()
        B = vals[torch.from_numpy(b[g]).long()] * torch.from_numpy(np.repeat(np.repeat(sb[g], BLOCK, 0)[:N], BLOCK, 1)).double()
        ref = (A @ B.T).numpy()
        assert np.all(np.abs(got[lo:hi] - ref) <= 1e-12 * _terms_abs(a[lo:hi], sa[lo:hi], b[g], sb[g]) + 1e-300), g
    one = orc.gemm_grouped(a, sa, b[:1], sb[:1], np.array([0, T], np.int32))
    assert np.array_equal(one, orc.gemm(a, sa, b[0], sb[0]))
    # a row that belongs to no group (offsets ending early) is reported as NaN
    partial = orc.gemm_grouped(a, sa, b[:2], sb[:2], np.array([0, 2, 4], np.int32))
    assert np.all(np.isnan(partial[4:])) and not np.any(np.isnan(partial[:4]))


# ------------------------------------------------------------- BF16 branch pins
#
# Source: pyshine "DeepSeek-V3" tour, "FP8 with per-block scales": the other
# branch of linear() dequantizes the weight and runs an ordinary BF16 matmul.

def _rand_bf16_bits(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return torch_bf16((rng.standard_normal(shape) * scale).astype(np.float32)).reshape(shape)


def pin_gemm_bf16_exact_rational(orc):
    """B1: bf16 GEMM == the exact rational sum (fractions), up to one fp64 rounding per term."""
    a = _rand_bf16_bits((3, 40), 1001)
    b = _rand_bf16_bits((5, 40), 1002, 3.0)
    got = orc.gemm_bf16(a, b)
    av, bv = bf16_bits_to_f32(a).astype(np.float64), bf16_bits_to_f32(b).astype(np.float64)
    for i in range(3):
        for n in range(5):
            exact = sum(Fraction(float(av[i, k])) * Fraction(float(bv[n, k])) for k in range(40))
            bound = 1e-15 * float(np.sum(np.abs(av[i] * bv[n])))
            assert abs(got[i, n] - float(exact)) <= bound, (i, n)


def pin_gemm_bf16_identity_and_integers(orc):
    """B2: identity weight returns A exactly; integer-valued operands give exact integer sums."""
    a = _rand_bf16_bits((6, 32), 1003)
    eye = torch_bf16(np.eye(32, dtype=np.float32))
    assert np.array_equal(orc.gemm_bf16(a, eye), bf16_bits_to_f32(a).astype(np.float64))
    rng = np.random.default_rng(1004)
    ai = rng.integers(-100, 100, size=(4, 96)).astype(np.float32)
    bi = rng.integers(-100, 100, size=(9, 96)).astype(np.float32)
    got = orc.gemm_bf16(torch_bf16(ai).reshape(4, 96), torch_bf16(bi).reshape(9, 96))
    assert np.array_equal(got, ai.astype(np.int64) @ bi.astype(np.int64).T)


def pin_bf16_branch_vs_torch(orc):
    """B3: x @ dequant(W)^T through the oracle == torch float64 matmul of the same bf16 values
    (ragged N and K, several rows), and the row subset computes the same rows."""
    N, K, M = 200, 320, 7
    w = _rand_codes((N, K), 1005)
    S = _rand_scales((-(-N // BLOCK), -(-K // BLOCK)), 1006)
    wd = orc.weight_dequant(w, S)                          # bf16 bits [N, K]
    x = _rand_bf16_bits((M, K), 1007)
    got = orc.gemm_bf16(x, wd)
    ref = (torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64)) @
           torch.from_numpy(bf16_bits_to_f32(wd).astype(np.float64)).T).numpy()
    tol = 1e-13 * (np.abs(bf16_bits_to_f32(x)).astype(np.float64) @ np.abs(bf16_bits_to_f32(wd)).astype(np.float64).T)
    assert np.all(np.abs(got - ref) <= tol)
    rows = np.array([6, 0, 3])
    assert np.array_equal(orc.gemm_bf16(x, wd, rows=rows), got[rows])


# ------------------------------------------------------------ gated FFN pins
#
# The gated FFN's activation is not printed on the pages; the oracle's reading
# is SiLU (pinned here against torch's own silu), with the bf16 rounding steps
# of a bf16 model.

def pin_swiglu_vs_torch_silu(orc):
    """G1: with u = 1 the gate output is bf16(silu(bf16 g)), torch's float64 silu rounded by torch."""
    rng = np.random.default_rng(1100)
    g = np.concatenate([rng.standard_normal(4000) * 4, [0.0, -0.0, 30.0, -30.0, 1e-3, -1e-3]])
    h = orc.swiglu_bf16(g, np.ones_like(g))
    gb = torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16).double()
    ref = torch.nn.functional.silu(gb).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)


def pin_swiglu_bf16_model_steps(orc):
    """G3: random g, u through torch's bf16 ops: silu(bf16 g) rounded to bf16 by torch, times
    bf16 u (exact in fp32), rounded to bf16 by torch."""
    rng = np.random.default_rng(1102)
    g, u = rng.standard_normal(5000) * 3, rng.standard_normal(5000) * 2
    h = orc.swiglu_bf16(g, u)
    gb = torch.from_numpy(g.astype(np.float32)).to(torch.bfloat16)
    ub = torch.from_numpy(u.astype(np.float32)).to(torch.bfloat16)
    sg = torch.nn.functional.silu(gb.double()).float().to(torch.bfloat16)
    ref = (sg.float() * ub.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(h, ref)


def pin_swiglu_identities(orc):
    """G2: silu(x) - silu(-x) = x within the roundings; zero gate or zero up gives 0; the
    product with an exact power-of-two u is exact."""
    rng = np.random.default_rng(1101)
    x = rng.standard_normal(2000) * 3
    hp = bf16_bits_to_f32(orc.swiglu_bf16(x, np.ones_like(x))).astype(np.float64)
    hm = bf16_bits_to_f32(orc.swiglu_bf16(-x, np.ones_like(x))).astype(np.float64)
    xb = bf16_bits_to_f32(torch_bf16(x.astype(np.float32))).astype(np.float64)
    assert np.all(np.abs((hp - hm) - xb) <= 2.0 ** -7 * (np.abs(hp) + np.abs(hm)) + 1e-30)
    assert np.all(orc.swiglu_bf16(np.zeros(5), rng.standard_normal(5)) & 0x7FFF == 0)
    assert np.all(orc.swiglu_bf16(rng.standard_normal(5), np.zeros(5)) & 0x7FFF == 0)
    h1 = bf16_bits_to_f32(orc.swiglu_bf16(x, np.ones_like(x))).astype(np.float64)
    h4 = bf16_bits_to_f32(orc.swiglu_bf16(x, np.full_like(x, 4.0))).astype(np.float64)
    assert np.array_equal(h4, 4.0 * h1)


# ------------------------------------------------------- power-of-two scale pins
#
# scale_fmt is a ModelArgs field whose meaning the pages do not give; the
# oracle's reading is "scale rounded up to a power of two".  These pins tie the
# oracle to that reading through independent numpy/torch arithmetic.

def pin_act_quant_pow2_vs_numpy(orc):
    """P1: scale = 2^ceil(log2(fl32(max(amax, 1e-4) / 448))) (numpy), codes = torch's e4m3 cast
    of x / scale (exact: a power-of-two division), with outliers, tiny and zero blocks."""
    rng = np.random.default_rng(1300)
    x = rng.standard_normal((12, 640)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (12, 1)))
    x[3, :128] = 0.0
    x[4, 128:256] = 1e-6
    x[5, 5] = 3e4
    xb = torch_bf16(x).reshape(x.shape)
    q, s = orc.act_quant_pow2(xb)
    xf = bf16_bits_to_f32(xb).reshape(12, 5, 128)
    amax = np.abs(xf).max(axis=2)
    y = (np.maximum(amax, np.float32(1e-4)) / np.float32(448.0)).astype(np.float32)
    s_ref = np.exp2(np.ceil(np.log2(y.astype(np.float64)))).astype(np.float32)
    assert np.array_equal(s, s_ref)
    codes = torch_e4m3_cast((xf / s_ref[:, :, None]).reshape(12, 640))
    assert np.array_equal(q, codes.reshape(12, 640))


def pin_act_quant_pow2_bounds(orc):
    """P2: the power-of-two scale is within [y, 2y) of the plain scale y, and no code
    saturates below the block max (max |code value| <= 448, > 224)."""
    x = _rand_bf16(20, 384, 1301)
    q, s = orc.act_quant_pow2(x)
    q0, s0 = orc.act_quant(x)
    assert np.all(s >= s0) and np.all(s < 2 * s0)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)
    vals = torch_e4m3_values()[q].reshape(20, 3, 128)
    mx = np.abs(vals).max(axis=2)
    assert np.all(mx <= 448.0) and np.all(mx > 224.0 - 1e-9)


def _e4m3_brute(v: Fraction) -> int:
    """e4m3 magnitude code of the exact value v by search: the nearest of the 127 finite
    magnitudes, ties to the even code, saturating at 448 (written from the OCP format,
    independently of the oracle's encoder); the caller adds the sign bit."""
    mags = []
    for c in range(127):
        e, m = c >> 3, c & 7
        mags.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    a = abs(v)
    return min(range(127), key=lambda c: (abs(mags[c] - a), c & 1))


def pin_act_quant_pow2_exact_rational(orc):
    """P3: act_quant with power-of-two scales against exact rational arithmetic: y is the
    fp32-rounded max(amax, 1e-4f) / 448, the scale the smallest power of two >= y found by
    stepping exponents, and each code the brute-force nearest e4m3 value of x / scale
    (exact, a power-of-two division).  Blocks: random, a max of exactly 448 * 2^-5 (y is
    itself a power of two, so the scale equals y), a block below the floor, a zero block."""
    rng = np.random.default_rng(1302)
    x = (rng.standard_normal((3, 256)) * 3).astype(np.float32)
    x[1, :128] = (rng.standard_normal(128) * 2).astype(np.float32).clip(-13, 13)
    x[1, 7] = 14.0                                    # 448 * 2^-5
    x[1, 128:256] = (rng.standard_normal(128) * 1e-6).astype(np.float32)
    x[2, 128:256] = 0.0
    xb = torch_bf16(x).reshape(x.shape)
    q, s = orc.act_quant_pow2(xb)
    xf = bf16_bits_to_f32(xb)
    floor32 = Fraction(float(np.float32(1e-4)))
    for m in range(3):
        for kb in range(2):
            blk = [Fraction(float(v)) for v in xf[m, 128 * kb:128 * kb + 128]]
            amax = max(abs(v) for v in blk)
            y = Fraction(float(np.float32(float(max(amax, floor32) / 448))))   # one fp32 rounding
            k = -200
            while Fraction(2) ** k < y:
                k += 1
            scale = Fraction(2) ** k
            assert Fraction(float(s[m, kb])) == scale, (m, kb, float(s[m, kb]), float(scale))
            for j, v in enumerate(blk):
                want = _e4m3_brute(v / scale)
                if v < 0:
                    want |= 0x80
                assert q[m, 128 * kb + j] == want, (m, kb, j)
    assert float(s[1, 0]) == 2.0 ** -5


# ------------------------------------------------------ MoE dispatch / combine pins
#
# Source: "Behavior traces - deepseek-ai/DeepSeek-V3" (codevetter), MoE trace
# bullet (per local expert with tokens: select the tokens routed to it in
# ascending order, add expert(x[idx]) times the routing weight into y, which
# starts at zero); "Data flow" (codevetter), expert sharding (a GPU holds a
# contiguous range of expert ids).

def _read_moe_golden():
    lines = [ln.split() for ln in open(os.path.join(GOLDEN, "moe_dispatch_combine_hand.txt"))
             if ln.strip() and not ln.startswith("#")]
    common, cases = {}, []
    for key, *vals in lines:
        if key == "case":
            cases.append({"expert_lo": int(vals[0]), "G": int(vals[1])})
        elif cases and key in ("offsets", "row_token", "slot_row"):
            cases[-1][key] = np.array(vals, np.int64)
        else:
            common[key] = np.array(vals, np.float64)
    return common, cases


def _routing_table(T, k, n_experts, seed, distinct=True):
    rng = np.random.default_rng(seed)
    if distinct:
        return np.argsort(rng.random((T, n_experts)), axis=1)[:, :k].astype(np.int32)
    return rng.integers(-3, n_experts + 3, size=(T, k)).astype(np.int32)


def _dispatch_by_stable_sort(topk, lo, G):
    """Independent construction: a stable argsort of the flat (token, slot) list by local expert id."""
    T, k = topk.shape
    flat = topk.astype(np.int64).ravel()
    local = (flat >= lo) & (flat < lo + G)
    key = np.where(local, flat - lo, G)                 # non-local entries sort last
    order = np.argsort(key, kind="stable")[:int(local.sum())]
    counts = np.bincount(flat[local] - lo, minlength=G)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot_row = np.full(T * k, -1, np.int64)
    slot_row[order] = np.arange(order.size)
    return offsets, order // k, slot_row.reshape(T, k)


def pin_moe_dispatch_golden(orc):
    """M1: the hand-worked dispatch of four tokens, two expert ranges."""
    common, cases = _read_moe_golden()
    topk = common["topk"].astype(np.int32).reshape(int(common["T"][0]), int(common["k"][0]))
    for c in cases:
        off, rt, sr = orc.moe_dispatch(topk, c["expert_lo"], c["G"])
        assert np.array_equal(off, c["offsets"]), c
        assert np.array_equal(rt, c["row_token"]), c
        assert np.array_equal(sr.ravel(), c["slot_row"]), c


def pin_moe_dispatch_vs_stable_sort(orc):
    """M2: dispatch == a stable sort by expert id (numpy argsort + bincount), any expert range."""
    for seed, (T, k, E, lo, G, distinct) in enumerate(
            [(300, 8, 64, 16, 24, True), (97, 6, 40, 0, 40, True), (128, 4, 10, 3, 5, False),
             (50, 8, 256, 200, 56, True), (64, 2, 8, 8, 4, True)]):
        topk = _routing_table(T, k, E, 900 + seed, distinct)
        off, rt, sr = orc.moe_dispatch(topk, lo, G)
        ref_off, ref_rt, ref_sr = _dispatch_by_stable_sort(topk, lo, G)
        assert np.array_equal(off, ref_off) and np.array_equal(rt, ref_rt) and np.array_equal(sr, ref_sr)
        # invariants: each local slot owns one row, that row names the slot's token,
        # and rows of an expert hold ascending tokens
        rows = sr[sr >= 0]
        assert np.array_equal(np.sort(rows), np.arange(off[-1]))
        t_of = np.nonzero(sr >= 0)[0]
        assert np.array_equal(rt[sr[sr >= 0]], t_of)
        for g in range(G):
            assert np.all(np.diff(rt[off[g]:off[g + 1]]) >= 0)


def pin_moe_dispatch_degenerate(orc):
    """M3: no local expert hit, every slot local, a single token."""
    topk = _routing_table(20, 4, 16, 950)
    off, rt, sr = orc.moe_dispatch(topk, 16, 8)             # experts 16..23 do not exist
    assert np.all(off == 0) and rt.size == 0 and np.all(sr == -1)
    off, rt, sr = orc.moe_dispatch(topk, 0, 16)             # every expert is local
    assert off[-1] == 80 and np.array_equal(np.sort(sr.ravel()), np.arange(80))
    off, rt, sr = orc.moe_dispatch(np.array([[5, 2, 7]], np.int32), 2, 6)
    assert np.array_equal(off, [0, 1, 1, 1, 2, 2, 3]) and np.array_equal(rt, [0, 0, 0])
    assert np.array_equal(sr, [[1, 0, 2]])


def pin_moe_combine_golden(orc):
    """M4: the hand-worked combine of the golden file (exact in fp64)."""
    common, cases = _read_moe_golden()
    T, k, N = int(common["T"][0]), int(common["k"][0]), int(common["N"][0])
    topk = common["topk"].astype(np.int32).reshape(T, k)
    _, _, sr = orc.moe_dispatch(topk, cases[0]["expert_lo"], cases[0]["G"])
    out = torch_bf16(common["out"].astype(np.float32)).reshape(-1, N)
    y = orc.moe_combine(out, sr, common["weights"].astype(np.float32).reshape(T, k))
    assert np.array_equal(y.ravel(), common["y"])


def pin_moe_combine_vs_dense_matmul(orc):
    """M5: combine == R @ out with R[t, slot_row[t, j]] = weight[t, j] (numpy fp64 matmul)."""
    T, k, E, lo, G, N = 120, 8, 64, 8, 20, 72
    topk = _routing_table(T, k, E, 960)
    _, _, sr = orc.moe_dispatch(topk, lo, G)
    rows = int((sr >= 0).sum())
    rng = np.random.default_rng(961)
    out = torch_bf16(rng.standard_normal((rows, N)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    R = np.zeros((T, rows))
    for t in range(T):
        for j in range(k):
            if sr[t, j] >= 0:
                R[t, sr[t, j]] += w[t, j]
    ref = R @ bf16_bits_to_f32(out).astype(np.float64)
    y = orc.moe_combine(out, sr, w)
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(R) @ np.abs(bf16_bits_to_f32(out).astype(np.float64))) + 1e-300)


def pin_moe_layer_matches_per_expert_loop(orc):
    """M6: dispatch -> per-expert function on gathered rows -> combine == the pages' loop.

    The expert of id e is x -> 2**(e % 5 - 2) * x (exact in bf16 for these inputs), so
    the loop over local experts with where(indices == e) can be written in plain
    numpy and compared exactly."""
    T, k, E, lo, G, N = 90, 6, 32, 4, 12, 16
    topk = _routing_table(T, k, E, 970)
    rng = np.random.default_rng(971)
    x = rng.integers(-64, 64, size=(T, N)).astype(np.float32)
    w = (rng.integers(1, 16, size=(T, k)) / 16.0).astype(np.float32)
    off, rt, sr = orc.moe_dispatch(topk, lo, G)
    out = np.empty((int(off[-1]), N), np.float32)
    for g in range(G):
        out[off[g]:off[g + 1]] = x[rt[off[g]:off[g + 1]]] * np.float32(2.0 ** ((lo + g) % 5 - 2))
    y = orc.moe_combine(torch_bf16(out), sr, w)
    ref = np.zeros((T, N))
    for e in range(lo, lo + G):
        idx, top = np.nonzero(topk == e)
        if idx.size == 0:
            continue
        ref[idx] += (x[idx].astype(np.float64) * 2.0 ** (e % 5 - 2)) * w[idx, top][:, None]
    assert np.array_equal(y, ref)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
