"""Plants plausible mistakes in copies of the CPU oracle and checks that the pins catch each.

Every mutant is a text edit of ``oracle/bfp8_oracle.cpp`` compiled into a
temporary folder; the real oracle is never touched.  A mutant survives only if
every pin in tests/pins.py still passes, which would mean the pins cannot tell
that mistake from the method.
"""
import os
import subprocess

import pytest

import oracle
import pins
from oracle import build as oracle_build

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "bfp8_oracle.cpp")

MUTANTS = {
    # power-of-two scale rounded down instead of up
    "pow2_round_down": ("float scale = (float)ldexp(1.0, f == 0.5 ? e - 1 : e);", "float scale = (float)ldexp(1.0, e - 1);"),
    # power-of-two scale one octave too large for exact powers
    "pow2_exact_power": ("float scale = (float)ldexp(1.0, f == 0.5 ? e - 1 : e);", "float scale = (float)ldexp(1.0, e);"),
    # gated FFN: sigmoid of the wrong sign
    "swiglu_sign": ("const double sg = gb / (1.0 + exp(-gb));", "const double sg = gb / (1.0 + exp(gb));"),
    # gated FFN: the activation's bf16 rounding skipped
    "swiglu_no_round": ("h[i] = oracle_f32_to_bf16((float)(sgb * ub));", "h[i] = oracle_f32_to_bf16((float)(sg * ub));"),
    # bf16 GEMM: weight row stride lost
    "bf16_gemm_row_stride": ("const uint16_t* b = J->b + n * J->K;", "const uint16_t* b = J->b + n;"),
    # bf16 GEMM: fp32 accumulation
    "bf16_gemm_float_sum": ("double sum = 0.0;\n            for (int64_t k = 0; k < J->K; ++k) sum += arow[k]",
                            "float sum = 0.0f;\n            for (int64_t k = 0; k < J->K; ++k) sum += arow[k]"),
    # bf16 GEMM: last K element dropped
    "bf16_gemm_short_k": ("for (int64_t k = 0; k < J->K; ++k) sum += arow[k]", "for (int64_t k = 0; k + 1 < J->K; ++k) sum += arow[k]"),
    # dispatch: slots ordered slot-major instead of token-major inside an expert
    "dispatch_slot_major": ("for (int64_t t = 0; t < T; ++t)\n            for (int32_t j = 0; j < k; ++j)\n                if (topk",
                            "for (int32_t j = 0; j < k; ++j)\n            for (int64_t t = 0; t < T; ++t)\n                if (topk"),
    # dispatch: local range taken to start at expert 0
    "dispatch_ignores_lo": ("if (topk[t * k + j] == expert_lo + g)", "if (topk[t * k + j] == g)"),
    # dispatch: non-local slots marked 0 instead of -1
    "dispatch_nonlocal_zero": ("for (int64_t i = 0; i < T * k; ++i) slot_row[i] = -1;",
                               "for (int64_t i = 0; i < T * k; ++i) slot_row[i] = 0;"),
    # combine: routing weight dropped
    "combine_no_weight": ("acc += (double)weight[t * k + j] * (double)", "acc += (double)"),
    # combine: weight of the first slot used for every slot
    "combine_weight_index": ("(double)weight[t * k + j]", "(double)weight[t * k]"),
    # combine: reads the token's own row instead of the slot's gathered row
    "combine_row_index": ("oracle_bf16_to_f32(out[(int64_t)r * N + n])", "oracle_bf16_to_f32(out[(int64_t)t * N + n])"),
    # quantizer ceiling of a different fp8 flavour (e4m3 "fnuz" tops out at 240)
    "ceiling_240": ("float scale = clamped / ORACLE_E4M3_MAX;", "float scale = clamped / 240.0f;"),
    # no floor on the block max: an all-zero block divides by zero
    "no_floor": ("float scale = clamped / ORACLE_E4M3_MAX;", "float scale = amax / ORACLE_E4M3_MAX;"),
    # quotient through a reciprocal instead of an fp32 division
    "reciprocal_quotient": ("oracle_bf16_to_f32(xb[j]) / scale;", "oracle_bf16_to_f32(xb[j]) * (1.0f / scale);"),
    # ties away from zero instead of to even
    "ties_away": ("(frac == 0.5 && fmod(n, 2.0) != 0.0)", "(frac == 0.5)"),
    # overflow to the NaN code instead of saturating
    "no_saturation": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 464.0) return sign | 0x7F;"),
    # sign of zero lost
    "unsigned_zero": ("if (mag == 0.0) return sign;", "if (mag == 0.0) return 0;"),
    # exponent bias off by one in decode
    "decode_bias": ("ldexpf(1.0f + (float)m / 8.0f, E - 7)", "ldexpf(1.0f + (float)m / 8.0f, E - 8)"),
    # subnormal spacing wrong in decode
    "decode_subnormal": ("ldexpf((float)m, -9)", "ldexpf((float)m, -10)"),
    # block max taken without the absolute value
    "signed_amax": ("float a = fabsf(oracle_bf16_to_f32(xb[j]));", "float a = oracle_bf16_to_f32(xb[j]);"),
    # bf16 rounding: ties away
    "bf16_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    # bf16 rounding: truncation
    "bf16_truncate": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;", ""),
    # dequant uses the first k-block's scale for the whole row
    "dequant_scale_index": ("S[(n / ORACLE_BLOCK) * KB + k / ORACLE_BLOCK]", "S[(n / ORACLE_BLOCK) * KB]"),
    # dequant divides by the scale (the other reading of scale_inv)
    "dequant_divides": ("oracle_e4m3_decode(w[n * K + k]) * scale;", "oracle_e4m3_decode(w[n * K + k]) / scale;"),
    # GEMM drops the activation scale
    "gemm_no_sa": ("total += block_sum * (double)J->sa[m * KB + kb]", "total += block_sum * 1.0"),
    # GEMM reads the activation scale of the first block only
    "gemm_sa_index": ("(double)J->sa[m * KB + kb]", "(double)J->sa[m * KB]"),
    # GEMM weight-scale row taken from k instead of n
    "gemm_sb_index": ("(double)sb[(n / ORACLE_BLOCK) * KB + kb]", "(double)sb[kb]"),
    # GEMM weight column instead of row (transposed operand on a square weight)
    "gemm_transposed_b": ("(double)J->table[brow[k]]", "(double)J->table[b[(k % J->N) * J->K + n % J->K]]"),
    # grouped: row at an upper offset counted in the group
    "grouped_off_by_one": ("m >= J->off[h] && m < J->off[h + 1]", "m >= J->off[h] && m <= J->off[h + 1]"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation target for {name} not found"
    mutated = src.replace(old, new)
    c_path = mutant_dir / f"{name}.cpp"
    so_path = mutant_dir / f"lib_{name}.so"
    c_path.write_text(mutated)
    subprocess.run(oracle_build.compile_cmd(str(c_path), str(so_path), ["-w"]), check=True)
    orc = oracle.Oracle(str(so_path))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except Exception:            # an assertion, or an error the mistake provoked
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passes every pin"
