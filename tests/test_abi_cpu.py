"""C ABI checks that need no GPU: the library loads, exports every entry point that
include/bfp8.h declares, and rejects bad arguments with the documented status code
before making any HIP call (so no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import block_scaled_fp8_04_amd as bfp8
from block_scaled_fp8_04_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bfp8.h")

P = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x10000)           # aligned, never dereferenced: every call below is rejected
ODD = ctypes.c_void_p(0x10001)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(bfp8_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY):
        pytest.fail("libbfp8.so is not built (run __graft_entry__.build())")
    return _lib.library()


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("bfp8_act_quant", "bfp8_weight_dequant", "bfp8_gemm", "bfp8_gemm_grouped",
              "bfp8_gemm_workspace_size", "bfp8_status_string", "bfp8_version"):
        assert n in names
    assert set(names) == set(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in bfp8.h but not exported"


def test_version_and_status_strings(lib):
    assert bfp8.bfp8_version() == 8
    for code in range(9):
        assert bfp8.bfp8_status_string(code)
    assert bfp8.bfp8_status_string(0) == "ok"
    assert "unknown" in bfp8.bfp8_status_string(99)


def test_act_quant_validation(lib):
    f = lib.bfp8_act_quant
    assert f(FAKE, FAKE, FAKE, 4, 100, None) == _lib.BFP8_ERR_SHAPE     # K % 128
    assert f(FAKE, FAKE, FAKE, 4, 0, None) == _lib.BFP8_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, -1, 128, None) == _lib.BFP8_ERR_SHAPE
    assert f(None, FAKE, FAKE, 4, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, None, FAKE, 4, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, FAKE, None, 4, 128, None) == _lib.BFP8_ERR_NULL
    assert f(ODD, FAKE, FAKE, 4, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(FAKE, ctypes.c_void_p(0x10008), FAKE, 4, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(FAKE, FAKE, ctypes.c_void_p(0x10002), 4, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(None, None, None, 0, 128, None) == _lib.BFP8_OK               # empty: no launch


def test_weight_dequant_validation(lib):
    f = lib.bfp8_weight_dequant
    assert f(FAKE, FAKE, FAKE, -1, 128, None) == _lib.BFP8_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 128, -5, None) == _lib.BFP8_ERR_SHAPE
    assert f(None, FAKE, FAKE, 128, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, None, FAKE, 128, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, FAKE, None, 128, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, FAKE, ODD, 128, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(FAKE, ctypes.c_void_p(0x10002), FAKE, 128, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(None, None, None, 0, 128, None) == _lib.BFP8_OK
    assert f(None, None, None, 128, 0, None) == _lib.BFP8_OK


def test_gemm_validation(lib):
    f = lib.bfp8_gemm
    ok = dict(M=64, N=64, K=256)

    def call(a=FAKE, a_s=FAKE, b=FAKE, b_s=FAKE, c=FAKE, M=64, N=64, K=256, ws=None, wsb=0):
        return f(a, a_s, b, b_s, c, M, N, K, ws, wsb, None)

    assert call(K=200) == _lib.BFP8_ERR_SHAPE
    assert call(K=0) == _lib.BFP8_ERR_SHAPE
    assert call(M=-1) == _lib.BFP8_ERR_SHAPE
    assert call(N=-1) == _lib.BFP8_ERR_SHAPE
    for name in ("a", "a_s", "b", "b_s", "c"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(a=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(b=ctypes.c_void_p(0x10004)) == _lib.BFP8_ERR_ALIGN
    assert call(a_s=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(c=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(ws=ODD, wsb=1 << 20) == _lib.BFP8_ERR_ALIGN
    assert call(a=None, M=0) == _lib.BFP8_OK
    assert call(a=None, N=0) == _lib.BFP8_OK
    del ok


def test_gemm_workspace_contract(lib):
    for (M, N, K) in ((64, 1536, 7168), (16, 256, 256), (8192, 18432, 7168), (1, 1, 128)):
        need = bfp8.bfp8_gemm_workspace_size(M, N, K)
        assert need >= 0 and need % 16 == 0
        if need > 0:
            rc = lib.bfp8_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, FAKE, need - 16, None)
            assert rc == _lib.BFP8_ERR_WORKSPACE
    assert bfp8.bfp8_gemm_workspace_size(0, 5, 128) == 0
    assert bfp8.bfp8_gemm_workspace_size(5, 5, 100) == 0


def test_gemm_tail_split_plan():
    """The workspace a large GEMM asks for: only when its 256 x 256 tiles leave a last round
    (of 256 CUs) at most half full that is whole tile columns, and K has at least 80 blocks;
    then 2 halves x M x (tail columns) fp32 partial sums."""
    ws = bfp8.bfp8_gemm_workspace_size
    # dense down projection: 32 x 28 tiles = 3.5 rounds, tail = 4 tile columns
    assert ws(8192, 7168, 18432) == 2 * 8192 * 4 * 256 * 4
    assert ws(8192, 5120, 18432) == 2 * 8192 * 4 * 256 * 4       # 2.5 rounds
    assert ws(8192, 7168, 10240) == 2 * 8192 * 4 * 256 * 4       # exactly 80 K blocks
    assert ws(8192, 7168, 10112) == 0                               # 79 K blocks
    assert ws(8192, 7168, 7168) == 0
    assert ws(8192, 18432, 7168) == 0                               # 9 whole rounds
    assert ws(8192, 6144, 18432) == 0                               # 3 whole rounds
    assert ws(4096, 7168, 18432) == 0                               # 1.75 rounds: tail too full
    assert ws(512, 33024, 10240) == 2 * 512 * 1 * 256 * 4           # 2 x 129 tiles
    assert ws(2048, 8448, 10368) == 2 * 2048 * 1 * 256 * 4          # 8 x 33 tiles, 81 K blocks
    assert ws(8192 + 128, 7168, 18432) == 0                         # M not a multiple of 256
    assert ws(8192, 7168 + 128, 18432) == 0                         # N not a multiple of 256
    assert ws(512, 512, 18432) == 0                                 # less than one round


def test_gemm_skinny_split_plan():
    """Split-K (splits x M x N fp32 partial sums) for M <= 64, and for M <= 256 only when the
    problem makes at most 32 output tiles of 128 x 128."""
    ws = bfp8.bfp8_gemm_workspace_size
    assert ws(64, 18432, 7168) > 0
    assert ws(128, 2048, 7168) > 0                                  # 1 x 16 tiles
    assert ws(128, 4096, 7168) > 0                                  # 1 x 32 tiles
    assert ws(128, 4224, 7168) == 0                                 # 1 x 33 tiles
    assert ws(256, 2048, 7168) > 0                                  # 2 x 16 tiles
    assert ws(256, 4096, 7168) == 0                                 # 2 x 32 tiles
    assert ws(257, 128, 7168) == 0                                  # M > 256
    for (M, N, K) in ((128, 2048, 7168), (256, 1536, 7168), (37, 300, 1152)):
        need = ws(M, N, K)
        assert need % (M * N * 4) == 0 and need // (M * N * 4) >= 2


def test_gemm_grouped_validation(lib):
    f = lib.bfp8_gemm_grouped

    def call(a=FAKE, a_s=FAKE, b=FAKE, b_s=FAKE, c=FAKE, off=FAKE, G=4, T=100, N=256, K=256):
        return f(a, a_s, b, b_s, c, off, G, T, N, K, None)

    assert call(K=100) == _lib.BFP8_ERR_SHAPE
    assert call(T=-1) == _lib.BFP8_ERR_SHAPE
    assert call(G=0) == _lib.BFP8_ERR_GROUPS
    assert call(G=-3) == _lib.BFP8_ERR_GROUPS
    for name in ("a", "a_s", "b", "b_s", "c", "off"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(off=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(a=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(a=None, T=0) == _lib.BFP8_OK


def test_gemm_act_quant_validation(lib):
    f = lib.bfp8_gemm_act_quant

    def call(a=FAKE, a_s=FAKE, b=FAKE, b_s=FAKE, q=FAKE, qs=FAKE, M=64, N=256, K=256):
        return f(a, a_s, b, b_s, q, qs, M, N, K, None)

    assert call(N=200) == _lib.BFP8_ERR_SHAPE          # N % 128
    assert call(K=100) == _lib.BFP8_ERR_SHAPE
    assert call(M=-1) == _lib.BFP8_ERR_SHAPE
    for name in ("a", "a_s", "b", "b_s", "q", "qs"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(q=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(a=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(a=None, M=0) == _lib.BFP8_OK


def test_gemm_swiglu_act_quant_validation(lib):
    f = lib.bfp8_gemm_swiglu_act_quant

    def call(a=FAKE, a_s=FAKE, w=FAKE, s=FAKE, q=FAKE, qs=FAKE, M=64, N=256, K=256):
        return f(a, a_s, w, s, q, qs, M, N, K, None)

    assert call(N=192) == _lib.BFP8_ERR_SHAPE
    assert call(K=64) == _lib.BFP8_ERR_SHAPE
    for name in ("a", "a_s", "w", "s", "q", "qs"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(q=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(a=None, M=0) == _lib.BFP8_OK


def test_interleave_w13_layout():
    """The interleaved weight puts w1 and w3 in alternating 64-row groups, scales per group."""
    import torch
    N, K = 256, 256
    w1 = torch.arange(N * K, dtype=torch.int64).reshape(N, K) % 251
    w3 = (torch.arange(N * K, dtype=torch.int64).reshape(N, K) * 7 + 3) % 253
    s1 = torch.arange(4, dtype=torch.float32).reshape(2, 2)
    s3 = 10 + torch.arange(4, dtype=torch.float32).reshape(2, 2)
    w13, s13 = bfp8.interleave_w13(w1, s1, w3, s3)
    for t in range(N // 64):
        assert torch.equal(w13[128 * t:128 * t + 64], w1[64 * t:64 * t + 64])
        assert torch.equal(w13[128 * t + 64:128 * t + 128], w3[64 * t:64 * t + 64])
        assert torch.equal(s13[2 * t], s1[t // 2]) and torch.equal(s13[2 * t + 1], s3[t // 2])


def test_ue8m0_validation(lib):
    f = lib.bfp8_act_quant_ue8m0
    assert f(FAKE, FAKE, FAKE, 4, 100, None) == _lib.BFP8_ERR_SHAPE
    assert f(None, FAKE, FAKE, 4, 128, None) == _lib.BFP8_ERR_NULL
    assert f(ODD, FAKE, FAKE, 4, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(None, None, None, 0, 128, None) == _lib.BFP8_OK
    g = lib.bfp8_gemm_ue8m0
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 200, None, 0, None) == _lib.BFP8_ERR_SHAPE
    assert g(FAKE, None, FAKE, FAKE, FAKE, 64, 64, 256, None, 0, None) == _lib.BFP8_ERR_NULL
    assert g(ODD, FAKE, FAKE, FAKE, FAKE, 64, 64, 256, None, 0, None) == _lib.BFP8_ERR_ALIGN
    assert g(None, FAKE, FAKE, FAKE, FAKE, 0, 64, 256, None, 0, None) == _lib.BFP8_OK
    # a workspace for the split last round: misaligned or too small is refused before any launch
    M, N, K = 8192, 7168, 18432
    need = lib.bfp8_gemm_ue8m0_workspace_size(M, N, K)
    assert need == lib.bfp8_gemm_workspace_size(M, N, K) == 2 * 8192 * 4 * 256 * 4
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, ODD, need, None) == _lib.BFP8_ERR_ALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, FAKE, need - 16, None) == _lib.BFP8_ERR_WORKSPACE
    # nothing to split: no workspace (skinny problems do not split K on this path)
    assert lib.bfp8_gemm_ue8m0_workspace_size(64, 1536, 7168) == 0
    assert lib.bfp8_gemm_ue8m0_workspace_size(8192, 18432, 7168) == 0
    assert lib.bfp8_gemm_ue8m0_workspace_size(0, 7168, 18432) == 0


def test_gemm_k_limit(lib):
    """Every fp8 GEMM entry point rejects K >= 2^22 (32-bit tile row offsets) before any launch."""
    K = 1 << 22
    big = ctypes.c_void_p(0x100000)
    assert lib.bfp8_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, K, None, 0, None) == _lib.BFP8_ERR_SHAPE
    assert lib.bfp8_gemm(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, K - 128, None, 0, None) == _lib.BFP8_OK
    assert lib.bfp8_gemm_act_quant(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 128, K, None) == _lib.BFP8_ERR_SHAPE
    assert lib.bfp8_gemm_swiglu_act_quant(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 256, K, None) == _lib.BFP8_ERR_SHAPE
    assert lib.bfp8_gemm_ue8m0(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, K, None, 0, None) == _lib.BFP8_ERR_SHAPE
    assert lib.bfp8_linear_fp8(FAKE, FAKE, FAKE, FAKE, 1, 1, K, big, 1 << 30, None) == _lib.BFP8_ERR_SHAPE
    off = ctypes.c_void_p(0x200000)
    assert lib.bfp8_gemm_grouped(FAKE, FAKE, FAKE, FAKE, FAKE, off, 1, 1, 1, K, None) == _lib.BFP8_ERR_SHAPE


def test_linear_fp8_validation(lib):
    f = lib.bfp8_linear_fp8
    need = bfp8.bfp8_linear_fp8_workspace_size(64, 1536, 7168)
    assert need > 0 and need % 256 == 0
    assert bfp8.bfp8_linear_fp8_workspace_size(4096, 2048, 7168) >= 4096 * 7168
    WS = ctypes.c_void_p(0x100000)

    def call(x=FAKE, w=FAKE, s=FAKE, y=FAKE, M=64, N=1536, K=7168, ws=WS, wsb=need):
        return f(x, w, s, y, M, N, K, ws, wsb, None)

    assert call(K=100) == _lib.BFP8_ERR_SHAPE
    for name in ("x", "w", "s", "y", "ws"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(ws=ctypes.c_void_p(0x100010)) == _lib.BFP8_ERR_ALIGN
    assert call(wsb=need - 256) == _lib.BFP8_ERR_WORKSPACE
    assert call(x=None, M=0) == _lib.BFP8_OK


def test_gemm_bf16_validation(lib):
    f = lib.bfp8_gemm_bf16

    def call(a=FAKE, b=FAKE, c=FAKE, M=64, N=64, K=128, ws=None, wsb=0):
        return f(a, b, c, M, N, K, ws, wsb, None)

    assert call(K=100) == _lib.BFP8_ERR_SHAPE
    assert call(K=0) == _lib.BFP8_ERR_SHAPE
    assert call(K=1 << 22) == _lib.BFP8_ERR_SHAPE
    assert call(M=-1) == _lib.BFP8_ERR_SHAPE
    for name in ("a", "b", "c"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(a=ctypes.c_void_p(0x10008)) == _lib.BFP8_ERR_ALIGN
    assert call(c=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(a=None, M=0) == _lib.BFP8_OK
    # the split last round's workspace: the fp8 GEMM's plan, misaligned or short refused
    M, N, K = 8192, 7168, 18432
    need = lib.bfp8_gemm_bf16_workspace_size(M, N, K)
    assert need == lib.bfp8_gemm_workspace_size(M, N, K) > 0
    assert lib.bfp8_gemm_bf16_workspace_size(8192, 18432, 7168) == 0
    assert lib.bfp8_gemm_bf16_workspace_size(8192, 7168, 100) == 0
    assert call(M=M, N=N, K=K, ws=ODD, wsb=need) == _lib.BFP8_ERR_ALIGN
    assert call(M=M, N=N, K=K, ws=FAKE, wsb=need - 16) == _lib.BFP8_ERR_WORKSPACE


def test_moe_dispatch_validation(lib):
    f = lib.bfp8_moe_dispatch
    need = bfp8.bfp8_moe_dispatch_workspace_size(100, 8, 32)
    assert need > 0 and need % 16 == 0
    assert bfp8.bfp8_moe_dispatch_workspace_size(0, 8, 32) == 0
    assert bfp8.bfp8_moe_dispatch_workspace_size(100, 8, 2000) == 0

    def call(topk=FAKE, T=100, k=8, lo=0, G=32, off=FAKE, rt=FAKE, sr=FAKE, ws=FAKE, wsb=need):
        return f(topk, T, k, lo, G, off, rt, sr, ws, wsb, None)

    assert call(T=-1) == _lib.BFP8_ERR_SHAPE
    assert call(k=0) == _lib.BFP8_ERR_SHAPE
    assert call(T=1 << 28, k=8) == _lib.BFP8_ERR_SHAPE          # T*k reaches 2^31
    assert call(G=0) == _lib.BFP8_ERR_GROUPS
    assert call(G=1025) == _lib.BFP8_ERR_GROUPS
    for name in ("topk", "off", "rt", "sr", "ws"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(off=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(ws=ctypes.c_void_p(0x10001)) == _lib.BFP8_ERR_ALIGN
    assert call(wsb=need - 16) == _lib.BFP8_ERR_WORKSPACE
    assert call(T=0, off=None) == _lib.BFP8_ERR_NULL             # offsets are written even for T=0


def test_act_quant_rows_validation(lib):
    f = lib.bfp8_act_quant_rows

    def call(x=FAKE, T=10, rt=FAKE, nr=FAKE, q=FAKE, s=FAKE, M=20, K=256):
        return f(x, T, rt, nr, q, s, M, K, None)

    assert call(K=100) == _lib.BFP8_ERR_SHAPE
    assert call(T=-1) == _lib.BFP8_ERR_SHAPE
    assert call(M=-1) == _lib.BFP8_ERR_SHAPE
    for name in ("x", "rt", "q", "s"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(x=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(q=ctypes.c_void_p(0x10008)) == _lib.BFP8_ERR_ALIGN
    assert call(nr=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(M=0, x=None, rt=None) == _lib.BFP8_OK


def test_moe_combine_validation(lib):
    f = lib.bfp8_moe_combine

    def call(o=FAKE, rows=50, sr=FAKE, w=FAKE, y=FAKE, T=10, k=8, N=64):
        return f(o, rows, sr, w, y, T, k, N, None)

    assert call(T=-1) == _lib.BFP8_ERR_SHAPE
    assert call(k=0) == _lib.BFP8_ERR_SHAPE
    assert call(rows=-1) == _lib.BFP8_ERR_SHAPE
    assert call(T=(1 << 24) + 1, k=1) == _lib.BFP8_ERR_SHAPE
    for name in ("o", "sr", "w", "y"):
        assert call(**{name: None}) == _lib.BFP8_ERR_NULL, name
    assert call(o=ODD) == _lib.BFP8_ERR_ALIGN
    assert call(sr=ctypes.c_void_p(0x10002)) == _lib.BFP8_ERR_ALIGN
    assert call(T=0) == _lib.BFP8_OK
    assert call(o=None, rows=0, T=0) == _lib.BFP8_OK


def test_encode_range_validation(lib):
    f = lib.bfp8_e4m3_encode_range
    assert f(0, -1, FAKE, 0, None) == _lib.BFP8_ERR_SHAPE
    assert f(0xFFFFFFFF, 2, FAKE, 0, None) == _lib.BFP8_ERR_SHAPE
    assert f(0, 16, FAKE, 2, None) == _lib.BFP8_ERR_ARG
    assert f(0, 16, None, 0, None) == _lib.BFP8_ERR_NULL
    assert f(0, 0, None, 0, None) == _lib.BFP8_OK


def test_bf16_round_range_validation(lib):
    f = lib.bfp8_bf16_round_range
    assert f(0, -1, FAKE, 0, None) == _lib.BFP8_ERR_SHAPE
    assert f(0xFFFFFFFF, 2, FAKE, 0, None) == _lib.BFP8_ERR_SHAPE
    assert f(0, 16, FAKE, 5, None) == _lib.BFP8_ERR_ARG
    assert f(0, 16, None, 0, None) == _lib.BFP8_ERR_NULL
    assert f(0, 16, ODD, 0, None) == _lib.BFP8_ERR_ALIGN
    assert f(0, 0, None, 0, None) == _lib.BFP8_OK


def test_python_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)            # CPU tensor: refused before any call
    with pytest.raises(ValueError):
        bfp8.bfp8_act_quant(x, torch.zeros(4, 256, dtype=torch.uint8),
                            torch.zeros(4, 2, dtype=torch.float32))
    with pytest.raises(TypeError):
        bfp8.bfp8_gemm(torch.zeros(4, 256, dtype=torch.int16), None, None, None, None)


def test_gemm_noalloc_validation(lib):
    f = lib.bfp8_gemm_noalloc
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 100, None) == _lib.BFP8_ERR_SHAPE    # K % 128
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 64, 128, None) == _lib.BFP8_ERR_SHAPE
    assert f(None, FAKE, FAKE, FAKE, FAKE, 64, 64, 128, None) == _lib.BFP8_ERR_NULL
    assert f(FAKE, FAKE, FAKE, FAKE, None, 64, 64, 128, None) == _lib.BFP8_ERR_NULL
    assert f(ODD, FAKE, FAKE, FAKE, FAKE, 64, 64, 128, None) == _lib.BFP8_ERR_ALIGN
    assert f(None, None, None, None, None, 0, 64, 128, None) == _lib.BFP8_OK
    # a skinny, long-K problem whose split-K partials exceed the fixed scratch array
    M, N, K = 64, 12288, 128 * 1000
    assert lib.bfp8_gemm_workspace_size(M, N, K) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, M, N, K, None) == _lib.BFP8_ERR_SCRATCH
    assert "scratch" in bfp8.bfp8_status_string(_lib.BFP8_ERR_SCRATCH)
    # the configurations it serves fit: the dense MLP's down projection needs exactly the maximum
    assert lib.bfp8_gemm_workspace_size(8192, 7168, 18432) == _lib.NOALLOC_SCRATCH_BYTES
    assert 0 < lib.bfp8_gemm_workspace_size(64, 1536, 7168) < _lib.NOALLOC_SCRATCH_BYTES
