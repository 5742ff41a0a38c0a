"""CPU oracle for the block-scaled FP8 linear path (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path never imports this
package, and this package never imports the product package.

Every function is a thin ctypes call into ``bfp8_oracle.cpp`` (plain loops, no
blocking or reordering).  Conventions:

* bf16 tensors travel as ``numpy.uint16`` arrays of bit patterns;
* e4m3 tensors travel as ``numpy.uint8`` arrays of codes;
* scales are ``numpy.float32``;
* GEMM references are ``numpy.float64``.

Sources (what is computed): "Data flow - deepseek-ai/DeepSeek-V3"
(codevetter), FP8 quantization bullet; pyshine "DeepSeek-V3" tour, "The Three
Ideas That Make V3 Fast", paragraph "FP8 with per-block scales";
"Behavior traces" (codevetter), fp8->bf16 trace bullet.

Parity unpinned: the value of the block-max floor (``amax_floor()``), which the
pages do not give.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BLOCK = 128
E4M3_MAX = 448.0


class Oracle:
    """ctypes front end over one build of ``bfp8_oracle.cpp``.

    The module-level functions use the library built in this folder; the
    tests also load deliberately broken builds through this class to show
    that the pins catch plausible mistakes.
    """

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_e4m3_encode_array.argtypes = [P, P, I64]
        lib.oracle_e4m3_decode_array.argtypes = [P, P, I64]
        lib.oracle_f32_to_bf16_array.argtypes = [P, P, I64]
        lib.oracle_amax_floor.restype = ctypes.c_float
        lib.oracle_act_quant.argtypes = [P, P, P, I64, I64]
        lib.oracle_act_quant.restype = ctypes.c_int
        lib.oracle_weight_dequant.argtypes = [P, P, P, I64, I64]
        lib.oracle_gemm_rows.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, ctypes.c_int]
        lib.oracle_gemm_rows.restype = ctypes.c_int
        lib.oracle_gemm_grouped_rows.argtypes = [P, P, P, P, P, ctypes.c_int32, I64, I64, I64,
                                                 P, I64, P, ctypes.c_int]
        lib.oracle_gemm_grouped_rows.restype = ctypes.c_int
        lib.oracle_gemm_bf16_rows.argtypes = [P, P, I64, I64, I64, P, I64, P, ctypes.c_int]
        lib.oracle_gemm_bf16_rows.restype = ctypes.c_int
        lib.oracle_swiglu_bf16.argtypes = [P, P, I64, P]
        lib.oracle_act_quant_pow2.argtypes = [P, P, P, I64, I64]
        lib.oracle_act_quant_pow2.restype = ctypes.c_int
        lib.oracle_moe_dispatch.argtypes = [P, I64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            P, P, P]
        lib.oracle_moe_combine.argtypes = [P, P, P, I64, ctypes.c_int32, I64, P]
        self.lib = lib
        self.path = path

    def amax_floor(self) -> float:
        """Lower clamp on a block's max |x| (a reading; the pages give no value)."""
        return float(self.lib.oracle_amax_floor())

    # ------------------------------------------------------------- formats

    def e4m3_decode(self, codes) -> np.ndarray:
        """e4m3 codes -> float32 values (exact)."""
        c = _c(codes, np.uint8)
        out = np.empty(c.shape, np.float32)
        self.lib.oracle_e4m3_decode_array(_ptr(c), _ptr(out), c.size)
        return out

    def e4m3_encode(self, values) -> np.ndarray:
        """float32 values -> e4m3 codes, nearest-even, saturating at +-448."""
        v = _c(values, np.float32)
        out = np.empty(v.shape, np.uint8)
        self.lib.oracle_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
        return out

    def f32_to_bf16(self, values) -> np.ndarray:
        """float32 -> bf16 bit patterns, nearest-even."""
        v = _c(values, np.float32)
        out = np.empty(v.shape, np.uint16)
        self.lib.oracle_f32_to_bf16_array(_ptr(v), _ptr(out), v.size)
        return out

    @staticmethod
    def bf16_to_f32(bits) -> np.ndarray:
        """bf16 bit patterns -> float32 (exact)."""
        b = _c(bits, np.uint16)
        return (b.astype(np.uint32) << 16).view(np.float32)

    # ----------------------------------------------------------- act_quant

    def act_quant(self, x_bits):
        """bf16 [M,K] -> (e4m3 codes [M,K], fp32 scales [M, K/128])."""
        x = _c(x_bits, np.uint16)
        if x.ndim != 2:
            raise ValueError("act_quant expects a 2-D [M, K] array")
        M, K = x.shape
        if K <= 0 or K % BLOCK:
            raise ValueError("K must be a positive multiple of 128")
        q = np.empty((M, K), np.uint8)
        s = np.empty((M, K // BLOCK), np.float32)
        rc = self.lib.oracle_act_quant(_ptr(x), _ptr(q), _ptr(s), M, K)
        if rc:
            raise ValueError(f"oracle_act_quant failed ({rc})")
        return q, s

    # ------------------------------------------------------ weight_dequant

    def weight_dequant(self, w, S):
        """e4m3 [N,K] with fp32 scales [ceil(N/128), ceil(K/128)] -> bf16 bits [N,K]."""
        w = _c(w, np.uint8)
        S = _c(S, np.float32)
        N, K = w.shape
        if S.shape != (-(-N // BLOCK), -(-K // BLOCK)):
            raise ValueError(f"scale grid shape {S.shape} does not tile [{N},{K}] by 128x128")
        out = np.empty((N, K), np.uint16)
        self.lib.oracle_weight_dequant(_ptr(w), _ptr(S), _ptr(out), N, K)
        return out

    # ---------------------------------------------------------------- GEMM

    def gemm(self, a, sa, b, sb, rows=None, threads=None) -> np.ndarray:
        """fp64 reference of C = A * B^T with per-block scales, for the given rows.

        a: e4m3 [M,K]; sa: fp32 [M,K/128]; b: e4m3 [N,K]; sb: fp32 [ceil(N/128), K/128].
        Returns float64 [len(rows), N].
        """
        a = _c(a, np.uint8); sa = _c(sa, np.float32)
        b = _c(b, np.uint8); sb = _c(sb, np.float32)
        M, K = a.shape
        N = b.shape[0]
        if b.shape[1] != K or sa.shape != (M, K // BLOCK) or \
                sb.shape != (-(-N // BLOCK), K // BLOCK):
            raise ValueError("gemm operand shapes do not agree")
        r = _rows(rows, M)
        out = np.empty((r.size, N), np.float64)
        rc = self.lib.oracle_gemm_rows(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), M, N, K,
                                       _ptr(r), r.size, _ptr(out),
                                       threads or default_threads())
        if rc:
            raise ValueError(f"oracle_gemm_rows failed ({rc})")
        return out

    def gemm_grouped(self, a, sa, b, sb, offsets, rows=None, threads=None) -> np.ndarray:
        """fp64 reference of the grouped GEMM for the given rows (NaN for rows in no group).

        a: e4m3 [T,K] sorted by group; sa: [T,K/128]; b: e4m3 [G,N,K];
        sb: [G, ceil(N/128), K/128]; offsets: int32 [G+1].
        """
        a = _c(a, np.uint8); sa = _c(sa, np.float32)
        b = _c(b, np.uint8); sb = _c(sb, np.float32)
        off = _c(offsets, np.int32)
        T, K = a.shape
        G, N, _ = b.shape
        if off.shape != (G + 1,) or sb.shape != (G, -(-N // BLOCK), K // BLOCK):
            raise ValueError("grouped operand shapes do not agree")
        r = _rows(rows, T)
        out = np.empty((r.size, N), np.float64)
        rc = self.lib.oracle_gemm_grouped_rows(_ptr(a), _ptr(sa), _ptr(b), _ptr(sb), _ptr(off),
                                               G, T, N, K, _ptr(r), r.size, _ptr(out),
                                               threads or default_threads())
        if rc:
            raise ValueError(f"oracle_gemm_grouped_rows failed ({rc})")
        return out


    def gemm_bf16(self, a_bits, b_bits, rows=None, threads=None) -> np.ndarray:
        """fp64 reference of C = A * B^T for bf16 A [M,K] and B [N,K] (bit patterns), given rows."""
        a = _c(a_bits, np.uint16); b = _c(b_bits, np.uint16)
        M, K = a.shape
        N = b.shape[0]
        if b.shape[1] != K:
            raise ValueError("gemm_bf16 operand shapes do not agree")
        r = _rows(rows, M)
        out = np.empty((r.size, N), np.float64)
        rc = self.lib.oracle_gemm_bf16_rows(_ptr(a), _ptr(b), M, N, K, _ptr(r), r.size, _ptr(out),
                                            threads or default_threads())
        if rc:
            raise ValueError(f"oracle_gemm_bf16_rows failed ({rc})")
        return out

    def act_quant_pow2(self, x_bits):
        """act_quant with scales rounded up to powers of two (the e8m0 reading of scale_fmt)."""
        x = _c(x_bits, np.uint16)
        M, K = x.shape
        q = np.empty((M, K), np.uint8)
        s = np.empty((M, K // BLOCK), np.float32)
        if self.lib.oracle_act_quant_pow2(_ptr(x), _ptr(q), _ptr(s), M, K):
            raise ValueError("K must be a positive multiple of 128")
        return q, s

    def swiglu_bf16(self, g, u) -> np.ndarray:
        """bf16 bits of bf16(bf16(silu(bf16(g))) * bf16(u)) for fp64 arrays g, u of one shape."""
        g = _c(g, np.float64); u = _c(u, np.float64)
        if g.shape != u.shape:
            raise ValueError("g and u must have one shape")
        h = np.empty(g.shape, np.uint16)
        self.lib.oracle_swiglu_bf16(_ptr(g), _ptr(u), g.size, _ptr(h))
        return h

    # ---------------------------------------------------------------- MoE

    def moe_dispatch(self, topk, expert_lo, G):
        """Stable dispatch of routed tokens to local experts expert_lo .. expert_lo+G-1.

        topk: int32 [T, k].  Returns (offsets int32 [G+1], row_token int32 [rows],
        slot_row int32 [T, k] with -1 for non-local slots).
        """
        tk = _c(topk, np.int32)
        T, k = tk.shape
        offsets = np.empty(G + 1, np.int32)
        row_token = np.empty(max(1, T * k), np.int32)
        slot_row = np.empty((T, k), np.int32)
        self.lib.oracle_moe_dispatch(_ptr(tk), T, k, int(expert_lo), int(G), _ptr(offsets),
                                     _ptr(row_token), _ptr(slot_row))
        return offsets, row_token[:int(offsets[-1])].copy(), slot_row

    def moe_combine(self, out_bits, slot_row, weights):
        """fp64 y [T, N] = sum over local slots of weight * out[row] (out: bf16 bits [rows, N])."""
        o = _c(out_bits, np.uint16)
        sr = _c(slot_row, np.int32)
        w = _c(weights, np.float32)
        T, k = sr.shape
        N = o.shape[1]
        y = np.empty((T, N), np.float64)
        self.lib.oracle_moe_combine(_ptr(o), _ptr(sr), _ptr(w), T, k, N, _ptr(y))
        return y


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _rows(rows, M):
    if rows is None:
        return np.arange(M, dtype=np.int64)
    return _c(rows, np.int64)


def default_threads() -> int:
    if hasattr(os, "sched_getaffinity"):
        return len(os.sched_getaffinity(0))
    return os.cpu_count() or 1


_default = None


def default() -> Oracle:
    """The oracle built from this folder's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        _default = Oracle(_build.LIBRARY)
    return _default


def amax_floor():
    return default().amax_floor()


def e4m3_decode(codes):
    return default().e4m3_decode(codes)


def e4m3_encode(values):
    return default().e4m3_encode(values)


def f32_to_bf16(values):
    return default().f32_to_bf16(values)


def bf16_to_f32(bits):
    return Oracle.bf16_to_f32(bits)


def act_quant(x_bits):
    return default().act_quant(x_bits)


def weight_dequant(w, S):
    return default().weight_dequant(w, S)


def gemm(a, sa, b, sb, rows=None, threads=None):
    return default().gemm(a, sa, b, sb, rows, threads)


def gemm_grouped(a, sa, b, sb, offsets, rows=None, threads=None):
    return default().gemm_grouped(a, sa, b, sb, offsets, rows, threads)


def gemm_bf16(a_bits, b_bits, rows=None, threads=None):
    return default().gemm_bf16(a_bits, b_bits, rows, threads)


def act_quant_pow2(x_bits):
    return default().act_quant_pow2(x_bits)


def swiglu_bf16(g, u):
    return default().swiglu_bf16(g, u)


def moe_dispatch(topk, expert_lo, G):
    return default().moe_dispatch(topk, expert_lo, G)


def moe_combine(out_bits, slot_row, weights):
    return default().moe_combine(out_bits, slot_row, weights)
