"""ctypes binding of libbfp8.so: the C ABI of include/bfp8.h, one Python function per entry point.

Argument marshalling only: every function takes torch tensors that already
live on the GPU, checks that their dtypes and shapes agree with the C
signature, and passes their device pointers, the sizes and the current HIP
stream to the library.  No arithmetic of the path happens here, and there is
no fallback: if the library is missing the call raises.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libbfp8.so")

BLOCK = 128

# status codes of include/bfp8.h
BFP8_OK = 0
BFP8_ERR_NULL = 1
BFP8_ERR_SHAPE = 2
BFP8_ERR_ALIGN = 3
BFP8_ERR_WORKSPACE = 4
BFP8_ERR_GROUPS = 5
BFP8_ERR_HIP = 6
BFP8_ERR_ARG = 7
BFP8_ERR_SCRATCH = 8

# bytes of the device scratch array behind bfp8_gemm_noalloc (include/bfp8.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("bfp8_act_quant", "bfp8_weight_dequant", "bfp8_gemm", "bfp8_gemm_workspace_size",
           "bfp8_gemm_grouped", "bfp8_e4m3_encode_range", "bfp8_bf16_round_range",
           "bfp8_gemm_kernel_name", "bfp8_moe_dispatch_workspace_size", "bfp8_moe_dispatch",
           "bfp8_act_quant_rows", "bfp8_moe_combine", "bfp8_gemm_bf16", "bfp8_gemm_bf16_workspace_size",
           "bfp8_gemm_act_quant", "bfp8_gemm_swiglu_act_quant", "bfp8_act_quant_ue8m0",
           "bfp8_gemm_ue8m0", "bfp8_gemm_ue8m0_workspace_size", "bfp8_linear_fp8_workspace_size", "bfp8_linear_fp8", "bfp8_gemm_noalloc",
           "bfp8_status_string", "bfp8_version")

_lib = None


class Bfp8Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def library():
    """Load libbfp8.so (built by __graft_entry__.build()); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is not built; run __graft_entry__.build() first "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(LIBRARY)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.bfp8_act_quant.argtypes = [P, P, P, I64, I64, P]
    lib.bfp8_act_quant.restype = ctypes.c_int
    lib.bfp8_weight_dequant.argtypes = [P, P, P, I64, I64, P]
    lib.bfp8_weight_dequant.restype = ctypes.c_int
    lib.bfp8_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.bfp8_gemm.restype = ctypes.c_int
    lib.bfp8_gemm_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, P]
    lib.bfp8_gemm_noalloc.restype = ctypes.c_int
    lib.bfp8_gemm_workspace_size.argtypes = [I64, I64, I64]
    lib.bfp8_gemm_workspace_size.restype = ctypes.c_size_t
    lib.bfp8_gemm_grouped.argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, P]
    lib.bfp8_gemm_grouped.restype = ctypes.c_int
    lib.bfp8_e4m3_encode_range.argtypes = [ctypes.c_uint32, I64, P, ctypes.c_int, P]
    lib.bfp8_e4m3_encode_range.restype = ctypes.c_int
    lib.bfp8_bf16_round_range.argtypes = [ctypes.c_uint32, I64, P, ctypes.c_int, P]
    lib.bfp8_bf16_round_range.restype = ctypes.c_int
    lib.bfp8_gemm_kernel_name.argtypes = [I64, I64, I64]
    lib.bfp8_gemm_kernel_name.restype = ctypes.c_char_p
    lib.bfp8_moe_dispatch_workspace_size.argtypes = [I64, I32, I32]
    lib.bfp8_moe_dispatch_workspace_size.restype = ctypes.c_size_t
    lib.bfp8_moe_dispatch.argtypes = [P, I64, I32, I32, I32, P, P, P, P, ctypes.c_size_t, P]
    lib.bfp8_moe_dispatch.restype = ctypes.c_int
    lib.bfp8_act_quant_rows.argtypes = [P, I64, P, P, P, P, I64, I64, P]
    lib.bfp8_act_quant_rows.restype = ctypes.c_int
    lib.bfp8_moe_combine.argtypes = [P, I64, P, P, P, I64, I32, I64, P]
    lib.bfp8_moe_combine.restype = ctypes.c_int
    lib.bfp8_gemm_act_quant.argtypes = [P, P, P, P, P, P, I64, I64, I64, P]
    lib.bfp8_gemm_act_quant.restype = ctypes.c_int
    lib.bfp8_gemm_swiglu_act_quant.argtypes = [P, P, P, P, P, P, I64, I64, I64, P]
    lib.bfp8_gemm_swiglu_act_quant.restype = ctypes.c_int
    lib.bfp8_act_quant_ue8m0.argtypes = [P, P, P, I64, I64, P]
    lib.bfp8_act_quant_ue8m0.restype = ctypes.c_int
    lib.bfp8_gemm_ue8m0.argtypes = [P, P, P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.bfp8_gemm_ue8m0.restype = ctypes.c_int
    lib.bfp8_gemm_ue8m0_workspace_size.argtypes = [I64, I64, I64]
    lib.bfp8_gemm_ue8m0_workspace_size.restype = ctypes.c_size_t
    lib.bfp8_linear_fp8_workspace_size.argtypes = [I64, I64, I64]
    lib.bfp8_linear_fp8_workspace_size.restype = ctypes.c_size_t
    lib.bfp8_linear_fp8.argtypes = [P, P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.bfp8_linear_fp8.restype = ctypes.c_int
    lib.bfp8_gemm_bf16.argtypes = [P, P, P, I64, I64, I64, P, ctypes.c_size_t, P]
    lib.bfp8_gemm_bf16.restype = ctypes.c_int
    lib.bfp8_gemm_bf16_workspace_size.argtypes = [I64, I64, I64]
    lib.bfp8_gemm_bf16_workspace_size.restype = ctypes.c_size_t
    lib.bfp8_status_string.argtypes = [ctypes.c_int]
    lib.bfp8_status_string.restype = ctypes.c_char_p
    lib.bfp8_version.argtypes = []
    lib.bfp8_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return library().bfp8_status_string(int(status)).decode()


def _check(fn, status):
    if status != BFP8_OK:
        raise Bfp8Error(fn, status)


def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _bytes_view(t):
    """e4m3 tensors may arrive as torch.float8_e4m3fn or as raw uint8 codes."""
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(f"expected e4m3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    return t


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _cuda_contig(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda, "all tensors must be on the GPU")
            _need(t.is_contiguous(), "all tensors must be contiguous")


# ------------------------------------------------------------------ entry points

def bfp8_version() -> int:
    return int(library().bfp8_version())


def bfp8_status_string(status: int) -> str:
    return status_string(status)


def bfp8_gemm_kernel_name(M, N, K) -> str:
    """Name of the tile configuration bfp8_gemm uses for this shape on the current device."""
    return library().bfp8_gemm_kernel_name(int(M), int(N), int(K)).decode()


def bfp8_act_quant(x, q, scales, stream=None):
    """x bf16 [M,K] -> q e4m3 [M,K], scales fp32 [M,K/128] (written in place)."""
    q = _bytes_view(q)
    _cuda_contig(x, q, scales)
    _need(x.dtype == torch.bfloat16 and scales.dtype == torch.float32, "x must be bf16, scales fp32")
    _need(x.dim() == 2, "x must be [M, K]")
    M, K = x.shape
    _need(q.shape == (M, K) and scales.shape == (M, K // BLOCK), "output shapes do not match x")
    _check("bfp8_act_quant", library().bfp8_act_quant(_ptr(x), _ptr(q), _ptr(scales), M, K,
                                                      _stream(stream, x.device)))


def bfp8_act_quant_ue8m0(x, q, scales, stream=None):
    """act_quant with power-of-two scales (the e8m0 reading of scale_fmt)."""
    q = _bytes_view(q)
    _cuda_contig(x, q, scales)
    _need(x.dtype == torch.bfloat16 and scales.dtype == torch.float32, "x must be bf16, scales fp32")
    M, K = x.shape
    _need(q.shape == (M, K) and scales.shape == (M, K // BLOCK), "output shapes do not match x")
    _check("bfp8_act_quant_ue8m0", library().bfp8_act_quant_ue8m0(_ptr(x), _ptr(q), _ptr(scales), M, K,
                                                                  _stream(stream, x.device)))


def bfp8_gemm_ue8m0(a, a_s, b, b_s, c, workspace=None, stream=None):
    """bfp8_gemm for power-of-two scales, applied by the MFMA itself."""
    a, b = _bytes_view(a), _bytes_view(b)
    _cuda_contig(a, a_s, b, b_s, c, workspace)
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b must share K")
    _need(a_s.shape == (M, K // BLOCK) and b_s.shape == (-(-N // BLOCK), K // BLOCK),
          "a_s [M, K/128], b_s [ceil(N/128), K/128]")
    _need(c.dtype == torch.bfloat16 and c.shape == (M, N), "c must be bf16 [M, N]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bfp8_gemm_ue8m0", library().bfp8_gemm_ue8m0(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(c),
                                                        M, N, K, _ptr(workspace), ws_bytes,
                                                        _stream(stream, a.device)))


def bfp8_gemm_ue8m0_workspace_size(M, N, K) -> int:
    return int(library().bfp8_gemm_ue8m0_workspace_size(int(M), int(N), int(K)))


def bfp8_weight_dequant(w, s, out, stream=None):
    """w e4m3 [N,K], s fp32 [ceil(N/128), ceil(K/128)] -> out bf16 [N,K]."""
    w = _bytes_view(w)
    _cuda_contig(w, s, out)
    _need(out.dtype == torch.bfloat16 and s.dtype == torch.float32, "out must be bf16, s fp32")
    N, K = w.shape
    _need(out.shape == (N, K), "out must match w")
    _need(s.shape == (-(-N // BLOCK), -(-K // BLOCK)), "scale grid must tile w by 128x128")
    _check("bfp8_weight_dequant", library().bfp8_weight_dequant(_ptr(w), _ptr(s), _ptr(out), N, K,
                                                                _stream(stream, w.device)))


def bfp8_gemm_workspace_size(M, N, K) -> int:
    return int(library().bfp8_gemm_workspace_size(int(M), int(N), int(K)))


def bfp8_gemm(a, a_s, b, b_s, c, workspace=None, stream=None):
    """c bf16 [M,N] = block-scaled a e4m3 [M,K] x b e4m3 [N,K]^T."""
    a, b = _bytes_view(a), _bytes_view(b)
    _cuda_contig(a, a_s, b, b_s, c, workspace)
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b must share K")
    _need(a_s.dtype == torch.float32 and b_s.dtype == torch.float32, "scales must be fp32")
    _need(a_s.shape == (M, K // BLOCK), "a_s must be [M, K/128]")
    _need(b_s.shape == (-(-N // BLOCK), K // BLOCK), "b_s must be [ceil(N/128), K/128]")
    _need(c.dtype == torch.bfloat16 and c.shape == (M, N), "c must be bf16 [M, N]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bfp8_gemm", library().bfp8_gemm(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(c),
                                            M, N, K, _ptr(workspace), ws_bytes,
                                            _stream(stream, a.device)))


def bfp8_gemm_noalloc(a, a_s, b, b_s, c, stream=None):
    """bfp8_gemm with its workspace in the library's fixed per-GPU scratch array (no allocation)."""
    a, b = _bytes_view(a), _bytes_view(b)
    _cuda_contig(a, a_s, b, b_s, c)
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b must share K")
    _need(a_s.dtype == torch.float32 and b_s.dtype == torch.float32, "scales must be fp32")
    _need(a_s.shape == (M, K // BLOCK), "a_s must be [M, K/128]")
    _need(b_s.shape == (-(-N // BLOCK), K // BLOCK), "b_s must be [ceil(N/128), K/128]")
    _need(c.dtype == torch.bfloat16 and c.shape == (M, N), "c must be bf16 [M, N]")
    _check("bfp8_gemm_noalloc", library().bfp8_gemm_noalloc(_ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s),
                                                            _ptr(c), M, N, K,
                                                            _stream(stream, a.device)))


def bfp8_gemm_act_quant(a, a_s, b, b_s, q, q_scales, stream=None):
    """q e4m3 [M,N], q_scales [M,N/128] = act_quant(bf16(a x b^T)) in one kernel (N % 128 == 0)."""
    a, b, q = _bytes_view(a), _bytes_view(b), _bytes_view(q)
    _cuda_contig(a, a_s, b, b_s, q, q_scales)
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K, "a and b must share K")
    _need(a_s.dtype == torch.float32 and b_s.dtype == torch.float32 and q_scales.dtype == torch.float32,
          "scales must be fp32")
    _need(a_s.shape == (M, K // BLOCK) and b_s.shape == (-(-N // BLOCK), K // BLOCK),
          "a_s [M, K/128], b_s [ceil(N/128), K/128]")
    _need(q.shape == (M, N) and q_scales.shape == (M, N // BLOCK), "q [M, N], q_scales [M, N/128]")
    _check("bfp8_gemm_act_quant", library().bfp8_gemm_act_quant(
        _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(q), _ptr(q_scales), M, N, K,
        _stream(stream, a.device)))


def bfp8_gemm_swiglu_act_quant(a, a_s, w13, s13, q, q_scales, stream=None):
    """q, q_scales = act_quant(bf16(bf16(silu(bf16(a w1^T))) * bf16(a w3^T))) for the 64-row
    interleaved w13 [2N, K] (see interleave_w13) with its per-64-row scales s13 [2N/64, K/128]."""
    a, w13, q = _bytes_view(a), _bytes_view(w13), _bytes_view(q)
    _cuda_contig(a, a_s, w13, s13, q, q_scales)
    M, K = a.shape
    N2 = w13.shape[0]
    _need(w13.shape[1] == K and N2 % 256 == 0, "w13 must be [2N, K] with N % 128 == 0")
    N = N2 // 2
    _need(a_s.shape == (M, K // BLOCK) and s13.shape == (N2 // 64, K // BLOCK),
          "a_s [M, K/128], s13 [2N/64, K/128]")
    _need(q.shape == (M, N) and q_scales.shape == (M, N // BLOCK), "q [M, N], q_scales [M, N/128]")
    _check("bfp8_gemm_swiglu_act_quant", library().bfp8_gemm_swiglu_act_quant(
        _ptr(a), _ptr(a_s), _ptr(w13), _ptr(s13), _ptr(q), _ptr(q_scales), M, N, K,
        _stream(stream, a.device)))


def interleave_w13(w1, s1, w3, s3):
    """One-time weight preparation (data movement only) for bfp8_gemm_swiglu_act_quant:
    w1, w3 e4m3 [N, K] with 128x128 scale grids s1, s3 [N/128, K/128] ->
    w13 [2N, K] (64-row groups alternating w1, w3) and s13 [2N/64, K/128]."""
    N, K = w1.shape
    _need(w3.shape == (N, K) and N % 128 == 0, "w1 and w3 must be [N, K] with N % 128 == 0")
    w13 = torch.stack([w1.reshape(N // 64, 64, K), w3.reshape(N // 64, 64, K)], dim=1).reshape(2 * N, K)
    g1 = s1.repeat_interleave(2, dim=0)                  # scale of each 64-row group of w1
    g3 = s3.repeat_interleave(2, dim=0)
    s13 = torch.stack([g1, g3], dim=1).reshape(2 * N // 64, -1)
    return w13.contiguous(), s13.contiguous()


def bfp8_linear_fp8_workspace_size(M, N, K) -> int:
    return int(library().bfp8_linear_fp8_workspace_size(int(M), int(N), int(K)))


def bfp8_linear_fp8(x, w, w_s, y, workspace, stream=None):
    """y bf16 [M,N] = fp8_gemm(act_quant(x bf16 [M,K]), w, w_s) in one call (see include/bfp8.h).

    workspace: a device tensor of at least bfp8_linear_fp8_workspace_size(M, N, K) bytes
    (linear_workspace() allocates one)."""
    w = _bytes_view(w)
    _cuda_contig(x, w, w_s, y, workspace)
    _need(x.dtype == torch.bfloat16 and y.dtype == torch.bfloat16, "x and y must be bf16")
    M, K = x.shape
    N = w.shape[0]
    _need(w.shape[1] == K and w_s.shape == (-(-N // BLOCK), K // BLOCK) and y.shape == (M, N),
          "w [N, K], w_s [ceil(N/128), K/128], y [M, N]")
    nbytes = workspace.numel() * workspace.element_size()
    _check("bfp8_linear_fp8", library().bfp8_linear_fp8(_ptr(x), _ptr(w), _ptr(w_s), _ptr(y), M, N, K,
                                                        _ptr(workspace), nbytes,
                                                        _stream(stream, x.device)))


def linear_workspace(M, N, K, device):
    """A workspace for bfp8_linear_fp8 at this shape."""
    n = max(256, bfp8_linear_fp8_workspace_size(M, N, K))
    return torch.empty((n + 255) // 256 * 256, dtype=torch.uint8, device=device)


def bfp8_gemm_grouped(a, a_s, b, b_s, c, group_offsets, stream=None):
    """Rows [off[g], off[g+1]) of a times b[g]^T into the same rows of c."""
    a, b = _bytes_view(a), _bytes_view(b)
    _cuda_contig(a, a_s, b, b_s, c, group_offsets)
    T, K = a.shape
    G, N, Kb = b.shape
    _need(Kb == K, "a and b must share K")
    _need(group_offsets.dtype == torch.int32 and group_offsets.shape == (G + 1,),
          "group_offsets must be int32 [G+1] on the GPU")
    _need(a_s.shape == (T, K // BLOCK), "a_s must be [total_M, K/128]")
    _need(b_s.shape == (G, -(-N // BLOCK), K // BLOCK), "b_s must be [G, ceil(N/128), K/128]")
    _need(c.dtype == torch.bfloat16 and c.shape == (T, N), "c must be bf16 [total_M, N]")
    _check("bfp8_gemm_grouped", library().bfp8_gemm_grouped(
        _ptr(a), _ptr(a_s), _ptr(b), _ptr(b_s), _ptr(c), _ptr(group_offsets), G, T, N, K,
        _stream(stream, a.device)))


def bfp8_gemm_bf16(a, b, c, workspace=None, stream=None):
    """c bf16 [M,N] = a bf16 [M,K] x b bf16 [N,K]^T (the BF16 branch's matmul)."""
    _cuda_contig(a, b, c, workspace)
    _need(a.dtype == torch.bfloat16 and b.dtype == torch.bfloat16 and c.dtype == torch.bfloat16,
          "a, b and c must be bf16")
    M, K = a.shape
    N = b.shape[0]
    _need(b.shape[1] == K and c.shape == (M, N), "shapes must be a [M,K], b [N,K], c [M,N]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bfp8_gemm_bf16", library().bfp8_gemm_bf16(_ptr(a), _ptr(b), _ptr(c), M, N, K,
                                                      _ptr(workspace), ws_bytes,
                                                      _stream(stream, a.device)))


def bfp8_gemm_bf16_workspace_size(M, N, K) -> int:
    return int(library().bfp8_gemm_bf16_workspace_size(int(M), int(N), int(K)))


def bfp8_e4m3_encode_range(first, count, out, variant=0, stream=None):
    """Device encode of the fp32 bit patterns first .. first+count-1 into out (uint8)."""
    _cuda_contig(out)
    _need(out.dtype == torch.uint8 and out.numel() >= count, "out must be uint8 with count bytes")
    _check("bfp8_e4m3_encode_range", library().bfp8_e4m3_encode_range(
        int(first), int(count), _ptr(out), int(variant), _stream(stream, out.device)))


def bfp8_bf16_round_range(first, count, out, variant=0, stream=None):
    """Device bf16 rounding of the fp32 bit patterns first .. first+count-1 into out (int16/uint16)."""
    _cuda_contig(out)
    _need(out.element_size() == 2 and out.numel() >= count, "out must be 2-byte elements, count long")
    _check("bfp8_bf16_round_range", library().bfp8_bf16_round_range(
        int(first), int(count), _ptr(out), int(variant), _stream(stream, out.device)))


def bfp8_moe_dispatch_workspace_size(T, k, G) -> int:
    return int(library().bfp8_moe_dispatch_workspace_size(int(T), int(k), int(G)))


def bfp8_moe_dispatch(topk_idx, expert_lo, group_offsets, row_token, slot_row, workspace,
                      stream=None):
    """Stable sort of the (token, slot) pairs of topk_idx int32 [T, k] by local expert.

    Local experts are expert_lo .. expert_lo + G - 1 with G = group_offsets.numel() - 1.
    Writes group_offsets int32 [G+1], row_token int32 [T*k], slot_row int32 [T, k].
    """
    _cuda_contig(topk_idx, group_offsets, row_token, slot_row, workspace)
    for t in (topk_idx, group_offsets, row_token, slot_row):
        _need(t.dtype == torch.int32, "index tensors must be int32")
    _need(topk_idx.dim() == 2, "topk_idx must be [T, k]")
    T, k = topk_idx.shape
    G = group_offsets.numel() - 1
    _need(row_token.numel() >= T * k and slot_row.shape == (T, k), "row_token [T*k], slot_row [T, k]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("bfp8_moe_dispatch", library().bfp8_moe_dispatch(
        _ptr(topk_idx), T, k, int(expert_lo), G, _ptr(group_offsets), _ptr(row_token),
        _ptr(slot_row), _ptr(workspace), ws_bytes, _stream(stream, group_offsets.device)))


def bfp8_act_quant_rows(x, row_token, num_rows, q, scales, stream=None):
    """q[r], scales[r] = act_quant(x[row_token[r]]) for r < min(num_rows[0], M)."""
    q = _bytes_view(q)
    _cuda_contig(x, row_token, num_rows, q, scales)
    _need(x.dtype == torch.bfloat16 and scales.dtype == torch.float32, "x must be bf16, scales fp32")
    _need(row_token.dtype == torch.int32 and (num_rows is None or num_rows.dtype == torch.int32),
          "row_token and num_rows must be int32")
    T, K = x.shape
    M = q.shape[0]
    _need(q.shape == (M, K) and scales.shape == (M, K // BLOCK) and row_token.numel() >= M,
          "q [M, K], scales [M, K/128], row_token [M]")
    _check("bfp8_act_quant_rows", library().bfp8_act_quant_rows(
        _ptr(x), T, _ptr(row_token), _ptr(num_rows), _ptr(q), _ptr(scales), M, K,
        _stream(stream, x.device)))


def bfp8_moe_combine(expert_out, slot_row, weights, y, stream=None):
    """y bf16 [T, N] = sum over local slots of weights[t, j] * expert_out[slot_row[t, j]]."""
    _cuda_contig(expert_out, slot_row, weights, y)
    _need(expert_out.dtype == torch.bfloat16 and y.dtype == torch.bfloat16, "bf16 expert_out and y")
    _need(slot_row.dtype == torch.int32 and weights.dtype == torch.float32,
          "slot_row int32, weights fp32")
    rows, N = expert_out.shape
    T, k = slot_row.shape
    _need(weights.shape == (T, k) and y.shape == (T, N), "weights [T, k], y [T, N]")
    _check("bfp8_moe_combine", library().bfp8_moe_combine(
        _ptr(expert_out), rows, _ptr(slot_row), _ptr(weights), _ptr(y), T, k, N,
        _stream(stream, y.device)))


# ------------------------------------------------------- allocating conveniences

def act_quant(x, stream=None):
    """(q e4m3 as uint8 [M,K], scales fp32 [M,K/128]) = act_quant(x bf16 [M,K])."""
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // BLOCK), dtype=torch.float32, device=x.device)
    bfp8_act_quant(x, q, s, stream)
    return q, s


def weight_dequant(w, s, stream=None):
    out = torch.empty(w.shape, dtype=torch.bfloat16, device=w.device)
    bfp8_weight_dequant(w, s, out, stream)
    return out


def gemm(a, a_s, b, b_s, workspace=None, stream=None):
    c = torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device=a.device)
    bfp8_gemm(a, a_s, b, b_s, c, workspace, stream)
    return c


def gemm_grouped(a, a_s, b, b_s, group_offsets, stream=None):
    c = torch.empty((a.shape[0], b.shape[1]), dtype=torch.bfloat16, device=a.device)
    bfp8_gemm_grouped(a, a_s, b, b_s, c, group_offsets, stream)
    return c


def gemm_bf16(a, b, workspace=None, stream=None):
    c = torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device=a.device)
    bfp8_gemm_bf16(a, b, c, workspace, stream)
    return c


def linear_bf16(x, w, w_s, workspace=None, stream=None):
    """The BF16 branch of linear(): weight_dequant(w, w.scale) then the bf16 matmul."""
    return gemm_bf16(x, weight_dequant(w, w_s, stream), workspace, stream)


def gemm_act_quant(a, a_s, b, b_s, stream=None):
    M, N = a.shape[0], b.shape[0]
    q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    qs = torch.empty((M, N // BLOCK), dtype=torch.float32, device=a.device)
    bfp8_gemm_act_quant(a, a_s, b, b_s, q, qs, stream)
    return q, qs


def gemm_swiglu_act_quant(a, a_s, w13, s13, stream=None):
    M, N = a.shape[0], w13.shape[0] // 2
    q = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    qs = torch.empty((M, N // BLOCK), dtype=torch.float32, device=a.device)
    bfp8_gemm_swiglu_act_quant(a, a_s, w13, s13, q, qs, stream)
    return q, qs


def act_quant_ue8m0(x, stream=None):
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // BLOCK), dtype=torch.float32, device=x.device)
    bfp8_act_quant_ue8m0(x, q, s, stream)
    return q, s


def gemm_ue8m0(a, a_s, b, b_s, workspace=None, stream=None):
    c = torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device=a.device)
    bfp8_gemm_ue8m0(a, a_s, b, b_s, c, workspace, stream)
    return c


def linear_fp8(x, w, w_s, workspace=None, stream=None):
    """The FP8 branch of linear(): act_quant(x) then the block-scaled GEMM with (w, w.scale)."""
    q, s = act_quant(x, stream)
    return gemm(q, s, w, w_s, workspace, stream)


def moe_dispatch(topk_idx, expert_lo, G, stream=None):
    """(group_offsets [G+1], row_token [T*k], slot_row [T, k]) for local experts expert_lo..+G-1."""
    T, k = topk_idx.shape
    dev = topk_idx.device
    off = torch.empty(G + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(1, T * k), dtype=torch.int32, device=dev)
    slot_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, bfp8_moe_dispatch_workspace_size(T, k, G) // 4), dtype=torch.int32,
                     device=dev)
    bfp8_moe_dispatch(topk_idx, expert_lo, off, row_token, slot_row, ws, stream)
    return off, row_token, slot_row


def moe_combine(expert_out, slot_row, weights, stream=None):
    y = torch.empty((slot_row.shape[0], expert_out.shape[1]), dtype=torch.bfloat16,
                    device=expert_out.device)
    bfp8_moe_combine(expert_out, slot_row, weights, y, stream)
    return y


def moe_experts_fp8(x, topk_idx, weights, w, w_s, expert_lo, stream=None):
    """Routed experts of one GPU, one block-scaled GEMM each, fully on the device.

    dispatch -> act_quant of the gathered rows -> grouped GEMM -> weighted combine.
    x bf16 [T, K]; topk_idx int32 [T, k]; weights fp32 [T, k]; w e4m3 [G, N, K] with
    scales w_s [G, ceil(N/128), K/128].  Returns y bf16 [T, N].  Row buffers are sized
    for the worst case T*k rows; only the first group_offsets[G] are touched.
    """
    T, K = x.shape
    k = topk_idx.shape[1]
    G, N, _ = w.shape
    off, row_token, slot_row = moe_dispatch(topk_idx, expert_lo, G, stream)
    cap = T * k
    q = torch.empty((cap, K), dtype=torch.uint8, device=x.device)
    qs = torch.empty((cap, K // BLOCK), dtype=torch.float32, device=x.device)
    bfp8_act_quant_rows(x, row_token[:cap], off[G:], q, qs, stream)
    out = torch.empty((cap, N), dtype=torch.bfloat16, device=x.device)
    bfp8_gemm_grouped(q, qs, w, w_s, out, off, stream)
    return moe_combine(out, slot_row, weights, stream)
