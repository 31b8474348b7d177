"""Python binding of libgemm, the gfx950 dense GEMM library.

The binding only marshals arguments: every step of the product runs in the
HIP kernels of ``libgemm.so``.  PyTorch provides device memory and the current
stream.  If the library is missing the calls raise; there is no fallback.

Raw entry points mirror the C ABI of include/libgemm.h and
include/attention.h one to one (``gemm_bf16``, ``gemm_bf16_nt``,
``gemm_mxfp8``, ..., ``attn_fwd_bf16``, ``attn_fwd_bf16_out``, ``gemm_strerror``, ``gemm_version``)
and take integers for pointers and the stream.  The tensor helpers ``bf16``,
``mxfp8`` and ``attention`` build those arguments from torch tensors.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libgemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = -1
GEMM_ERR_UNSUPPORTED = -2
GEMM_ERR_LAUNCH = -3
GEMM_ERR_SCRATCH = -4
GEMM_SCRATCH_BYTES = 64 << 20
GEMM_OUT_F32 = 0
GEMM_OUT_BF16 = 1
GEMM_OUT_E4M3 = 2
GEMM_DYNAMIC_WORKSPACE_BYTES = 1024

_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def library() -> ctypes.CDLL:
    """The loaded libgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with "
                               "`python -m dense_gemm_mxfp8_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        sig = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]
        for name in ("gemm_bf16", "gemm_bf16_nt"):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = sig
        lib.gemm_mxfp8.restype = ctypes.c_int
        lib.gemm_mxfp8.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp]
        lib.gemm_bf16_fused.restype = ctypes.c_int
        lib.gemm_bf16_fused.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64,
                                        ctypes.c_int, _vp, _vp, _vp, _vp]
        lib.gemm_mxfp8_fused.restype = ctypes.c_int
        lib.gemm_mxfp8_fused.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                                         ctypes.c_int, _vp, _vp, _vp, _vp]
        lib.gemm_bf16_splitk.restype = ctypes.c_int
        lib.gemm_bf16_splitk.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64,
                                         ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.gemm_bf16_splitk_plan.restype = ctypes.c_int
        lib.gemm_bf16_splitk_plan.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_size_t)]
        lib.gemm_mxfp8_splitk.restype = ctypes.c_int
        lib.gemm_mxfp8_splitk.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64, ctypes.c_int,
                                          _vp, _vp, _vp, ctypes.c_int, _vp, ctypes.c_size_t, _vp]
        lib.gemm_mxfp8_splitk_workspace.restype = ctypes.c_int
        lib.gemm_mxfp8_splitk_workspace.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                                                    ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_size_t)]
        lib.gemm_bf16_splitk_noalloc.restype = ctypes.c_int
        lib.gemm_bf16_splitk_noalloc.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64,
                                                 ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, _vp]
        lib.gemm_bf16_splitk_workspace.restype = ctypes.c_int
        lib.gemm_bf16_splitk_workspace.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp,
                                                   _i64, ctypes.c_int, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int,
                                                   ctypes.POINTER(ctypes.c_int),
                                                   ctypes.POINTER(ctypes.c_size_t)]
        lib.gemm_bf16_dynamic.restype = ctypes.c_int
        lib.gemm_bf16_dynamic.argtypes = [_i64, _i64, _i64, _vp, _i64, _vp, _i64, ctypes.c_int, _vp, _i64, _vp,
                                          ctypes.c_size_t, _vp]
        lib.attn_fwd_bf16.restype = ctypes.c_int
        lib.attn_fwd_bf16.argtypes = [_i64] * 6 + [_vp, _vp] * 4 + [_vp, ctypes.c_float, ctypes.c_int, _vp]
        lib.attn_fwd_bf16_out.restype = ctypes.c_int
        lib.attn_fwd_bf16_out.argtypes = ([_i64] * 6 + [_vp, _vp] * 4 + [ctypes.c_int, _vp, ctypes.c_float,
                                          ctypes.c_int, _vp])
        lib.gemm_strerror.restype = ctypes.c_char_p
        lib.gemm_strerror.argtypes = [ctypes.c_int]
        lib.gemm_version.restype = ctypes.c_int
        lib.gemm_version.argtypes = []
        _lib = lib
    return _lib


# ---------------------------------------------------------------- raw C ABI

def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return library().gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_nt(M, N, K, A, lda, B, ldb, C, ldc, stream) -> int:
    return library().gemm_bf16_nt(M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_mxfp8(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, stream) -> int:
    return library().gemm_mxfp8(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, stream)


def gemm_bf16_fused(M, N, K, A, lda, B, ldb, b_colmajor, C, ldc, out_type, row_scale, col_scale, bias,
                    stream) -> int:
    return library().gemm_bf16_fused(M, N, K, A, lda, B, ldb, int(b_colmajor), C, ldc, out_type, row_scale,
                                     col_scale, bias, stream)


def gemm_mxfp8_fused(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type, row_scale, col_scale, bias,
                     stream) -> int:
    return library().gemm_mxfp8_fused(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type, row_scale,
                                      col_scale, bias, stream)


def gemm_bf16_splitk(M, N, K, A, lda, B, ldb, b_colmajor, C, ldc, out_type, row_scale, col_scale, bias,
                     splits, workspace, workspace_bytes, stream) -> int:
    return library().gemm_bf16_splitk(M, N, K, A, lda, B, ldb, int(b_colmajor), C, ldc, out_type, row_scale,
                                      col_scale, bias, splits, workspace, workspace_bytes, stream)


def gemm_bf16_splitk_plan(M, N, K, b_colmajor, splits=0, cus=0):
    """(return code, K ranges used, workspace bytes) of the split-K plan."""
    used = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    rc = library().gemm_bf16_splitk_plan(M, N, K, int(b_colmajor), splits, cus, ctypes.byref(used),
                                         ctypes.byref(ws))
    return rc, used.value, ws.value


def gemm_mxfp8_splitk(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type, row_scale, col_scale, bias,
                      splits, workspace, workspace_bytes, stream) -> int:
    return library().gemm_mxfp8_splitk(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type, row_scale,
                                       col_scale, bias, splits, workspace, workspace_bytes, stream)


def gemm_mxfp8_splitk_workspace(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type, row_scale, col_scale,
                                bias, splits=0, cus=0):
    """(return code, K ranges used, workspace bytes) of gemm_mxfp8_splitk's plan."""
    used = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    rc = library().gemm_mxfp8_splitk_workspace(M, N, K, A, lda, B, ldb, scaleA, scaleB, C, ldc, out_type,
                                               row_scale, col_scale, bias, splits, cus, ctypes.byref(used),
                                               ctypes.byref(ws))
    return rc, used.value, ws.value


def gemm_bf16_splitk_noalloc(M, N, K, A, lda, B, ldb, b_colmajor, C, ldc, out_type, row_scale, col_scale, bias,
                             splits, stream) -> int:
    return library().gemm_bf16_splitk_noalloc(M, N, K, A, lda, B, ldb, int(b_colmajor), C, ldc, out_type,
                                              row_scale, col_scale, bias, splits, stream)


def gemm_bf16_splitk_workspace(M, N, K, A, lda, B, ldb, b_colmajor, C, ldc, out_type, row_scale, col_scale,
                               bias, splits=0, cus=0):
    """(return code, K ranges used, workspace bytes) of the plan gemm_bf16_splitk
    runs for these arguments (pointers are inspected, never dereferenced)."""
    used = ctypes.c_int(0)
    ws = ctypes.c_size_t(0)
    rc = library().gemm_bf16_splitk_workspace(M, N, K, A, lda, B, ldb, int(b_colmajor), C, ldc, out_type,
                                              row_scale, col_scale, bias, splits, cus, ctypes.byref(used),
                                              ctypes.byref(ws))
    return rc, used.value, ws.value


def gemm_bf16_dynamic(M, N, K, A, lda, B, ldb, b_colmajor, C, ldc, workspace, workspace_bytes, stream) -> int:
    return library().gemm_bf16_dynamic(M, N, K, A, lda, B, ldb, int(b_colmajor), C, ldc, workspace,
                                       workspace_bytes, stream)


def _strides3(s):
    """None, or 3 element strides as a host int64 array (the pointer keeps the array alive)."""
    if s is None:
        return None
    a = (ctypes.c_int64 * 3)(*[int(x) for x in s])
    return ctypes.cast(a, _vp)


def attn_fwd_bf16(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, Q, q_strides, K, k_strides, V,
                  v_strides, O, o_strides, lse, scale, causal, stream) -> int:
    """Strides: None (dense [B][H][S][D]) or a sequence of 3 element strides
    (batch, head, sequence), passed to the library as a host int64 array."""
    qa, ka, va, oa = (_strides3(s) for s in (q_strides, k_strides, v_strides, o_strides))
    return library().attn_fwd_bf16(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, Q, qa, K, ka, V, va, O,
                                   oa, lse, float(scale), int(bool(causal)), stream)


def attn_fwd_bf16_out(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, Q, q_strides, K, k_strides, V,
                      v_strides, O, o_strides, out_type, lse, scale, causal, stream) -> int:
    """attn_fwd_bf16 with the output type chosen by out_type (GEMM_OUT_F32 or GEMM_OUT_BF16)."""
    qa, ka, va, oa = (_strides3(s) for s in (q_strides, k_strides, v_strides, o_strides))
    return library().attn_fwd_bf16_out(batch, heads_q, heads_kv, seq_q, seq_k, head_dim, Q, qa, K, ka, V, va,
                                       O, oa, int(out_type), lse, float(scale), int(bool(causal)), stream)


def gemm_strerror(code: int) -> str:
    return library().gemm_strerror(code).decode()


def gemm_version() -> int:
    return library().gemm_version()


class GemmError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"libgemm error {code}: {gemm_strerror(code)}")
        self.code = code


def _check(rc: int):
    if rc != GEMM_OK:
        raise GemmError(rc)


# ---------------------------------------------------------------- tensor API

def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _out(out, M, N, device, dtype=None):
    import torch
    dtype = torch.float32 if dtype is None else dtype
    if out is None:
        return torch.empty((M, N), dtype=dtype, device=device)
    if out.shape != (M, N) or out.dtype != dtype or (N > 1 and out.stride(1) != 1):
        raise ValueError(f"out must be a {dtype} (M, N) tensor with unit column stride")
    return out


def _epilogue(out_dtype, row_scale, col_scale, bias, M, N):
    """(fused?, out_type, pointers) of the optional epilogue arguments."""
    import torch
    fused = out_dtype is not None or row_scale is not None or col_scale is not None or bias is not None
    if out_dtype not in (None, torch.float32, torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("out_dtype must be torch.float32, torch.bfloat16 or torch.float8_e4m3fn")
    ptrs = []
    for v, n, name in ((row_scale, M, "row_scale"), (col_scale, N, "col_scale"), (bias, N, "bias")):
        if v is None:
            ptrs.append(None)
            continue
        if v.dtype != torch.float32 or v.dim() != 1 or v.shape[0] != n or (n > 1 and v.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous float32 vector of length {n}")
        ptrs.append(v.data_ptr())
    out_type = {torch.bfloat16: GEMM_OUT_BF16, torch.float8_e4m3fn: GEMM_OUT_E4M3}.get(out_dtype, GEMM_OUT_F32)
    return fused, out_type, ptrs


def _bf16_operands(A, B, b_colmajor=None):
    """(M, N, K, lda, ldb, b_colmajor) of bf16 operands A (M, K) and B.

    b_colmajor None: B is the (K, N) operand, and its strides say whether it
    is row-major (unit column stride) or column-major (unit row stride).
    b_colmajor True: B is the (N, K) storage of a column-major K x N operand
    (unit stride along K), as gemm_bf16_nt reads it.  False: B is a (K, N)
    row-major tensor (unit column stride), as gemm_bf16 reads it."""
    import torch
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if b_colmajor:
        if B.dim() != 2:
            raise ValueError("B must be 2-D")
        if B.shape[0] > 1 and B.shape[1] > 1 and B.stride(1) != 1:
            raise ValueError("b_colmajor=True: B must be (N, K) with unit stride along K")
        B = B.t()
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("A must be (M, K) and B (K, N)" + (" (given as (N, K))" if b_colmajor else ""))
    M, K = A.shape
    N = B.shape[1]
    if M > 0 and K > 1 and A.stride(1) != 1:
        raise ValueError("A needs unit column stride")
    lda = A.stride(0) if M > 1 else max(K, 1)
    if b_colmajor:
        return M, N, K, lda, (B.stride(1) if N > 1 else max(K, 1)), True
    if N <= 1 or B.stride(1) == 1:
        return M, N, K, lda, (B.stride(0) if K > 1 else max(N, 1)), False
    if b_colmajor is None and B.stride(0) == 1:
        return M, N, K, lda, B.stride(1), True
    raise ValueError("B must have a unit stride along N (row-major)" +
                     (" or K (column-major)" if b_colmajor is None else ""))


def bf16(A, B, out=None, *, b_colmajor=None, out_dtype=None, row_scale=None, col_scale=None, bias=None):
    """C = A @ B in fp32 from bf16 CUDA tensors.

    A: (M, K), row-major rows (unit column stride).  B, with b_colmajor None
    (the default): a (K, N) tensor that is either row-major (unit column
    stride: ``gemm_bf16``) or column-major (unit row stride, e.g. ``Bt.t()``
    of an (N, K) tensor: ``gemm_bf16_nt``), told apart by its strides.
    b_colmajor=True: B is that (N, K) tensor itself (``gemm_bf16_nt``);
    b_colmajor=False: B must be row-major (K, N) (``gemm_bf16``).
    With any of out_dtype (float32, bfloat16 or float8_e4m3fn: OCP E4M3,
    nearest even, saturating to +-448), row_scale (M), col_scale (N) or bias
    (N) the fused epilogue applies: C = A @ B * row_scale[:, None] *
    col_scale[None, :] + bias[None, :] (``gemm_bf16_fused``)."""
    M, N, K, lda, ldb, colmajor = _bf16_operands(A, B, b_colmajor)
    fn = gemm_bf16_nt if colmajor else gemm_bf16
    fused, out_type, (rs, cs, bs) = _epilogue(out_dtype, row_scale, col_scale, bias, M, N)
    C = _out(out, M, N, A.device, out_dtype)
    ldc = C.stride(0) if M > 1 else max(N, 1)
    if fused:
        _check(gemm_bf16_fused(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, colmajor, C.data_ptr(), ldc,
                               out_type, rs, cs, bs, _stream(A.device)))
    else:
        _check(fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, _stream(A.device)))
    return C


def bf16_splitk(A, B, out=None, *, b_colmajor=None, splits=0, workspace=None, out_dtype=None, row_scale=None,
                col_scale=None, bias=None):
    """``bf16`` through ``gemm_bf16_splitk``: K cut into `splits` ranges (0:
    the library's plan) whose fp32 partial products are added in range
    order.  workspace: a CUDA tensor of at least the bytes
    ``gemm_bf16_splitk_workspace`` reports for these arguments (16-byte
    aligned); None allocates one with torch for this call."""
    import torch
    M, N, K, lda, ldb, colmajor = _bf16_operands(A, B, b_colmajor)
    _, out_type, (rs, cs, bs) = _epilogue(out_dtype, row_scale, col_scale, bias, M, N)
    C = _out(out, M, N, A.device, out_dtype)
    ldc = C.stride(0) if M > 1 else max(N, 1)
    if workspace is None:
        rc, _, nbytes = gemm_bf16_splitk_workspace(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, colmajor,
                                                   C.data_ptr(), ldc, out_type, rs, cs, bs, splits)
        _check(rc)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=A.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(gemm_bf16_splitk(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, colmajor, C.data_ptr(), ldc, out_type,
                            rs, cs, bs, splits, workspace.data_ptr(), nbytes, _stream(A.device)))
    return C


def mxfp8(A, SA, B, SB, out=None, *, out_dtype=None, row_scale=None, col_scale=None, bias=None):
    """MX block-scaled fp8 GEMM from uint8 CUDA tensors.

    A: (M, K) E4M3 codes, row-major.  B: (N, K) E4M3 codes, i.e. the K x N
    operand stored column-major.  SA: (M, K/32) and SB: (N, K/32) E8M0 codes,
    dense row-major.  The epilogue arguments are those of ``bf16``."""
    import torch
    for t, name in ((A, "A"), (B, "B"), (SA, "SA"), (SB, "SB")):
        if t.dtype != torch.uint8 or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-D uint8 tensor")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K or K % 32:
        raise ValueError("B must be (N, K) with K a multiple of 32")
    if SA.shape != (M, K // 32) or SB.shape != (N, K // 32):
        raise ValueError("scales must be (M, K/32) and (N, K/32)")
    if not (SA.is_contiguous() and SB.is_contiguous()):
        raise ValueError("scales must be dense row-major")
    if (M > 0 and K > 1 and A.stride(1) != 1) or (N > 0 and K > 1 and B.stride(1) != 1):
        raise ValueError("A and B need unit stride along K")
    lda = A.stride(0) if M > 1 else max(K, 1)
    ldb = B.stride(0) if N > 1 else max(K, 1)
    fused, out_type, (rs, cs, bs) = _epilogue(out_dtype, row_scale, col_scale, bias, M, N)
    C = _out(out, M, N, A.device, out_dtype)
    ldc = C.stride(0) if M > 1 else max(N, 1)
    if fused:
        _check(gemm_mxfp8_fused(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, SA.data_ptr(), SB.data_ptr(),
                                C.data_ptr(), ldc, out_type, rs, cs, bs, _stream(A.device)))
    else:
        _check(gemm_mxfp8(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, SA.data_ptr(),
                          SB.data_ptr(), C.data_ptr(), ldc, _stream(A.device)))
    return C


def attention(Q, K, V, *, causal=False, scale=None, out=None, lse=False, out_dtype=None):
    """Fused attention forward (``attn_fwd_bf16_out``) of bf16 CUDA tensors.

    Q: (B, Hq, Sq, D); K, V: (B, Hkv, Sk, D), Hq a multiple of Hkv, D 64 or
    128, any strides with a contiguous last dimension (so [B][S][H][D]
    storage viewed as (B, H, S, D) works).  Returns the output (B, Hq, Sq, D)
    in out_dtype (float32 by default, or bfloat16; an ``out`` tensor sets it),
    and with lse=True also the fp32 log-sum-exp (B, Hq, Sq).  scale defaults
    to 1/sqrt(D)."""
    import math
    import torch
    for t, name in ((Q, "Q"), (K, "K"), (V, "V")):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-D bfloat16 tensor")
        if t.shape[3] > 1 and t.stride(3) != 1:
            raise ValueError(f"{name} needs a contiguous last dimension")
    B, Hq, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    if K.shape != V.shape or K.shape[0] != B or K.shape[3] != D:
        raise ValueError("K and V must be (B, Hkv, Sk, D) with Q's B and D")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be torch.float32 or torch.bfloat16")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=out_dtype, device=Q.device)
    elif out.shape != (B, Hq, Sq, D) or out.dtype != out_dtype or (D > 1 and out.stride(3) != 1):
        raise ValueError("out must be a (B, Hq, Sq, D) tensor of out_dtype with a contiguous last dimension")
    L = torch.empty((B, Hq, Sq), dtype=torch.float32, device=Q.device) if lse else None
    st = lambda t: (t.stride(0), t.stride(1), t.stride(2))
    out_type = GEMM_OUT_BF16 if out_dtype == torch.bfloat16 else GEMM_OUT_F32
    _check(attn_fwd_bf16_out(B, Hq, Hkv, Sq, Sk, D, Q.data_ptr(), st(Q), K.data_ptr(), st(K), V.data_ptr(),
                             st(V), out.data_ptr(), st(out), out_type, L.data_ptr() if lse else None, scale,
                             causal, _stream(Q.device)))
    return (out, L) if lse else out
