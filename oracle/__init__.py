"""ctypes front end of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GEMM library never does.  It shares
no code with the HIP library and does not import it.

Operands are passed as numpy arrays of raw codes (``uint16`` bf16 bits,
``uint8`` e4m3 / e8m0 codes).  Any 2-D view works: the element strides of the
view are handed to the C loops, so a transposed view of a column-major B is
read in place.

``Oracle(path)`` binds one compiled copy of oracle.c; the module-level
functions use the default copy ``oracle/liboracle.so``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def build(src: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile an oracle source with the host C compiler into a shared object."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def default_threads() -> int:
    """Host threads the oracle uses: the cores this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _strides(x: np.ndarray):
    return tuple(s // x.itemsize for s in x.strides)


def _check2d(x: np.ndarray, dtype, name: str):
    if not isinstance(x, np.ndarray) or x.ndim != 2 or x.dtype != dtype:
        raise TypeError(f"{name} must be a 2-D numpy array of {np.dtype(dtype).name}")
    for s in x.strides:
        if s % x.itemsize:
            raise ValueError(f"{name} strides must be whole elements")


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        lib = ctypes.CDLL(path)
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = ctypes.c_double
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_tile_ledger.restype = ctypes.c_int
        lib.oracle_tile_ledger.argtypes = [_i64] * 6 + [_vp, _vp]
        lib.oracle_gemm_bf16.restype = ctypes.c_int
        lib.oracle_gemm_bf16.argtypes = ([_i64] * 3 + [_vp, _i64, _i64] * 2
                                         + [_vp, _vp, _i64, ctypes.c_int])
        lib.oracle_gemm_bf16_at.restype = ctypes.c_int
        lib.oracle_gemm_bf16_at.argtypes = ([_i64] * 3 + [_vp, _i64, _i64] * 2
                                            + [_vp, _vp, _i64, _vp, _vp, ctypes.c_int])
        lib.oracle_gemm_mxfp8.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8.argtypes = ([_i64] * 3 + [_vp, _i64, _i64] * 2 + [_vp, _i64] * 2
                                          + [_vp, _vp, _i64, ctypes.c_int])
        lib.oracle_gemm_mxfp8_at.restype = ctypes.c_int
        lib.oracle_gemm_mxfp8_at.argtypes = ([_i64] * 3 + [_vp, _i64, _i64] * 2
                                             + [_vp, _i64] * 2
                                             + [_vp, _vp, _i64, _vp, _vp, ctypes.c_int])
        lib.oracle_attention_fwd.restype = ctypes.c_int
        lib.oracle_attention_fwd.argtypes = ([_i64] * 6 + [_vp, _vp] * 3
                                             + [ctypes.c_double, ctypes.c_int, _vp, _vp, _vp,
                                                ctypes.c_int])
        lib.oracle_attention_fwd_at.restype = ctypes.c_int
        lib.oracle_attention_fwd_at.argtypes = ([_i64] * 6 + [_vp, _vp] * 3
                                                + [ctypes.c_double, ctypes.c_int, _vp, _i64,
                                                   _vp, _vp, _vp, ctypes.c_int])
        self.lib = lib
        self.path = path

    # ---------------------------------------------------------------- decoders
    def bf16_value(self, code: int) -> float:
        return self.lib.oracle_bf16_value(int(code))

    def e4m3_value(self, code: int) -> float:
        return self.lib.oracle_e4m3_value(int(code))

    def e8m0_value(self, code: int) -> float:
        return self.lib.oracle_e8m0_value(int(code))

    # ------------------------------------------------------------------ ledger
    def tile_ledger(self, m_tile, n_tile, k_tile, element_bytes, stages, smem_limit) -> dict:
        """Per-K-step tile ledger ("GPU 执行模型", section "Tile 小账本")."""
        out = (ctypes.c_int64 * 4)()
        ai = ctypes.c_double()
        rc = self.lib.oracle_tile_ledger(m_tile, n_tile, k_tile, element_bytes, stages,
                                         smem_limit, ctypes.cast(out, _vp),
                                         ctypes.cast(ctypes.pointer(ai), _vp))
        if rc != 0:
            raise ValueError("tile sizes, element bytes and stages must all be positive")
        return {"smem_bytes": out[0], "flops": out[1], "hbm_bytes": out[2],
                "arithmetic_intensity": ai.value, "fits_smem": bool(out[3])}

    # -------------------------------------------------------------------- GEMM
    def gemm_bf16(self, A: np.ndarray, B: np.ndarray, nthreads: int | None = None):
        """C = A @ B for bf16 bit arrays A (M,K) and B (K,N), any strides.

        Returns (C, absC): binary64 arrays of shape (M,N); absC[i,j] is
        sum_k |a(i,k)| |b(k,j)|.  Round C to float32 for the fp32 result."""
        _check2d(A, np.uint16, "A")
        _check2d(B, np.uint16, "B")
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        C = np.zeros((M, N), np.float64)
        absC = np.zeros((M, N), np.float64)
        ars, acs = _strides(A)
        brs, bcs = _strides(B)
        rc = self.lib.oracle_gemm_bf16(M, N, K, A.ctypes.data, ars, acs, B.ctypes.data, brs, bcs,
                                       C.ctypes.data, absC.ctypes.data, N,
                                       nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_gemm_bf16 rejected its arguments ({rc})")
        return C, absC

    def gemm_bf16_at(self, A: np.ndarray, B: np.ndarray, rows, cols,
                     nthreads: int | None = None):
        """(A @ B)[rows[t], cols[t]] and the matching magnitude products."""
        _check2d(A, np.uint16, "A")
        _check2d(B, np.uint16, "B")
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        rows = np.ascontiguousarray(rows, np.int64)
        cols = np.ascontiguousarray(cols, np.int64)
        n = rows.size
        out = np.zeros(n, np.float64)
        absout = np.zeros(n, np.float64)
        ars, acs = _strides(A)
        brs, bcs = _strides(B)
        rc = self.lib.oracle_gemm_bf16_at(M, N, K, A.ctypes.data, ars, acs, B.ctypes.data,
                                          brs, bcs, rows.ctypes.data, cols.ctypes.data, n,
                                          out.ctypes.data, absout.ctypes.data,
                                          nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_gemm_bf16_at rejected its arguments ({rc})")
        return out, absout

    @staticmethod
    def _mx_args(A, B, SA, SB):
        _check2d(A, np.uint8, "A")
        _check2d(B, np.uint8, "B")
        M, K = A.shape
        K2, N = B.shape
        if K2 != K:
            raise ValueError("inner dimensions differ")
        if K % 32:
            raise ValueError("K must be a multiple of 32")
        for S, rows_, name in ((SA, M, "SA"), (SB, N, "SB")):
            _check2d(S, np.uint8, name)
            if S.shape != (rows_, K // 32) or (K > 0 and S.strides[1] != 1):
                raise ValueError(f"{name} must be ({rows_}, K/32) with unit column stride")
        return M, N, K

    def gemm_mxfp8(self, A, B, SA, SB, nthreads: int | None = None):
        """MX block-scaled GEMM.  A (M,K) and B (K,N) e4m3 codes, SA (M,K/32)
        and SB (N,K/32) e8m0 codes.  Returns (C, absC) in binary64."""
        M, N, K = self._mx_args(A, B, SA, SB)
        C = np.zeros((M, N), np.float64)
        absC = np.zeros((M, N), np.float64)
        ars, acs = _strides(A)
        brs, bcs = _strides(B)
        rc = self.lib.oracle_gemm_mxfp8(M, N, K, A.ctypes.data, ars, acs, B.ctypes.data, brs, bcs,
                                        SA.ctypes.data, SA.strides[0], SB.ctypes.data,
                                        SB.strides[0], C.ctypes.data, absC.ctypes.data, N,
                                        nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_gemm_mxfp8 rejected its arguments ({rc})")
        return C, absC

    def gemm_mxfp8_at(self, A, B, SA, SB, rows, cols, nthreads: int | None = None):
        M, N, K = self._mx_args(A, B, SA, SB)
        rows = np.ascontiguousarray(rows, np.int64)
        cols = np.ascontiguousarray(cols, np.int64)
        n = rows.size
        out = np.zeros(n, np.float64)
        absout = np.zeros(n, np.float64)
        ars, acs = _strides(A)
        brs, bcs = _strides(B)
        rc = self.lib.oracle_gemm_mxfp8_at(M, N, K, A.ctypes.data, ars, acs, B.ctypes.data,
                                           brs, bcs, SA.ctypes.data, SA.strides[0],
                                           SB.ctypes.data, SB.strides[0], rows.ctypes.data,
                                           cols.ctypes.data, n, out.ctypes.data,
                                           absout.ctypes.data, nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_gemm_mxfp8_at rejected its arguments ({rc})")
        return out, absout


    # --------------------------------------------------------------- attention
    @staticmethod
    def _attn_args(Q, K, V):
        for x, name in ((Q, "Q"), (K, "K"), (V, "V")):
            if not isinstance(x, np.ndarray) or x.ndim != 4 or x.dtype != np.uint16:
                raise TypeError(f"{name} must be a 4-D numpy array of uint16 (bf16 bits)")
        B, Hq, Sq, D = Q.shape
        Bk, Hkv, Sk, Dk = K.shape
        if K.shape != V.shape or Bk != B or Dk != D:
            raise ValueError("K and V must be [B][Hkv][Sk][D] with Q's B and D")
        st = [np.ascontiguousarray(_strides(x), np.int64) for x in (Q, K, V)]
        return (B, Hq, Hkv, Sq, Sk, D), st

    def attention_fwd(self, Q, K, V, scale: float, causal: bool = False,
                      nthreads: int | None = None):
        """Softmax attention of bf16 bit arrays Q [B,Hq,Sq,D], K and V
        [B,Hkv,Sk,D] (any strides).  Returns (O, Omag, lse): O and Omag float64
        [B,Hq,Sq,D] (Omag = sum_j p_j |v(j,d)|), lse float64 [B,Hq,Sq]."""
        dims, st = self._attn_args(Q, K, V)
        B, Hq, Hkv, Sq, Sk, D = dims
        O = np.zeros((B, Hq, Sq, D), np.float64)
        Om = np.zeros_like(O)
        lse = np.zeros((B, Hq, Sq), np.float64)
        rc = self.lib.oracle_attention_fwd(B, Hq, Hkv, Sq, Sk, D,
                                           Q.ctypes.data, st[0].ctypes.data,
                                           K.ctypes.data, st[1].ctypes.data,
                                           V.ctypes.data, st[2].ctypes.data,
                                           float(scale), int(bool(causal)), O.ctypes.data,
                                           Om.ctypes.data, lse.ctypes.data,
                                           nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_attention_fwd rejected its arguments ({rc})")
        return O, Om, lse

    def attention_fwd_at(self, Q, K, V, scale: float, causal: bool, rows,
                         nthreads: int | None = None):
        """The same for sampled rows: rows is an (n, 3) array of (b, h, i).
        Returns O, Omag of shape (n, D) and lse of shape (n,)."""
        dims, st = self._attn_args(Q, K, V)
        B, Hq, Hkv, Sq, Sk, D = dims
        rows = np.ascontiguousarray(rows, np.int64).reshape(-1, 3)
        n = rows.shape[0]
        O = np.zeros((n, D), np.float64)
        Om = np.zeros_like(O)
        lse = np.zeros(n, np.float64)
        rc = self.lib.oracle_attention_fwd_at(B, Hq, Hkv, Sq, Sk, D,
                                              Q.ctypes.data, st[0].ctypes.data,
                                              K.ctypes.data, st[1].ctypes.data,
                                              V.ctypes.data, st[2].ctypes.data,
                                              float(scale), int(bool(causal)),
                                              rows.ctypes.data, n, O.ctypes.data,
                                              Om.ctypes.data, lse.ctypes.data,
                                              nthreads or default_threads())
        if rc != 0:
            raise ValueError(f"oracle_attention_fwd_at rejected its arguments ({rc})")
        return O, Om, lse


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from oracle.c in this directory (rebuilt if stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIBRARY)
    return _default


def bf16_value(code):
    return default().bf16_value(code)


def e4m3_value(code):
    return default().e4m3_value(code)


def e8m0_value(code):
    return default().e8m0_value(code)


def tile_ledger(*args, **kw):
    return default().tile_ledger(*args, **kw)


def gemm_bf16(*args, **kw):
    return default().gemm_bf16(*args, **kw)


def gemm_bf16_at(*args, **kw):
    return default().gemm_bf16_at(*args, **kw)


def gemm_mxfp8(*args, **kw):
    return default().gemm_mxfp8(*args, **kw)


def gemm_mxfp8_at(*args, **kw):
    return default().gemm_mxfp8_at(*args, **kw)


def attention_fwd(*args, **kw):
    return default().attention_fwd(*args, **kw)


def attention_fwd_at(*args, **kw):
    return default().attention_fwd_at(*args, **kw)


# ---------------------------------------------------------------- epilogue
#
# The fused epilogue is the writeback role ("Modern GPU Programming For MLSys
# - 书籍总结", section 4.3, Step 7) with the elementwise work of the fusion
# model ("GPU 执行模型", section "Fusion 的收益与上限") applied before the one
# store: t(i, j) = acc(i, j) * row_scale[i] * col_scale[j] + bias[j].  Here it
# is evaluated in binary64 on the oracle's exact product; rounding to the
# output type is a separate step.  Parity unpinned beyond the special cases
# the tests check (unit scales reduce it to the plain product; power-of-two
# scales and integer biases keep every step exact).

def epilogue(acc, mag, row_scale=None, col_scale=None, bias=None, rows=None, cols=None):
    """(t, m): t as above in float64 and m = |row_scale[i] col_scale[j]| mag,
    the magnitude the product's accuracy bound scales with.  acc and mag are
    the oracle's product and sum |a||b|, either full (M, N) arrays or values
    at the positions (rows, cols)."""
    t = np.asarray(acc, dtype=np.float64).copy()
    m = np.asarray(mag, dtype=np.float64).copy()
    full = rows is None
    if row_scale is not None:
        r = np.asarray(row_scale, dtype=np.float64)
        r = r[:, None] if full else r[rows]
        t = t * r
        m = m * np.abs(r)
    if col_scale is not None:
        c = np.asarray(col_scale, dtype=np.float64)
        c = c[None, :] if full else c[cols]
        t = t * c
        m = m * np.abs(c)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)
        b = b[None, :] if full else b[cols]
        t = t + b
    return t, m


def round_bf16(x):
    """Round float64 values to bfloat16 (8 significant bits, exponent range of
    binary32), nearest even, returned as float64.  Overflow gives +-inf, NaN
    stays NaN.  Written from the format's definition: the quantum of a value
    in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below the normal range."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    v = x[fin]
    e = np.floor(np.log2(np.abs(v)))
    # log2 can be off by one next to powers of two: correct the exponent
    e = np.where(np.abs(v) >= np.exp2(e + 1), e + 1, e)
    e = np.where(np.abs(v) < np.exp2(e), e - 1, e)
    q = np.exp2(np.maximum(e, -126.0) - 7.0)
    r = np.rint(v / q) * q  # np.rint rounds half to even
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, v), r)
    out[fin] = r
    return out


def round_e4m3(x):
    """Round float64 values to OCP FP8 E4M3 ("fn": 4 exponent bits with bias 7,
    3 mantissa bits, no infinities, largest finite value 448), nearest even,
    with saturation: results beyond +-448, infinities included, become +-448;
    NaN stays NaN.  Returned as float64 (zeros keep their sign).  Written from
    the format's definition: the quantum of a value in [2^e, 2^(e+1)) is
    2^(e-3), and 2^-9 below the normal range (e < -6).  Saturation is the
    reading taken for the fused epilogue's fp8 output (the pages name fp8
    outputs but no encoding or overflow rule)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    inf = np.isinf(x)
    out[inf] = np.copysign(448.0, x[inf])
    fin = np.isfinite(x) & (x != 0)
    v = x[fin]
    e = np.floor(np.log2(np.abs(v)))
    # log2 can be off by one next to powers of two: correct the exponent
    e = np.where(np.abs(v) >= np.exp2(e + 1), e + 1, e)
    e = np.where(np.abs(v) < np.exp2(e), e - 1, e)
    q = np.exp2(np.maximum(e, -6.0) - 3.0)
    r = np.rint(v / q) * q  # np.rint rounds half to even
    r = np.where(np.abs(r) > 448.0, np.copysign(448.0, v), r)
    out[fin] = r
    return out
