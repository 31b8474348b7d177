"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI,
run the CPU oracle on the same bytes, and compare elementwise.

Acceptance bound (floating point): |C_gpu - C_oracle| <= 1e-3 * (|A| |B|)_ij,
where (|A| |B|)_ij = sum_k |a(i,k)| |b(k,j)| comes from the oracle in binary64.
fp32 accumulation of K exact products in any order errs by at most
gamma_K * (|A||B|)_ij with gamma_K = K u / (1 - K u), u = 2^-24; for every
K used here (<= 8192) gamma_K < 4.9e-4, so the bound holds for any summation
order the kernels choose.  Integer-valued operands whose partial sums stay
below 2^24 must match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import dense_gemm_mxfp8_amd as dg
import oracle

BOUND = 1e-3


def note(msg: str):
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy().view(np.uint8)


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def assert_within_bound(got: np.ndarray, want: np.ndarray, mag: np.ndarray, what: str):
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    nan_w = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan_w), f"{what}: NaN pattern differs"
    inf_w = np.isinf(want)
    assert np.array_equal(got[inf_w], want[inf_w]), f"{what}: infinities differ"
    fin = ~(nan_w | inf_w)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite values where the oracle is finite"
    err = np.abs(got[fin] - want[fin])
    lim = BOUND * mag[fin]
    bad = err > lim
    if bad.any():
        idx = np.argwhere(fin)[bad][:5]
        ratio = (err / np.maximum(lim, 1e-300)).max()
        raise AssertionError(f"{what}: {bad.sum()} elements outside the bound "
                             f"(worst err/bound {ratio:.3g}); first at {idx.tolist()}")


def assert_exact(got: np.ndarray, want: np.ndarray, what: str):
    want32 = want.astype(np.float32)
    if not np.array_equal(got.astype(np.float32), want32):
        d = np.argwhere(got.astype(np.float32) != want32)[:5]
        raise AssertionError(f"{what}: not bit-exact at {d.tolist()}")


def sample_positions(M: int, N: int, n: int, seed: int, tile_m: int = 256, tile_n: int = 256):
    """Random output positions plus the corners, the last row/column and
    positions straddling the boundaries of the kernel's tiles (tile_m rows by
    tile_n columns: 256 x 256 for the direct-load kernels, 256 x 192 when the
    register kernel picks narrower tiles, 32-column blocks for small M)."""
    g = np.random.default_rng(seed)
    rows = list(g.integers(0, M, n))
    cols = list(g.integers(0, N, n))
    edge_r = sorted({0, M - 1, max(M - 2, 0)} | {min(M - 1, t + d) for t in range(tile_m, M, tile_m)
                                                  for d in (-1, 0)})
    edge_c = sorted({0, N - 1, max(N - 2, 0)} | {min(N - 1, t + d) for t in range(tile_n, N, tile_n)
                                                  for d in (-1, 0)})
    for r in edge_r[:64]:
        for c in g.choice(edge_c, size=min(8, len(edge_c)), replace=False):
            rows.append(r)
            cols.append(int(c))
    return np.array(rows, np.int64), np.array(cols, np.int64)


def band_lines(extent: int, tile: int, seed: int) -> np.ndarray:
    """Indices that cross every tile band of one dimension: one random index
    inside each band [b tile, (b + 1) tile), both sides of four band
    boundaries spread over the extent, and the first and last index."""
    g = np.random.default_rng(seed)
    idx = {0, extent - 1}
    for b0 in range(0, extent, tile):
        idx.add(int(g.integers(b0, min(b0 + tile, extent))))
    bounds = list(range(tile, extent, tile))
    for t in (bounds[:: max(1, len(bounds) // 4)] if bounds else []):
        idx.update((t - 1, t))
    return np.array(sorted(idx), np.int64)


def check_lines(C: np.ndarray, oracle_rows, oracle_cols, rows, cols, what: str, exact: bool = False):
    """Whole rows `rows` and whole columns `cols` of C against the oracle:
    oracle_rows(rows) -> (C[rows, :], mag) and oracle_cols(cols) -> (C[:, cols], mag)."""
    want, mag = oracle_rows(rows)
    got = C[rows, :]
    if exact:
        assert_exact(got, want, what + " (rows)")
    assert_within_bound(got, want, mag, what + " (rows)")
    want, mag = oracle_cols(cols)
    got = C[:, cols]
    if exact:
        assert_exact(got, want, what + " (columns)")
    assert_within_bound(got, want, mag, what + " (columns)")


# ------------------------------------------------------------------ bf16

def run_bf16(A: torch.Tensor, B: torch.Tensor, b_colmajor: bool, out: torch.Tensor | None = None,
             lda=None, ldb=None, ldc=None, M=None, N=None, K=None):
    """Call gemm_bf16 / gemm_bf16_nt through the C ABI on device tensors.
    A is (M, >=K) storage, B is (K, >=N) (NN) or (N, >=K) (NT) storage."""
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = (B.shape[0] if b_colmajor else B.shape[1]) if N is None else N
    lda = A.stride(0) if lda is None else lda
    ldb = B.stride(0) if ldb is None else ldb
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    ldc = out.stride(0) if ldc is None else ldc
    fn = dg.gemm_bf16_nt if b_colmajor else dg.gemm_bf16
    rc = fn(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, out.data_ptr(), ldc, stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return out


def oracle_bf16(A_bits: np.ndarray, B_bits: np.ndarray, b_colmajor: bool):
    Bv = B_bits.T if b_colmajor else B_bits
    return oracle.gemm_bf16(A_bits, Bv)


def oracle_bf16_at(A_bits, B_bits, b_colmajor, rows, cols):
    Bv = B_bits.T if b_colmajor else B_bits
    return oracle.gemm_bf16_at(A_bits, Bv, rows, cols)


def check_lines_bf16(C, A_bits, B_bits, b_colmajor, rows, cols, what, exact=False):
    """Whole rows and columns of a bf16 product against the oracle's full
    product of the matching rows of A / columns of B."""
    Bv = B_bits.T if b_colmajor else B_bits
    check_lines(C, lambda r: oracle.gemm_bf16(np.ascontiguousarray(A_bits[r]), Bv),
                lambda c: oracle.gemm_bf16(A_bits, np.ascontiguousarray(Bv[:, c])), rows, cols, what, exact)


# ------------------------------------------------------------------ MX

def run_mx(A: torch.Tensor, B: torch.Tensor, SA: torch.Tensor, SB: torch.Tensor,
           out: torch.Tensor | None = None):
    M, K = A.shape
    N = B.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    rc = dg.gemm_mxfp8(M, N, K, A.data_ptr(), A.stride(0), B.data_ptr(), B.stride(0),
                       SA.data_ptr(), SB.data_ptr(), out.data_ptr(), out.stride(0), stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return out


def oracle_mx(A, B, SA, SB):
    return oracle.gemm_mxfp8(bits8(A), bits8(B).T, bits8(SA), bits8(SB))


def oracle_mx_at(A, B, SA, SB, rows, cols):
    return oracle.gemm_mxfp8_at(bits8(A), bits8(B).T, bits8(SA), bits8(SB), rows, cols)


def check_lines_mx(C, A, B, SA, SB, rows, cols, what, exact=False):
    """Whole rows and columns of an MX product against the oracle's full
    product of the matching rows of A (and scale rows) / columns of B."""
    a, b, sa, sb = bits8(A), bits8(B), bits8(SA), bits8(SB)
    check_lines(C, lambda r: oracle.gemm_mxfp8(np.ascontiguousarray(a[r]), b.T, np.ascontiguousarray(sa[r]), sb),
                lambda c: oracle.gemm_mxfp8(a, np.ascontiguousarray(b[c]).T, sa, np.ascontiguousarray(sb[c])),
                rows, cols, what, exact)
