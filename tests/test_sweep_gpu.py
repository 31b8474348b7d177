"""Seeded sweep of the plain entry points (gemm_bf16, gemm_bf16_nt, gemm_mxfp8)
over random shapes, layouts, leading-dimension paddings and base offsets, so
that every kernel the dispatcher picks (the 128 x 128 generic kernel, the
small-M kernel, the 256 x 256 direct-load and register kernels, the MX
pipelines) meets the oracle away from the hand-picked shapes of the other
tests.

The cases come from one fixed numpy generator, in four regimes: small
products (M, N, K up to 700, and one with K = 0), skinny row-major products
(M <= 64, N >= 2048), products with enough 256 x 256 tiles for the big
kernels (M, N in [3400, 4300]), and MX products.  Each case draws a layout,
integer or normal operands, a padding of each leading dimension (aligned to
16 bytes or not) and a base offset of 0 or one element.  Padding elements
hold NaN and C has a sentinel guard band: neither may leak.  Integer cases
must be bit-exact; normal ones within |C - exact| <= 1e-3 sum_k |a||b|.
bf16 outputs are compared whole; large MX outputs by whole rows and columns
crossing every 256-row and 256-column band (the MX oracle decodes every
product and is about ten times slower than the bf16 one).

A third sweep runs gemm_bf16_splitk with a random epilogue (row scales,
column scales, bias, each present or not; fp32, bf16 or E4M3 output) and a
random range count (0 lets the plan decide), on long-K, skinny and ragged
products with padded leading dimensions, the workspace sized by
gemm_bf16_splitk_workspace for exactly those arguments and filled with NaN.
The tolerance is the fused epilogue's (oracle.epilogue, then the output
type's rounding)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
import oracle
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P
from tests.test_fused_gpu import OUT_DTYPE, OUT_TYPE, _compare, _vectors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = -4321.0


def _bf16_cases():
    g = np.random.default_rng(20261203)
    cases = []

    def add(regime, M, N, K, nt):
        aligned = bool(g.integers(0, 2))
        dist = "integer" if g.integers(0, 2) else "normal"
        if aligned:
            pad_a, pad_b, off = int(g.integers(0, 3)) * 8, int(g.integers(0, 3)) * 8, 0
        else:
            pad_a, pad_b, off = int(g.integers(1, 8)), int(g.integers(0, 8)), int(g.integers(0, 2))
        pad_c = int(g.integers(0, 9))
        cases.append((regime, M, N, K, nt, dist, pad_a, pad_b, pad_c, off, len(cases)))

    for _ in range(24):
        add("small", int(g.integers(1, 701)), int(g.integers(1, 701)), int(g.integers(0, 701)),
            bool(g.integers(0, 2)))
    add("small", 77, 129, 0, True)
    for _ in range(14):
        add("skinny", int(g.integers(1, 65)), int(g.integers(2048, 5001)), int(g.integers(32, 2001)), False)
    for _ in range(16):
        add("big", int(g.integers(3400, 4301)), int(g.integers(3400, 4301)), int(g.integers(16, 401)),
            bool(g.integers(0, 2)))
    return cases


def _mx_cases():
    g = np.random.default_rng(20261204)
    cases = []
    for i in range(14):
        big = i >= 6
        M = int(g.integers(3400, 4301)) if big else int(g.integers(1, 600))
        N = int(g.integers(3400, 4301)) if big else int(g.integers(1, 600))
        # big cases lean towards the direct-load MX pipelines (K a multiple of
        # 64, rows 16-byte aligned); the scale base offset (16-byte, 2-byte or
        # 1-byte aligned) then picks the scale ring, the four-stage pipeline or
        # the generic kernel
        K = 64 * int(g.integers(1, 9)) if big and g.integers(0, 4) else 32 * int(g.integers(1, 17))
        dist = "integer" if g.integers(0, 2) else "normal"
        pad = int(g.integers(0, 3)) * 16 if g.integers(0, 4) else int(g.integers(1, 16))
        soff = int(g.choice([0, 0, 2, 1]))
        cases.append((M, N, K, dist, pad, soff, i))
    return cases


def _split_cases():
    g = np.random.default_rng(20261205)
    cases = []
    for i in range(18):
        r = i % 3
        if r == 0:  # long K, few tiles
            M, N, K, nt = int(g.integers(64, 1200)), int(g.integers(64, 1200)), int(g.integers(2048, 12001)), \
                bool(g.integers(0, 2))
        elif r == 1:  # skinny, row-major B (32- or 128-column strips)
            M, N, K, nt = int(g.integers(1, 33)), int(g.integers(2048, 6001)), int(g.integers(1024, 8193)), False
        else:  # ragged edges, moderate K
            M, N, K, nt = int(g.integers(300, 1500)), int(g.integers(300, 1500)), int(g.integers(512, 4097)), \
                bool(g.integers(0, 2))
        splits = 0 if g.integers(0, 2) else int(g.integers(1, 13))
        which = "".join(ch for ch in "rcb" if g.integers(0, 2))
        out = str(g.choice(["f32", "bf16", "e4m3"]))
        exact = bool(g.integers(0, 2))
        pad = int(g.integers(0, 3)) * 8 if g.integers(0, 3) else int(g.integers(1, 8))
        cases.append((M, N, K, nt, splits, which, out, exact, pad, i))
    return cases


BF16 = _bf16_cases()
MX = _mx_cases()
SPLIT = _split_cases()


def _padded(t: torch.Tensor, ld: int, off: int, fill) -> tuple[torch.Tensor, int]:
    """Device storage holding t's rows at pitch ld, starting off elements in;
    the padding (and the offset) hold `fill`.  Returns (storage, byte offset)."""
    rows, cols = t.shape
    st = torch.full((off + rows * ld + 8,), fill, dtype=t.dtype)
    st[off:off + rows * ld].view(rows, ld)[:, :cols] = t
    return st.to(DEV), off * t.element_size()


@pytest.mark.parametrize("case", BF16, ids=lambda c: f"{c[10]}_{c[0]}_{c[1]}x{c[2]}x{c[3]}_{'nt' if c[4] else 'nn'}"
                         f"_{c[5]}_pad{c[6]}.{c[7]}.{c[8]}_off{c[9]}")
def test_bf16_sweep(case):
    regime, M, N, K, nt, dist, pad_a, pad_b, pad_c, off, idx = case
    g = inputs.generator(1000 + idx)
    make = inputs.integer_bf16 if dist == "integer" else inputs.normal_bf16
    A = make((M, K), g)
    B = make((N, K) if nt else (K, N), g)
    lda = K + pad_a
    ldb = B.shape[1] + pad_b
    ldc = N + pad_c
    nan = float("nan")
    Ad, aoff = _padded(A, max(lda, 1), off, nan)
    Bd, boff = _padded(B, max(ldb, 1), off, nan)
    C = torch.full((M + 2, ldc), SENTINEL, dtype=torch.float32, device=DEV)
    P.note(f"sweep bf16 {idx} {regime} {M}x{N}x{K} {'NT' if nt else 'NN'} {dist} lda {lda} ldb {ldb} "
           f"ldc {ldc} off {off}")
    fn = dg.gemm_bf16_nt if nt else dg.gemm_bf16
    rc = fn(M, N, K, Ad.data_ptr() + aoff, max(lda, 1), Bd.data_ptr() + boff, max(ldb, 1), C.data_ptr(), ldc,
            P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    assert (Ch[:, N:] == SENTINEL).all() and (Ch[M:] == SENTINEL).all(), "C written outside M x N"
    got = Ch[:M, :N].astype(np.float64)
    if K == 0:
        assert (got == 0).all()
        return
    want, mag = P.oracle_bf16(P.bits16(A), P.bits16(B), nt)
    if dist == "integer":
        P.assert_exact(got, want, f"sweep {idx}")
    P.assert_within_bound(got, want, mag, f"sweep {idx}")


@pytest.mark.parametrize("case", MX, ids=lambda c: f"{c[6]}_{c[0]}x{c[1]}x{c[2]}_{c[3]}_pad{c[4]}_soff{c[5]}")
def test_mx_sweep(case):
    M, N, K, dist, pad, soff, idx = case
    prob = inputs.mx_problem(M, N, K, dist=dist, seed=2000 + idx)
    lda = K + pad
    Ad, aoff = _padded(prob.A, lda, 0, 0x7F)  # padding: the E4M3 NaN code
    Bd, boff = _padded(prob.B, lda, 0, 0x7F)
    SA = torch.full((soff + prob.SA.numel() + 16,), 0xFF, dtype=torch.uint8)  # E8M0 NaN around the scales
    SA[soff:soff + prob.SA.numel()] = prob.SA.reshape(-1)
    SB = torch.full((soff + prob.SB.numel() + 16,), 0xFF, dtype=torch.uint8)
    SB[soff:soff + prob.SB.numel()] = prob.SB.reshape(-1)
    SAd, SBd = SA.to(DEV), SB.to(DEV)
    C = torch.full((M + 2, N + 3), SENTINEL, dtype=torch.float32, device=DEV)
    P.note(f"sweep mx {idx} {M}x{N}x{K} {dist} lda {lda} scale offset {soff}")
    rc = dg.gemm_mxfp8(M, N, K, Ad.data_ptr() + aoff, lda, Bd.data_ptr() + boff, lda, SAd.data_ptr() + soff,
                       SBd.data_ptr() + soff, C.data_ptr(), N + 3, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    assert (Ch[:, N:] == SENTINEL).all() and (Ch[M:] == SENTINEL).all(), "C written outside M x N"
    got = Ch[:M, :N].astype(np.float64)
    exact = dist == "integer"
    if M * N <= 600 * 600:
        want, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
        if exact:
            P.assert_exact(got, want, f"mx sweep {idx}")
        P.assert_within_bound(got, want, mag, f"mx sweep {idx}")
    else:
        rows = P.band_lines(M, 256, 3000 + idx)
        cols = P.band_lines(N, 256, 4000 + idx)
        P.check_lines_mx(got, prob.A, prob.B, prob.SA, prob.SB, rows, cols, f"mx sweep {idx}", exact)


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"{c[9]}_{c[0]}x{c[1]}x{c[2]}_{'nt' if c[3] else 'nn'}"
                         f"_s{c[4]}_{c[5] or 'none'}_{c[6]}_{'integer' if c[7] else 'normal'}_pad{c[8]}")
def test_splitk_sweep(case):
    M, N, K, nt, splits, which, out, exact, pad, idx = case
    prob = inputs.bf16_problem(M, N, K, dist="integer" if exact else "normal", b_colmajor=nt, seed=5000 + idx)
    vecs = _vectors(M, N, exact, 6000 + idx, which)
    lda = K + pad
    ldb = prob.B.shape[1] + pad
    Ad, _ = _padded(prob.A, lda, 0, float("nan"))
    Bd, _ = _padded(prob.B, ldb, 0, float("nan"))
    ldc = N + 5
    Cst = torch.full((M, ldc), -7.0, dtype=OUT_DTYPE[out], device=DEV)
    rs, cs, bias = (None if v is None else torch.from_numpy(v).to(DEV) for v in vecs)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    args = (M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, nt, Cst.data_ptr(), ldc, OUT_TYPE[out], ptr(rs),
            ptr(cs), ptr(bias), splits)
    rc, used, nbytes = dg.gemm_bf16_splitk_workspace(*args)
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    P.note(f"sweep split {idx} {M}x{N}x{K} {'NT' if nt else 'NN'} splits {splits} -> {used} {which} {out} "
           f"pad {pad}")
    rc = dg.gemm_bf16_splitk(*args, ws.data_ptr(), ws.numel() * 4, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    C = Cst.float().cpu().numpy()
    assert (C[:, N:] == -7.0).all(), "C written outside M x N"
    got = np.ascontiguousarray(C[:, :N]).astype(np.float64)
    acc, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), nt)
    t, m = oracle.epilogue(acc, mag, *vecs)
    b = np.zeros_like(t) if vecs[2] is None else np.abs(vecs[2].astype(np.float64))[None, :]
    _compare(got, t, m, b, out, exact, f"split sweep {idx} ({used} ranges)")
