"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact.  The pins come from:
  - the tile-ledger worked example and its stated invariants
    ("GPU 执行模型", section "Tile 小账本"), stored under tests/golden/;
  - exact rational brute force (``fractions.Fraction``) on tiny shapes;
  - closed forms: identity and permutation products, integer-valued
    operands whose sums are exact, Freivalds' identity C x = A (B x);
  - library special cases: torch's own bf16 / float8_e4m3fn / float8_e8m0fnu
    decoders and numpy's float64 and int64 matrix products;
  - IEEE special-value propagation and the MX block-scale algebra
    (a scale code shifted by d multiplies exactly that block by 2^d).
``tests/test_oracle.py`` runs every pin on the real oracle and
``tests/test_oracle_mutations.py`` checks that planted mistakes in copies of
oracle.c make at least one pin fail.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_from_f32(a) -> np.ndarray:
    return bf16_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def torch_bf16_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bits with torch (a library decoder, independent of the oracle)."""
    return torch.from_numpy(bits.astype(np.int16).copy()).view(torch.bfloat16).double().numpy()


def torch_e4m3_f64(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()


def rng(seed):
    return np.random.default_rng(seed)


def random_bf16(shape, seed, scale=1.0):
    return bf16_from_f32(rng(seed).standard_normal(shape) * scale)


VALID_E4M3 = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def random_e4m3(shape, seed):
    return rng(seed).choice(VALID_E4M3, size=shape).astype(np.uint8)


def frac_bf16(code) -> Fraction:
    """Exact rational value of a (finite) bf16 code from its bit fields."""
    code = int(code)
    s = -1 if code >> 15 else 1
    e = (code >> 7) & 0xFF
    m = code & 0x7F
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def frac_e4m3(code) -> Fraction:
    code = int(code)
    s = -1 if code >> 7 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(2) ** -6
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


# ---------------------------------------------------------------- ledger

def pin_ledger_worked_example(orc):
    with open(os.path.join(GOLDEN, "tile_ledger_worked_example.json")) as f:
        g = json.load(f)
    got = orc.tile_ledger(**g["args"])
    for key, want in g["expect"].items():
        assert got[key] == want, (key, got[key], want)


def pin_ledger_invariants(orc):
    for (m, n, k, eb) in [(64, 64, 32, 2), (256, 256, 64, 2), (256, 256, 128, 1), (16, 64, 512, 2),
                          (3, 5, 7, 4)]:
        base = orc.tile_ledger(m, n, k, eb, 1, 1 << 30)
        for stages in (1, 2, 3, 4):
            led = orc.tile_ledger(m, n, k, eb, stages, 1 << 30)
            # stages add residency only: the logical HBM read of the tile is unchanged
            assert led["hbm_bytes"] == base["hbm_bytes"] == eb * (m * k + k * n)
            assert led["smem_bytes"] == stages * led["hbm_bytes"]
            # one multiply-add is two operations
            assert led["flops"] == 2 * m * n * k
            assert led["arithmetic_intensity"] == led["flops"] / led["hbm_bytes"]
            assert orc.tile_ledger(m, n, k, eb, stages, led["smem_bytes"])["fits_smem"]
            assert not orc.tile_ledger(m, n, k, eb, stages, led["smem_bytes"] - 1)["fits_smem"]
    for bad in [(0, 1, 1, 1, 1), (1, 0, 1, 1, 1), (1, 1, 0, 1, 1), (1, 1, 1, 0, 1), (1, 1, 1, 1, 0)]:
        try:
            orc.tile_ledger(*bad, 1024)
        except ValueError:
            continue
        raise AssertionError(f"ledger accepted non-positive sizes {bad}")


# ---------------------------------------------------------------- decoders

def pin_bf16_decode(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch_bf16_f64(codes)
    got = np.array([orc.bf16_value(c) for c in codes.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert orc.bf16_value(0x3F80) == 1.0 and orc.bf16_value(0xC000) == -2.0
    assert orc.bf16_value(0x0001) == 2.0 ** -133


def pin_e4m3_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch_e4m3_f64(codes)
    got = np.array([orc.e4m3_value(c) for c in codes.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    # closed-form points of OCP E4M3: one, smallest normal, smallest subnormal, largest
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0xFE) == -448.0
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))
    assert orc.e4m3_value(0x80) == 0.0 and math.copysign(1, orc.e4m3_value(0x80)) < 0
    # every finite code equals its field-wise rational value
    for c in range(256):
        if (c & 0x7F) != 0x7F:
            assert Fraction(orc.e4m3_value(c)) == frac_e4m3(c), c


def pin_e8m0_decode(orc):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double()
    for e in range(256):
        got = orc.e8m0_value(e)
        if e == 255:
            assert math.isnan(got)
            continue
        assert got == 2.0 ** (e - 127), e
        assert got == ref[e].item() or (e == 0 and ref[e].item() == 2.0 ** -127), e


# ---------------------------------------------------------------- bf16 GEMM

TINY = [(0, 3, 2), (3, 0, 2), (2, 3, 0), (1, 1, 1), (1, 5, 3), (3, 1, 5), (2, 3, 17), (5, 8, 2),
        (8, 5, 17), (17, 3, 8), (3, 17, 5), (17, 17, 17)]


def pin_bf16_bruteforce(orc):
    for t, (M, N, K) in enumerate(TINY):
        A = random_bf16((M, K), 100 + t)
        B = random_bf16((K, N), 200 + t)
        C, absC = orc.gemm_bf16(A, B)
        assert C.shape == (M, N)
        for i in range(M):
            for j in range(N):
                exact = sum((frac_bf16(A[i, k]) * frac_bf16(B[k, j]) for k in range(K)), Fraction(0))
                mag = sum((abs(frac_bf16(A[i, k]) * frac_bf16(B[k, j])) for k in range(K)),
                          Fraction(0))
                tol = Fraction(K, 2 ** 50) * mag
                assert abs(Fraction(C[i, j]) - exact) <= tol, (M, N, K, i, j)
                assert abs(Fraction(absC[i, j]) - mag) <= tol, (M, N, K, i, j)


def pin_bf16_identity_permutation(orc):
    M, K, N = 37, 29, 23
    A = random_bf16((M, K), 1)
    B = random_bf16((K, N), 2)
    I_k = bf16_from_f32(np.eye(K))
    I_m = bf16_from_f32(np.eye(M))
    C, _ = orc.gemm_bf16(A, I_k)
    assert np.array_equal(C.astype(np.float32), torch_bf16_f64(A).astype(np.float32))
    C, _ = orc.gemm_bf16(I_k, B)
    assert np.array_equal(C, torch_bf16_f64(B))
    perm = rng(3).permutation(K)
    P = bf16_from_f32(np.eye(K)[perm])  # (P B)[r] = B[perm[r]]
    C, _ = orc.gemm_bf16(P, B)
    assert np.array_equal(C, torch_bf16_f64(B)[perm])
    C, _ = orc.gemm_bf16(I_m, A)
    assert np.array_equal(C, torch_bf16_f64(A))


def pin_bf16_integer_exact(orc):
    for t, (M, N, K) in enumerate([(64, 48, 40), (33, 65, 130), (7, 300, 257)]):
        g = rng(10 + t)
        Ai = g.integers(-4, 5, size=(M, K))
        Bi = g.integers(-4, 5, size=(K, N))
        C, absC = orc.gemm_bf16(bf16_from_f32(Ai), bf16_from_f32(Bi))
        assert np.array_equal(C, (Ai @ Bi).astype(np.float64))
        assert np.array_equal(absC, (np.abs(Ai) @ np.abs(Bi)).astype(np.float64))


def pin_bf16_freivalds(orc):
    M, K, N = 384, 256, 320
    A = random_bf16((M, K), 20)
    B = random_bf16((K, N), 21)
    C, absC = orc.gemm_bf16(A, B)
    for s in range(3):
        x = rng(30 + s).standard_normal(N)
        lhs = C @ x
        rhs = torch_bf16_f64(A) @ (torch_bf16_f64(B) @ x)
        tol = 1e-11 * (absC @ np.abs(x)) + 1e-300
        assert np.all(np.abs(lhs - rhs) <= tol)


def pin_bf16_strided_views(orc):
    """Column-major B read through a transposed view, a padded lda, and the
    sampled entry point all give the same (bit-identical) elements."""
    M, N, K = 19, 27, 45
    A = random_bf16((M, K), 40)
    Bt = random_bf16((N, K), 41)           # column-major K x N storage
    C_nt, _ = orc.gemm_bf16(A, Bt.T)
    C_nn, _ = orc.gemm_bf16(A, np.ascontiguousarray(Bt.T))
    assert np.array_equal(C_nt, C_nn)
    Apad = np.full((M, K + 13), 0x7FC0, np.uint16)  # NaN padding beyond K
    Apad[:, :K] = A
    C_pad, _ = orc.gemm_bf16(Apad[:, :K], Bt.T)
    assert np.array_equal(C_pad, C_nn)
    rows = rng(42).integers(0, M, 50)
    cols = rng(43).integers(0, N, 50)
    s, sabs = orc.gemm_bf16_at(A, Bt.T, rows, cols)
    _, absC = orc.gemm_bf16(A, Bt.T)
    assert np.array_equal(s, C_nn[rows, cols]) and np.array_equal(sabs, absC[rows, cols])
    # C^T = B^T A^T
    CT, _ = orc.gemm_bf16(Bt, A.T)
    assert np.array_equal(CT, C_nn.T)


def pin_bf16_special_values(orc):
    M, N, K = 6, 7, 9
    A = random_bf16((M, K), 50)
    B = random_bf16((K, N), 51)
    clean, _ = orc.gemm_bf16(A, B)
    An = A.copy()
    An[2, 4] = 0x7FC0  # NaN
    C, _ = orc.gemm_bf16(An, B)
    assert np.isnan(C[2]).all()
    keep = [r for r in range(M) if r != 2]
    assert np.array_equal(C[keep], clean[keep])
    Ai = A.copy()
    Ai[3, 1] = 0x7F80  # +Inf
    Bz = B.copy()
    Bz[1, 5] = 0x0000  # zero meets the infinity in column 5
    C, _ = orc.gemm_bf16(Ai, Bz)
    assert math.isnan(C[3, 5])
    for j in range(N):
        if j != 5:
            assert math.isinf(C[3, j])


# ---------------------------------------------------------------- MX GEMM

def _mx_random(M, N, K, seed, lo=120, hi=134):
    g = rng(seed)
    A = random_e4m3((M, K), seed + 1)
    Bt = random_e4m3((N, K), seed + 2)
    SA = g.integers(lo, hi + 1, size=(M, K // 32)).astype(np.uint8)
    SB = g.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)
    return A, Bt, SA, SB


def pin_mx_bruteforce(orc):
    for t, (M, N, K) in enumerate([(3, 4, 32), (5, 2, 64), (2, 3, 96), (1, 1, 32), (4, 4, 0)]):
        A, Bt, SA, SB = _mx_random(M, N, K, 300 + 10 * t)
        C, absC = orc.gemm_mxfp8(A, Bt.T, SA, SB)
        for i in range(M):
            for j in range(N):
                exact = Fraction(0)
                mag = Fraction(0)
                for b in range(K // 32):
                    sc = Fraction(2) ** (int(SA[i, b]) - 127) * Fraction(2) ** (int(SB[j, b]) - 127)
                    for k in range(32 * b, 32 * b + 32):
                        p = frac_e4m3(A[i, k]) * frac_e4m3(Bt[j, k]) * sc
                        exact += p
                        mag += abs(p)
                tol = Fraction(max(K, 1), 2 ** 50) * mag
                assert abs(Fraction(C[i, j]) - exact) <= tol, (M, N, K, i, j)
                assert abs(Fraction(absC[i, j]) - mag) <= tol


def pin_mx_unit_scales(orc):
    """With every scale code 127 (scale 1) the MX product is the plain product
    of the decoded e4m3 matrices (numpy float64 matmul of torch-decoded values)."""
    M, N, K = 40, 24, 96
    A, Bt, _, _ = _mx_random(M, N, K, 400)
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C, absC = orc.gemm_mxfp8(A, Bt.T, SA, SB)
    ref = torch_e4m3_f64(A) @ torch_e4m3_f64(Bt).T
    assert np.all(np.abs(C - ref) <= 1e-12 * absC)


def pin_mx_scale_algebra(orc):
    M, N, K = 6, 5, 128
    A, Bt, SA, SB = _mx_random(M, N, K, 500)
    C, _ = orc.gemm_mxfp8(A, Bt.T, SA, SB)
    # shifting every scale of row i by +1 doubles row i exactly
    SA2 = SA.copy()
    SA2[2, :] += 1
    C2, _ = orc.gemm_mxfp8(A, Bt.T, SA2, SB)
    assert np.array_equal(C2[2], 2 * C[2])
    assert np.array_equal(np.delete(C2, 2, 0), np.delete(C, 2, 0))
    # shifting one block's scale by d changes row i by (2^d - 1) times that block's part
    for (i, b, d) in [(1, 0, 3), (4, 3, 2), (0, 2, -1)]:
        SA3 = SA.copy()
        SA3[i, b] = int(SA[i, b]) + d
        C3, _ = orc.gemm_mxfp8(A, Bt.T, SA3, SB)
        part, _ = orc.gemm_mxfp8(np.ascontiguousarray(A[:, 32 * b:32 * b + 32]),
                                 np.ascontiguousarray(Bt[:, 32 * b:32 * b + 32]).T,
                                 np.ascontiguousarray(SA[:, b:b + 1]),
                                 np.ascontiguousarray(SB[:, b:b + 1]))
        want = C[i] + (2.0 ** d - 1) * part[i]
        assert np.all(np.abs(C3[i] - want) <= 1e-12 * np.abs(want).max()), (i, b, d)
    # a column's scale shift doubles that column
    SB2 = SB.copy()
    SB2[3, :] += 1
    C4, _ = orc.gemm_mxfp8(A, Bt.T, SA, SB2)
    assert np.array_equal(C4[:, 3], 2 * C[:, 3])


def pin_mx_integer_exact(orc):
    M, N, K = 48, 40, 256
    g = rng(600)
    Ai = g.integers(-8, 9, size=(M, K))
    Bi = g.integers(-8, 9, size=(N, K))
    enc = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    SA = np.full((M, K // 32), 127, np.uint8)
    SB = np.full((N, K // 32), 127, np.uint8)
    C, _ = orc.gemm_mxfp8(enc(Ai), enc(Bi).T, SA, SB)
    assert np.array_equal(C, (Ai @ Bi.T).astype(np.float64))


def pin_mx_nan(orc):
    M, N, K = 4, 5, 64
    A, Bt, SA, SB = _mx_random(M, N, K, 700)
    clean, _ = orc.gemm_mxfp8(A, Bt.T, SA, SB)
    A2 = A.copy()
    A2[1, 40] = 0x7F
    C, _ = orc.gemm_mxfp8(A2, Bt.T, SA, SB)
    assert np.isnan(C[1]).all() and np.array_equal(np.delete(C, 1, 0), np.delete(clean, 1, 0))
    SB2 = SB.copy()
    SB2[2, 1] = 0xFF
    C, _ = orc.gemm_mxfp8(A, Bt.T, SA, SB2)
    assert np.isnan(C[:, 2]).all() and np.array_equal(np.delete(C, 2, 1), np.delete(clean, 2, 1))


def pin_mx_sampled(orc):
    """The sampled MX entry point equals the full product element for element,
    at M != N, for positions that include the last row and column; a scale
    shift on a sampled row doubles exactly that row's sampled outputs."""
    M, N, K = 53, 37, 160
    A, Bt, SA, SB = _mx_random(M, N, K, 800)
    C, absC = orc.gemm_mxfp8(A, Bt.T, SA, SB)
    g = rng(801)
    # positions inside the leading min(M, N) square first: a sampler that
    # swaps or repeats the indices reads in bounds there and must disagree
    sq = min(M, N)
    rows = np.concatenate([g.integers(0, sq, 60), np.arange(sq)])
    cols = np.concatenate([g.integers(0, sq, 60), (np.arange(sq) * 7 + 3) % sq])
    s, sabs = orc.gemm_mxfp8_at(A, Bt.T, SA, SB, rows, cols)
    assert np.array_equal(s, C[rows, cols]) and np.array_equal(sabs, absC[rows, cols])
    # the whole range: every last row and last column position
    rows = np.concatenate([g.integers(0, M, 80), np.full(N, M - 1), np.arange(M)])
    cols = np.concatenate([g.integers(0, N, 80), np.arange(N), np.full(M, N - 1)])
    s, sabs = orc.gemm_mxfp8_at(A, Bt.T, SA, SB, rows, cols)
    assert np.array_equal(s, C[rows, cols]) and np.array_equal(sabs, absC[rows, cols])
    # +1 on every scale code of row 11 doubles its sampled outputs; +2 on
    # block 3 of column 5 adds 3 times that block's part to column 5
    SA2 = SA.copy()
    SA2[11, :] += 1
    s2, _ = orc.gemm_mxfp8_at(A, Bt.T, SA2, SB, rows, cols)
    on = rows == 11
    assert on.any() and np.array_equal(s2[on], 2 * s[on]) and np.array_equal(s2[~on], s[~on])
    SB2 = SB.copy()
    SB2[5, 3] += 2
    s3, _ = orc.gemm_mxfp8_at(A, Bt.T, SA, SB2, rows, cols)
    part, _ = orc.gemm_mxfp8(np.ascontiguousarray(A[:, 96:128]), np.ascontiguousarray(Bt[:, 96:128]).T,
                             np.ascontiguousarray(SA[:, 3:4]), np.ascontiguousarray(SB[:, 3:4]))
    on = cols == 5
    want = s[on] + 3.0 * part[rows[on], 5]
    assert on.any() and np.all(np.abs(s3[on] - want) <= 1e-12 * np.abs(absC[rows[on], 5]))
    assert np.array_equal(s3[~on], s[~on])


ALL_PINS = [
    pin_ledger_worked_example, pin_ledger_invariants,
    pin_bf16_decode, pin_e4m3_decode, pin_e8m0_decode,
    pin_bf16_bruteforce, pin_bf16_identity_permutation, pin_bf16_integer_exact,
    pin_bf16_freivalds, pin_bf16_strided_views, pin_bf16_special_values,
    pin_mx_bruteforce, pin_mx_unit_scales, pin_mx_scale_algebra, pin_mx_integer_exact, pin_mx_nan,
    pin_mx_sampled,
]


# the attention oracle's pins (part IV of the MLSys book summary) run with these
from tests.oracle_attn_pins import ATTN_PINS  # noqa: E402

ALL_PINS = ALL_PINS + ATTN_PINS
