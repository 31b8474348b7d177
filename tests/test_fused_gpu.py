"""GPU parity of the fused epilogue (gemm_bf16_fused, gemm_mxfp8_fused)
through the C ABI, on shapes that reach every kernel: the generic tiles, the
256 x 256 direct-load kernel (NT, NN, MX with the scale ring), the
register-load kernel (2-byte aligned rows, 192-column tiles) and the small-M
kernel, plus K == 0.

Reference: the oracle's exact product with the epilogue applied in binary64
(oracle.epilogue), rounded to bf16 by oracle.round_bf16 where that is the
output type.  Tolerance for floating point:
    |C - t| <= 1e-3 * |rs cs| sum|a||b|  +  2^-21 (|t| + |bias|)   (fp32 out)
and, for bf16 output, additionally half a bf16 unit of t (2^-8 |t|).
Integer operands with power-of-two scales and integer biases keep every step
exact, so those cases must match bit for bit (bf16: round_bf16 of the exact t)."""
import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
import oracle
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _vectors(M, N, exact, seed, which):
    g = np.random.default_rng(seed)
    if exact:
        rs = np.exp2(g.integers(-2, 3, size=M)).astype(np.float32)
        cs = np.exp2(g.integers(-2, 3, size=N)).astype(np.float32)
        bias = g.integers(-8, 9, size=N).astype(np.float32)
    else:
        rs = (g.standard_normal(M) * 2).astype(np.float32)
        cs = (g.uniform(-1, 1, size=N)).astype(np.float32)
        bias = (g.standard_normal(N) * 10).astype(np.float32)
    return (rs if "r" in which else None, cs if "c" in which else None, bias if "b" in which else None)


def _dev(v):
    return None if v is None else torch.from_numpy(v).to(DEV)


def _run(kind, prob, out_bf16, vecs, ldc_pad=3):
    M, N, K = prob.M, prob.N, prob.K
    rs, cs, bias = (_dev(v) for v in vecs)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    odt = torch.bfloat16 if out_bf16 else torch.float32
    ldc = N + ldc_pad
    Cst = torch.full((M, ldc), -7.0, dtype=odt, device=DEV)
    out_type = dg.GEMM_OUT_BF16 if out_bf16 else dg.GEMM_OUT_F32
    if kind == "mx":
        A, B, SA, SB = (x.to(DEV) for x in (prob.A, prob.B, prob.SA, prob.SB))
        rc = dg.gemm_mxfp8_fused(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(),
                                 Cst.data_ptr(), ldc, out_type, ptr(rs), ptr(cs), ptr(bias), P.stream())
    else:
        A, B = prob.A.to(DEV), prob.B.to(DEV)
        ldb = K if prob.b_colmajor else N
        rc = dg.gemm_bf16_fused(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor, Cst.data_ptr(),
                                ldc, out_type, ptr(rs), ptr(cs), ptr(bias), P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    C = Cst.float().cpu().numpy()
    assert (C[:, N:] == -7.0).all(), "C written outside M x N"
    return np.ascontiguousarray(C[:, :N]).astype(np.float64)


# The last problem built and its oracle product are kept, so the output
# types of one shape share them (problems are dataclasses, not hashable: the
# cache is keyed by the arguments that built the problem).
_LAST = {"key": None, "prob": None, "product": None}


def _problem(kind, M, N, K, colmajor, exact, seed):
    key = (kind, M, N, K, colmajor, exact, seed)
    if _LAST["key"] != key:
        _LAST.update(key=key, product=None, prob=(
            inputs.mx_problem(M, N, K, dist="integer" if exact else "normal", seed=seed) if kind == "mx"
            else _bf16_prob(M, N, K, colmajor, exact, seed)))
    return _LAST["prob"]


def _product(kind, prob):
    """The oracle's full product of one problem (cached for the last problem)."""
    if prob is _LAST["prob"] and _LAST["product"] is not None:
        return _LAST["product"]
    if kind == "mx":
        res = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    else:
        res = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), prob.b_colmajor)
    if prob is _LAST["prob"]:
        _LAST["product"] = res
    return res


def _reference(kind, prob, vecs, rows=None, cols=None):
    if rows is None:
        acc, mag = _product(kind, prob)
    elif kind == "mx":
        acc, mag = P.oracle_mx_at(prob.A, prob.B, prob.SA, prob.SB, rows, cols)
    else:
        acc, mag = P.oracle_bf16_at(P.bits16(prob.A), P.bits16(prob.B), prob.b_colmajor, rows, cols)
    rs, cs, bias = vecs
    t, m = oracle.epilogue(acc, mag, rs, cs, bias, rows=rows, cols=cols)
    b = np.zeros_like(t) if bias is None else np.abs(bias.astype(np.float64)[None, :] if rows is None
                                                    else bias.astype(np.float64)[cols])
    return t, m, b


def _compare(got, t, m, b, out_bf16, exact, what):
    if exact:
        want = oracle.round_bf16(t) if out_bf16 else t
        P.assert_exact(got, want, what)
        return
    tol = P.BOUND * m + 2.0 ** -21 * (np.abs(t) + b) + 2.0 ** -126
    if out_bf16:
        tol = tol + 2.0 ** -8 * np.abs(t)
    err = np.abs(got - t)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} outside (worst {np.nanmax(err / tol):.3g}); first {np.argwhere(bad)[:3].tolist()}"


def _bf16_prob(M, N, K, colmajor, exact, seed):
    return inputs.bf16_problem(M, N, K, dist="integer" if exact else "normal", b_colmajor=colmajor, seed=seed)


SMALL = [(300, 260, 200, False), (129, 257, 96, True)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}_{'nt' if s[3] else 'nn'}")
@pytest.mark.parametrize("out_bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("which", ["rcb", "c", "b", ""])
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_fused_generic_kernel(shape, out_bf16, which, exact):
    M, N, K, colmajor = shape
    prob = _bf16_prob(M, N, K, colmajor, exact, seed=61)
    vecs = _vectors(M, N, exact, 62, which)
    P.note(f"fused generic {M}x{N}x{K} {'NT' if colmajor else 'NN'} out {'bf16' if out_bf16 else 'f32'} {which}")
    got = _run("bf16", prob, out_bf16, vecs)
    t, m, b = _reference("bf16", prob, vecs)
    _compare(got, t, m, b, out_bf16, exact, prob.name)


# (M, N, K, b_colmajor): 256 x 256 direct-load tiles with partial tiles and a
# partial last k-tile, the register-load kernel on 2-byte aligned rows with
# 192-column tiles, and the small-M kernel; every output against the oracle.
# Cases of one shape and distribution run in a row so that they share one
# oracle product.
BIG = [(4096 + 77, 4096 + 133, 520, True), (4096 + 77, 4096 + 8, 520, False), (4001, 3003, 2050, False),
       (16, 4096, 776, False)]
OUTS = [False, True]
BIG_CASES = [(shape, exact, out) for shape in BIG for exact in (True, False) for out in OUTS]


@pytest.mark.parametrize("case", BIG_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}_{'nt' if c[0][3] else 'nn'}"
                         f"_{'integer' if c[1] else 'normal'}_{'bf16' if c[2] else 'f32'}")
def test_fused_fast_kernels(case):
    (M, N, K, colmajor), exact, out_bf16 = case
    prob = _problem("bf16", M, N, K, colmajor, exact, 63)
    vecs = _vectors(M, N, exact, 64, "rcb")
    P.note(f"fused big {M}x{N}x{K} {'NT' if colmajor else 'NN'} out {'bf16' if out_bf16 else 'f32'}")
    got = _run("bf16", prob, out_bf16, vecs)
    t, m, b = _reference("bf16", prob, vecs)
    _compare(got, t, m, b, out_bf16, exact, prob.name)


# MX: the scale ring (K a multiple of 512), the 64-code k-tile pipeline (K =
# 64 mod 128) and the generic kernel; every output against the oracle.
MX = [(4096 + 40, 4096 + 8, 1024), (4096 + 40, 4096 + 8, 192), (300, 200, 96)]
MX_CASES = [(shape, out) for shape in MX for out in OUTS]


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "x".join(map(str, c[0])) + ("_bf16" if c[1] else "_f32"))
def test_fused_mx(case):
    (M, N, K), out_bf16 = case
    prob = _problem("mx", M, N, K, False, True, 66)
    vecs = _vectors(M, N, True, 67, "rcb")
    P.note(f"fused mx {M}x{N}x{K} out {'bf16' if out_bf16 else 'f32'}")
    got = _run("mx", prob, out_bf16, vecs)
    t, m, b = _reference("mx", prob, vecs)
    _compare(got, t, m, b, out_bf16, True, prob.name)


@pytest.mark.parametrize("out_bf16", [False, True], ids=["f32", "bf16"])
def test_fused_k_zero(out_bf16):
    M, N = 33, 70
    prob = _bf16_prob(M, N, 0, False, True, seed=69)
    vecs = _vectors(M, N, False, 70, "rcb")
    P.note(f"fused K=0 out {'bf16' if out_bf16 else 'f32'}")
    got = _run("bf16", prob, out_bf16, vecs)
    want = np.broadcast_to(vecs[2].astype(np.float64)[None, :], (M, N))
    if out_bf16:
        want = oracle.round_bf16(want)
    P.assert_exact(got, want, "K == 0")
