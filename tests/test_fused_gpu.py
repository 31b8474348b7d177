"""GPU parity of the fused epilogue (gemm_bf16_fused, gemm_mxfp8_fused)
through the C ABI, on shapes that reach every kernel: the generic tiles, the
256 x 256 direct-load kernel (NT, NN, MX with the scale ring), the
register-load kernel (2-byte aligned rows, 192-column tiles) and the small-M
kernel, plus K == 0.

Reference: the oracle's exact product with the epilogue applied in binary64
(oracle.epilogue), rounded by oracle.round_bf16 / oracle.round_e4m3 where
that is the output type.  Tolerance for floating point:
    |C - t| <= 1e-3 * |rs cs| sum|a||b|  +  2^-21 (|t| + |bias|)   (fp32 out)
and, for bf16 output, additionally half a bf16 unit of t (2^-8 |t|); for
E4M3 output, C is compared with t clamped to +-448 (the saturation) and the
tolerance adds half an E4M3 unit (2^-4 |t|, and 2^-10 below the normal
range).  Integer operands with power-of-two scales and integer biases keep
every step exact, so those cases must match bit for bit (the rounding of the
exact t)."""
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


OUT_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
OUT_TYPE = {"f32": dg.GEMM_OUT_F32, "bf16": dg.GEMM_OUT_BF16, "e4m3": dg.GEMM_OUT_E4M3}


def _run(kind, prob, out, vecs, ldc_pad=3):
    """out: "f32", "bf16" or "e4m3"."""
    M, N, K = prob.M, prob.N, prob.K
    rs, cs, bias = (_dev(v) for v in vecs)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    ldc = N + ldc_pad
    Cst = torch.full((M, ldc), -7.0, dtype=OUT_DTYPE[out], device=DEV)
    out_type = OUT_TYPE[out]
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


def _round(t, out):
    return oracle.round_bf16(t) if out == "bf16" else oracle.round_e4m3(t) if out == "e4m3" else t


def _compare(got, t, m, b, out, exact, what):
    if exact:
        P.assert_exact(got, _round(t, out), what)
        return
    tol = P.BOUND * m + 2.0 ** -21 * (np.abs(t) + b) + 2.0 ** -126
    if out == "bf16":
        tol = tol + 2.0 ** -8 * np.abs(t)
    if out == "e4m3":
        t = np.clip(t, -448.0, 448.0)
        tol = tol + 2.0 ** -4 * np.abs(t) + 2.0 ** -10
    err = np.abs(got - t)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} outside (worst {np.nanmax(err / tol):.3g}); first {np.argwhere(bad)[:3].tolist()}"


def _bf16_prob(M, N, K, colmajor, exact, seed):
    return inputs.bf16_problem(M, N, K, dist="integer" if exact else "normal", b_colmajor=colmajor, seed=seed)


SMALL = [(300, 260, 200, False), (129, 257, 96, True)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}_{'nt' if s[3] else 'nn'}")
@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("which", ["rcb", "c", "b", ""])
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_fused_generic_kernel(shape, out, which, exact):
    M, N, K, colmajor = shape
    prob = _bf16_prob(M, N, K, colmajor, exact, seed=61)
    vecs = _vectors(M, N, exact, 62, which)
    P.note(f"fused generic {M}x{N}x{K} {'NT' if colmajor else 'NN'} out {out} {which}")
    got = _run("bf16", prob, out, vecs)
    t, m, b = _reference("bf16", prob, vecs)
    _compare(got, t, m, b, out, exact, prob.name)


# (M, N, K, b_colmajor): 256 x 256 direct-load tiles with partial tiles and a
# partial last k-tile (and with K = 40, only that), the register-load kernel on
# 2-byte aligned rows with 192-column tiles, and the small-M kernel; every
# output against the oracle.
# Cases of one shape and distribution run in a row so that they share one
# oracle product.
BIG = [(4096 + 77, 4096 + 133, 520, True), (4096 + 77, 4096 + 8, 520, False), (4001, 3003, 2050, False),
       (16, 4096, 776, False), (4096 + 77, 4096 + 136, 40, True)]
OUTS = ["f32", "bf16", "e4m3"]
BIG_CASES = [(shape, exact, out) for shape in BIG for exact in (True, False) for out in OUTS]


@pytest.mark.parametrize("case", BIG_CASES, ids=lambda c: f"{c[0][0]}x{c[0][1]}x{c[0][2]}_{'nt' if c[0][3] else 'nn'}"
                         f"_{'integer' if c[1] else 'normal'}_{c[2]}")
def test_fused_fast_kernels(case):
    (M, N, K, colmajor), exact, out = case
    prob = _problem("bf16", M, N, K, colmajor, exact, 63)
    vecs = _vectors(M, N, exact, 64, "rcb")
    P.note(f"fused big {M}x{N}x{K} {'NT' if colmajor else 'NN'} out {out}")
    got = _run("bf16", prob, out, vecs)
    t, m, b = _reference("bf16", prob, vecs)
    _compare(got, t, m, b, out, exact, prob.name)


# MX: the scale ring (K a multiple of 512), the 64-code k-tile pipeline (K =
# 64 mod 128) and the generic kernel; every output against the oracle.
MX = [(4096 + 40, 4096 + 8, 1024), (4096 + 40, 4096 + 8, 192), (300, 200, 96)]
MX_CASES = [(shape, out) for shape in MX for out in OUTS]


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "x".join(map(str, c[0])) + "_" + c[1])
def test_fused_mx(case):
    (M, N, K), out = case
    prob = _problem("mx", M, N, K, False, True, 66)
    vecs = _vectors(M, N, True, 67, "rcb")
    P.note(f"fused mx {M}x{N}x{K} out {out}")
    got = _run("mx", prob, out, vecs)
    t, m, b = _reference("mx", prob, vecs)
    _compare(got, t, m, b, out, True, prob.name)


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
def test_fused_k_zero(out):
    M, N = 33, 70
    prob = _bf16_prob(M, N, 0, False, True, seed=69)
    vecs = _vectors(M, N, False, 70, "rcb")
    P.note(f"fused K=0 out {out}")
    got = _run("bf16", prob, out, vecs)
    want = np.broadcast_to(vecs[2].astype(np.float64)[None, :], (M, N))
    P.assert_exact(got, _round(want, out), "K == 0")


def _e4m3_probe_values(n):
    """n float32 values that exercise the E4M3 rounding: every tie between
    neighbouring E4M3 values and the values just beside it, both signs, the
    saturation region (448 .. 464 .. inf), subnormals, signed zeros, NaN, and
    random values filling the rest."""
    codes = torch.tensor([c for c in range(128) if c != 0x7F], dtype=torch.uint8)
    vals = np.unique(codes.view(torch.float8_e4m3fn).double().numpy())
    mids = (vals[1:] + vals[:-1]) / 2
    v = np.concatenate([vals, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                        [448.5, 463.9, 464.0, 464.1, 479.0, 480.0, 1e6, 3e38, np.inf, 2.0 ** -10, 2.0 ** -12]])
    v = np.concatenate([v, -v, [0.0, -0.0, np.nan]])
    rest = np.random.default_rng(71).standard_normal(max(0, n - v.size)) * 100
    return np.concatenate([v, rest])[:n].astype(np.float32)


# (kind, M, N, K, b_colmajor): the kernel each shape reaches
E4M3_KERNELS = [("generic", 300, 1100, 64, False), ("fast_nt", 4096, 4096, 64, True),
                ("fast_nn", 4096, 4096, 64, False), ("small_m", 16, 4096, 64, False),
                ("reg", 4001, 3003, 66, False), ("k_zero", 40, 1100, 0, False)]


@pytest.mark.parametrize("case", E4M3_KERNELS, ids=lambda c: c[0])
def test_e4m3_rounding_in_every_kernel(case):
    """With B = 0 every accumulator is +0, so t = 0 + bias[j] (bias itself,
    except that -0 becomes +0) and C[i, j] is its E4M3 rounding: each
    kernel's conversion checked against oracle.round_e4m3 on ties,
    saturation, subnormals, zeros and NaN, bit for bit (sign of zero
    included)."""
    name, M, N, K, colmajor = case
    bias = _e4m3_probe_values(N)
    prob = _bf16_prob(M, N, K, colmajor, True, seed=72)
    prob.B.zero_()
    if name == "reg":
        # odd leading dimensions: the register-load kernel
        P.note(f"e4m3 rounding {name} {M}x{N}x{K}")
        A, B = prob.A.to(DEV), prob.B.to(DEV)
        Ast = torch.zeros((M, K + 1), dtype=torch.bfloat16, device=DEV)
        Ast[:, :K] = A
        Bst = torch.zeros((K, N + 1), dtype=torch.bfloat16, device=DEV)
        Cst = torch.full((M, N + 5), -7.0, dtype=torch.float8_e4m3fn, device=DEV)
        bd = torch.from_numpy(bias).to(DEV)
        rc = dg.gemm_bf16_fused(M, N, K, Ast.data_ptr(), K + 1, Bst.data_ptr(), N + 1, 0, Cst.data_ptr(), N + 5,
                                dg.GEMM_OUT_E4M3, 0, 0, bd.data_ptr(), P.stream())
        assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
        torch.cuda.synchronize()
        got8 = Cst[:, :N].contiguous()
    else:
        P.note(f"e4m3 rounding {name} {M}x{N}x{K}")
        got = _run("bf16", prob, "e4m3", (None, None, bias), ldc_pad=5)
        got8 = torch.from_numpy(got.astype(np.float32)).to(torch.float8_e4m3fn)
    want = oracle.round_e4m3(0.0 + bias.astype(np.float64))
    gotv = got8.float().cpu().numpy().astype(np.float64) if got8.is_cuda else got8.double().numpy()
    for i in (0, M // 2, M - 1):
        row = gotv[i]
        same = (row == want) | (np.isnan(row) & np.isnan(want))
        assert same.all(), (name, bias[~same][:6], row[~same][:6], want[~same][:6])
        assert np.array_equal(np.signbit(row[row == 0]), np.signbit(want[row == 0])), name
    assert np.array_equal(np.isnan(gotv), np.broadcast_to(np.isnan(want), gotv.shape)), name
    assert (gotv[~np.isnan(gotv)] == np.broadcast_to(want, gotv.shape)[~np.isnan(gotv)]).all(), name
