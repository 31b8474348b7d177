"""GPU parity of split-K (gemm_bf16_splitk) through the C ABI.

The K extent is cut into ranges whose fp32 partial products land in the
caller's workspace and are added in range order by a second kernel.  Cases
reach both partial kernels: the 256 x 256 direct-load kernel (NT and NN, with
partial tiles, a partial last k-tile inside the last range, explicit and
planned range counts) and the small-M kernel (planned and explicit counts, a
K that ends inside a 32-row step), plus the fused epilogue after the
reduction, an unsplit fallback that must leave the workspace alone, a
workspace that is too small, and determinism.

Reference: the oracle's exact product (binary64).  Tolerance: the acceptance
bound |C - exact| <= 1e-3 sum_k |a||b|; every range is summed in fp32 and the
ranges are added in fp32, so the total rounding stays within
gamma_(K + splits) sum|a||b|, below the bound for these K.  Integer operands
keep every partial sum below 2^24 and must match bit for bit."""
import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
import oracle
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _plan(M, N, K, colmajor, splits):
    rc, used, nbytes = dg.gemm_bf16_splitk_plan(M, N, K, colmajor, splits)
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    return used, nbytes


OUT_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
OUT_TYPE = {"f32": dg.GEMM_OUT_F32, "bf16": dg.GEMM_OUT_BF16, "e4m3": dg.GEMM_OUT_E4M3}


def _run(prob, splits, *, ldc_pad=3, out="f32", vecs=(None, None, None), ws=None, ws_fill=float("nan")):
    """gemm_bf16_splitk on the problem's operands; returns (C as float64,
    splits the plan uses, workspace tensor)."""
    M, N, K = prob.M, prob.N, prob.K
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    ldb = K if prob.b_colmajor else N
    used, nbytes = _plan(M, N, K, prob.b_colmajor, splits)
    if ws is None:
        # contents on entry must not matter: start from NaN
        ws = torch.full((max(nbytes, 16) // 4,), ws_fill, dtype=torch.float32, device=DEV)
    ldc = N + ldc_pad
    Cst = torch.full((M, ldc), -7.0, dtype=OUT_DTYPE[out], device=DEV)
    rs, cs, bias = (None if v is None else torch.from_numpy(v).to(DEV) for v in vecs)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    out_type = OUT_TYPE[out]
    rc = dg.gemm_bf16_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor, Cst.data_ptr(), ldc,
                             out_type, ptr(rs), ptr(cs), ptr(bias), splits, ws.data_ptr(), ws.numel() * 4,
                             P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    C = Cst.float().cpu().numpy()
    assert (C[:, N:] == -7.0).all(), "C written outside M x N"
    return np.ascontiguousarray(C[:, :N]).astype(np.float64), used, ws


def _check(prob, got, exact, sample=None):
    Ab, Bb = P.bits16(prob.A), P.bits16(prob.B)
    if sample is None:
        want, mag = P.oracle_bf16(Ab, Bb, prob.b_colmajor)
        g = got
    else:
        rows, cols = sample
        want, mag = P.oracle_bf16_at(Ab, Bb, prob.b_colmajor, rows, cols)
        g = got[rows, cols]
    if exact:
        P.assert_exact(g, want, prob.name)
    else:
        P.assert_within_bound(g, want, mag, prob.name)


def _prob(M, N, K, colmajor, exact, seed):
    return inputs.bf16_problem(M, N, K, dist="integer" if exact else "normal", b_colmajor=colmajor, seed=seed)


# (M, N, K, b_colmajor, splits): 256 x 256 partial kernel.  K = 4104 and 3000 end
# inside a k-tile (the last range carries the partial k-tile); 0 = the plan.
# M or N at most 32 takes the 32 x 32 MFMA instance, the others the 16 x 16 one.
FAST = [(1000, 777, 4104, True, 0), (1000, 777, 4104, True, 3), (513, 1032, 3000, False, 0),
        (513, 1032, 3000, False, 5), (300, 520, 1024, True, 2), (256, 256, 640, False, 7),
        (24, 1000, 4104, True, 3), (700, 24, 3000, False, 4), (33, 1000, 4104, True, 3)]


@pytest.mark.parametrize("case", FAST, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{'nt' if c[3] else 'nn'}_s{c[4]}")
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_splitk_fast_kernel(case, exact):
    M, N, K, colmajor, splits = case
    prob = _prob(M, N, K, colmajor, exact, seed=81)
    P.note(f"splitk fast {prob.name} splits={splits}")
    got, used, _ = _run(prob, splits)
    assert used > 1, "the plan should split this shape"
    _check(prob, got, exact)


# small-M partial kernel (row-major B, M <= 64, N >= 2048): 64 column
# blocks (the plan splits), K ending inside a 32-row step, 48 rows; with
# M <= 16 and enough columns the plan takes 128-column strips (16 x 8192 x
# 8192: 4 ranges; N = 8232 leaves a partial strip, 3 ranges; K = 4104 ends
# inside a step; M = 1)
SMALL = [(16, 2048, 8192, 0), (16, 2048, 1000, 3), (48, 4096, 2056, 4), (1, 2048, 4096, 0), (16, 8192, 8192, 2),
         (16, 8192, 8192, 0), (7, 8192 + 40, 4104, 0), (1, 8192, 8192, 4)]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}")
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_splitk_small_m(case, exact):
    M, N, K, splits = case
    prob = _prob(M, N, K, False, exact, seed=82)
    P.note(f"splitk small {prob.name} splits={splits}")
    got, used, _ = _run(prob, splits)
    assert used > 1
    _check(prob, got, exact)


def test_splitk_long_k_sampled():
    """2048 x 2048 x 16384 NT: 64 tiles, the plan fills the GPU with K ranges."""
    prob = _prob(2048, 2048, 16384, True, False, seed=84)
    P.note(f"splitk sampled {prob.name}")
    got, used, _ = _run(prob, 0, ldc_pad=0)
    assert used >= 2
    P.check_lines_bf16(got, P.bits16(prob.A), P.bits16(prob.B), True, P.band_lines(2048, 256, 85),
                       P.band_lines(2048, 256, 86), prob.name)


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("shape", [(700, 600, 2048), (24, 600, 2048)], ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}")
def test_splitk_fused_epilogue(out, shape):
    """The epilogue applied once, after the reduction, on the 16 x 16 and (M <= 32) the 32 x 32 partial instance."""
    M, N, K = shape
    prob = _prob(M, N, K, True, True, seed=86)
    g = np.random.default_rng(87)
    rs = np.exp2(g.integers(-2, 3, size=M)).astype(np.float32)
    cs = np.exp2(g.integers(-2, 3, size=N)).astype(np.float32)
    bias = g.integers(-8, 9, size=N).astype(np.float32)
    P.note(f"splitk fused {prob.name} out {out}")
    got, used, _ = _run(prob, 4, out=out, vecs=(rs, cs, bias))
    assert used == 4
    acc, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), True)
    t, _ = oracle.epilogue(acc, mag, rs, cs, bias)
    want = oracle.round_bf16(t) if out == "bf16" else oracle.round_e4m3(t) if out == "e4m3" else t
    P.assert_exact(got, want, prob.name)


def test_splitk_unsplit_fallback_leaves_workspace():
    """Operands that are not 16-byte aligned run unsplit; the workspace is not touched."""
    M, N, K = 200, 300, 1000
    prob = _prob(M, N, K, True, True, seed=88)
    Ast = torch.zeros(M * K + 8, dtype=torch.bfloat16, device=DEV)
    Ast[1:1 + M * K] = prob.A.reshape(-1).to(DEV)
    B = prob.B.to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = torch.full((4 * M * N,), 12345.0, dtype=torch.float32, device=DEV)
    P.note("splitk fallback (A offset by one element)")
    rc = dg.gemm_bf16_splitk(M, N, K, Ast.data_ptr() + 2, K, B.data_ptr(), K, 1, C.data_ptr(), N, dg.GEMM_OUT_F32,
                             0, 0, 0, 4, ws.data_ptr(), ws.numel() * 4, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    assert (ws == 12345.0).all().item(), "an unsplit call wrote the workspace"
    want, _ = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), True)
    P.assert_exact(C.cpu().numpy().astype(np.float64), want, "fallback")


def test_splitk_rejects_short_workspace():
    M, N, K = 512, 512, 4096
    prob = _prob(M, N, K, True, True, seed=89)
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    used, nbytes = _plan(M, N, K, True, 4)
    assert used == 4 and nbytes == 4 * M * N * 4
    C = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    P.note("splitk short workspace")
    args = (M, N, K, A.data_ptr(), K, B.data_ptr(), K, 1, C.data_ptr(), N, dg.GEMM_OUT_F32, 0, 0, 0, 4)
    assert dg.gemm_bf16_splitk(*args, ws.data_ptr(), nbytes - 4, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk(*args, 0, nbytes, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk(*args, ws.data_ptr() + 4, nbytes - 4, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (C == -7.0).all().item(), "C changed by a rejected call"


def test_splitk_deterministic():
    prob = _prob(1000, 777, 4104, True, False, seed=90)
    P.note(f"splitk determinism {prob.name}")
    a, _, _ = _run(prob, 6)
    b, _, _ = _run(prob, 6, ws_fill=0.0)
    assert np.array_equal(a, b)


def test_splitk_tensor_helper():
    prob = _prob(16, 2048, 4096, False, True, seed=91)
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    P.note("splitk tensor helper")
    C = dg.bf16_splitk(A, B)
    torch.cuda.synchronize()
    want, _ = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), False)
    P.assert_exact(C.cpu().numpy().astype(np.float64), want, "bf16_splitk")


@pytest.mark.parametrize("name,ranges", [("longk1024x1024x32768_nt", 16), ("skinny16x8192x8192_nt", 8),
                                        ("skinny16x8192x8192_nn_splitk", 4)])
def test_splitk_bench_workloads(name, ranges):
    """The split-K workloads at full size, in the launch configuration the
    benchmark times (the library's plan, ldc = N), on every output.  With
    K = 32768 the unsplit fp32 sum would not be inside the 1e-3 bound in
    general; each of the 16 ranges sums 2048 products (gamma < 1.3e-4) and the
    16 partials add at most gamma_16 more, so the bound holds."""
    prob = inputs.workload(name, seed=0)
    P.note(f"splitk workload {name}")
    got, used, _ = _run(prob, 0, ldc_pad=0)
    assert used == ranges
    _check(prob, got, False)


# Stream-K style plans: products that fill more than one round of the 256 x
# 256 kernel with a last round at most half full.  The whole rounds store
# straight to C with the arithmetic of the plain entry points; only the last
# round's tiles are split over K (compact partial tiles, tile-wise reduction).
# 4173 x 4360: 17 x 18 = 306 tiles, 50 left over in 4 ranges, the last range
# with a partial k-tile; the left-over tiles include the bottom and right
# edges.  4352 x 4352: 289 tiles, 33 left over.
STREAMK = [(4096 + 77, 4096 + 264, 2056, False, 4), (4352, 4352, 1024, True, 2), (4352, 4352, 4096, True, 7)]


@pytest.mark.parametrize("case", STREAMK, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{'nt' if c[3] else 'nn'}")
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_splitk_stream_k_style(case, exact):
    M, N, K, colmajor, ranges = case
    prob = _prob(M, N, K, colmajor, exact, seed=98)
    P.note(f"splitk stream-K style {prob.name} {'NT' if colmajor else 'NN'}")
    got, used, _ = _run(prob, 0, ldc_pad=0)
    assert used == ranges
    plain = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), colmajor).cpu().numpy().astype(np.float64)
    if exact:
        assert np.array_equal(got, plain)
    else:
        # whole tiles are computed as by the plain call, bit for bit; at most
        # the left-over tiles (under half a round of 256 x 256) may differ
        differ = np.count_nonzero(got != plain)
        assert differ <= 128 * 256 * 256, differ
    if K <= 2056:
        _check(prob, got, exact)
    else:
        # every tile row and column band, and the left-over tiles' edges
        P.check_lines_bf16(got, P.bits16(prob.A), P.bits16(prob.B), colmajor, P.band_lines(M, 256, 99),
                           P.band_lines(N, 256, 100), prob.name, exact)


@pytest.mark.parametrize("case", [(512, 512, 8193, 8200, 8200, True), (16, 2049, 8192, 8192, 2056, False)],
                         ids=["padded_odd_k_nt", "small_m_odd_n_nn"])
def test_splitk_helper_sizes_workspace_for_padded_views(case):
    """bf16_splitk without a workspace sizes it with gemm_bf16_splitk_workspace,
    which plans with the real leading dimensions: padded views whose extent is
    not a multiple of 8 elements (but whose leading dimension is) split."""
    M, N, K, lda, ldb, colmajor = case
    prob = _prob(M, N, K, colmajor, True, seed=101)
    Ast = torch.zeros((M, lda), dtype=torch.bfloat16, device=DEV)
    Ast[:, :K] = prob.A.to(DEV)
    rows_b, cols_b = prob.B.shape
    Bst = torch.zeros((rows_b, ldb), dtype=torch.bfloat16, device=DEV)
    Bst[:, :cols_b] = prob.B.to(DEV)
    A = Ast[:, :K]
    B = Bst[:, :cols_b].t() if colmajor else Bst[:, :cols_b]
    rc, used, nbytes = dg.gemm_bf16_splitk_workspace(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, colmajor,
                                                     0x10000, N, dg.GEMM_OUT_F32, None, None, None, 0, 0)
    assert rc == dg.GEMM_OK and used > 1 and nbytes == used * M * N * 4
    P.note(f"splitk helper padded {M}x{N}x{K} lda {lda} ldb {ldb}")
    C = dg.bf16_splitk(A, B, b_colmajor=None)
    torch.cuda.synchronize()
    want, _ = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), colmajor)
    P.assert_exact(C.cpu().numpy().astype(np.float64), want, prob.name)


# ---------------------------------------------------------------- MX split-K

def _mx_run(prob, splits, *, out="f32", vecs=(None, None, None), scale_off=0, ws_fill=float("nan"), ws=None):
    """gemm_mxfp8_splitk on the problem; returns (C as float64, ranges used, workspace)."""
    M, N, K = prob.M, prob.N, prob.K
    A, B = prob.A.to(DEV), prob.B.to(DEV)

    def at(S):  # scale codes starting scale_off bytes past a 256-byte boundary
        buf = torch.zeros(S.numel() + 256, dtype=torch.uint8, device=DEV)
        v = buf[scale_off:scale_off + S.numel()].view(S.shape)
        v.copy_(S.to(DEV))
        return v
    SA, SB = at(prob.SA), at(prob.SB)
    ldc = N + 3
    Cst = torch.full((M, ldc), -7.0, dtype=OUT_DTYPE[out], device=DEV)
    rs, cs, bias = (None if v is None else torch.from_numpy(v).to(DEV) for v in vecs)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    rc, used, nbytes = dg.gemm_mxfp8_splitk_workspace(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(),
                                                      SB.data_ptr(), Cst.data_ptr(), ldc, OUT_TYPE[out], ptr(rs),
                                                      ptr(cs), ptr(bias), splits)
    assert rc == dg.GEMM_OK
    if ws is None:
        ws = torch.full((max(nbytes, 16) // 4,), ws_fill, dtype=torch.float32, device=DEV)
    rc = dg.gemm_mxfp8_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(),
                              Cst.data_ptr(), ldc, OUT_TYPE[out], ptr(rs), ptr(cs), ptr(bias), splits, ws.data_ptr(),
                              ws.numel() * 4, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    C = Cst.float().cpu().numpy()
    assert (C[:, N:] == -7.0).all(), "C written outside M x N"
    return np.ascontiguousarray(C[:, :N]).astype(np.float64), used, ws


# (M, N, K, splits, ranges): 16 tiles with the plan (8 ranges of 1024; 4
# ranges of 1024), asked counts whose last range is shorter (3584 in ranges
# of 2048 and 1536) or with 2 tiles in N, partial tiles in M and N
MX_SPLIT = [(1024, 1024, 8192, 0, 8), (1000, 777, 4096, 0, 4), (512, 520, 3584, 2, 2), (300, 1100, 2048, 2, 2)]


@pytest.mark.parametrize("case", MX_SPLIT, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_s{c[3]}")
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_mx_splitk(case, exact):
    M, N, K, splits, ranges = case
    prob = inputs.mx_problem(M, N, K, dist="integer" if exact else "normal", seed=102)
    P.note(f"mx splitk {M}x{N}x{K} splits={splits}")
    got, used, _ = _mx_run(prob, splits)
    assert used == ranges
    want, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    if exact:
        P.assert_exact(got, want, prob.name)
    P.assert_within_bound(got, want, mag, prob.name)
    # the unsplit entry point gives the same result within the bound (equal
    # for integer operands)
    C1 = P.run_mx(prob.A.to(DEV), prob.B.to(DEV), prob.SA.to(DEV), prob.SB.to(DEV)).cpu().numpy()
    if exact:
        assert np.array_equal(C1.astype(np.float64), got)


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
def test_mx_splitk_fused_epilogue(out):
    M, N, K = 700, 600, 4096
    prob = inputs.mx_problem(M, N, K, dist="integer", seed=103)
    g = np.random.default_rng(104)
    rs = np.exp2(g.integers(-2, 3, size=M)).astype(np.float32)
    cs = np.exp2(g.integers(-2, 3, size=N)).astype(np.float32)
    bias = g.integers(-8, 9, size=N).astype(np.float32)
    P.note(f"mx splitk fused out {out}")
    got, used, _ = _mx_run(prob, 4, out=out, vecs=(rs, cs, bias))
    assert used == 4
    acc, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    t, _ = oracle.epilogue(acc, mag, rs, cs, bias)
    want = oracle.round_bf16(t) if out == "bf16" else oracle.round_e4m3(t) if out == "e4m3" else t
    P.assert_exact(got, want, prob.name)


def test_mx_splitk_unsplit_fallback_and_errors():
    prob = inputs.mx_problem(1024, 1024, 8192, dist="integer", seed=105)
    P.note("mx splitk fallback (scales 4 bytes off 16-byte alignment)")
    ws = torch.full((64,), 12345.0, dtype=torch.float32, device=DEV)
    got, used, ws = _mx_run(prob, 4, scale_off=4, ws=ws)
    assert used == 1 and (ws == 12345.0).all().item()
    want, _ = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    P.assert_exact(got, want, prob.name)
    # a short or misaligned workspace is refused with C untouched
    M, N, K = prob.M, prob.N, prob.K
    A, B, SA, SB = (x.to(DEV) for x in (prob.A, prob.B, prob.SA, prob.SB))
    C = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    rc, used, nbytes = dg.gemm_mxfp8_splitk_workspace(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(),
                                                      SB.data_ptr(), C.data_ptr(), N, dg.GEMM_OUT_F32, None, None,
                                                      None, 0)
    assert used == 8 and nbytes == 8 * M * N * 4
    w = torch.empty(nbytes // 4, dtype=torch.float32, device=DEV)
    args = (M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(), C.data_ptr(), N,
            dg.GEMM_OUT_F32, None, None, None, 0)
    assert dg.gemm_mxfp8_splitk(*args, w.data_ptr(), nbytes - 4, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_mxfp8_splitk(*args, w.data_ptr() + 4, nbytes - 4, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_mxfp8_splitk(*args[:-1], -1, w.data_ptr(), nbytes, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (C == -7.0).all().item()


def test_mx_splitk_deterministic():
    prob = inputs.mx_problem(1000, 777, 4096, dist="normal", seed=106)
    P.note("mx splitk determinism")
    a, _, _ = _mx_run(prob, 0)
    b, _, _ = _mx_run(prob, 0, ws_fill=0.0)
    assert np.array_equal(a, b)


def test_mx_splitk_bench_workload():
    """The MX split-K workload at full size in the benchmark's launch
    configuration (the plan: 16 ranges of 2048, ldc = N): whole rows and
    columns over every tile band against the oracle.  Each range sums 2048
    block-scaled products in fp32 and 16 partials are added, so the 1e-3
    bound holds although K = 32768."""
    prob = inputs.workload("mx1024x1024x32768_splitk", seed=0)
    M, N, K = prob.M, prob.N, prob.K
    A, B, SA, SB = (x.to(DEV) for x in (prob.A, prob.B, prob.SA, prob.SB))
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    rc, used, nbytes = dg.gemm_mxfp8_splitk_workspace(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(),
                                                      SB.data_ptr(), C.data_ptr(), N, dg.GEMM_OUT_F32, None, None,
                                                      None, 0)
    assert rc == dg.GEMM_OK and used == 16
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    P.note("mx splitk workload mx1024x1024x32768_splitk")
    rc = dg.gemm_mxfp8_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(), C.data_ptr(),
                              N, dg.GEMM_OUT_F32, None, None, None, 0, ws.data_ptr(), nbytes, P.stream())
    assert rc == dg.GEMM_OK
    torch.cuda.synchronize()
    P.check_lines_mx(C.cpu().numpy(), prob.A, prob.B, prob.SA, prob.SB, P.band_lines(M, 256, 107),
                     P.band_lines(N, 256, 108), prob.name)
