"""GPU parity: the HIP path (called through the C ABI) against the CPU oracle
on the same seeded inputs.  Needs an MI355X and the built libgemm.so."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

DEV = "cuda:0"


def _bf16_case(M, N, K, colmajor, dist, seed):
    return inputs.bf16_problem(M, N, K, dist=dist, b_colmajor=colmajor, seed=seed)


def _check_full_bf16(prob, exact=False):
    P.note(f"bf16 {'NT' if prob.b_colmajor else 'NN'} {prob.M}x{prob.N}x{prob.K} {prob.name}")
    C = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), prob.b_colmajor).cpu().numpy()
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), prob.b_colmajor)
    if exact:
        P.assert_exact(C, want, prob.name)
    P.assert_within_bound(C, want, mag, prob.name)


# ---------------------------------------------------------------- small shapes

def test_single_tile_config():
    """M=N=K=128, row-major A and B, uniform[-1,1] bf16 from seed 0."""
    _check_full_bf16(inputs.workload("tile128_nn", seed=0))


SHAPES = [(1, 1, 1), (256, 256, 128), (300, 260, 200), (513, 257, 129), (33, 65, 17),
          (255, 257, 64), (257, 255, 65), (64, 640, 192), (640, 64, 63), (1000, 1000, 333)]


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_integer_operands_bit_exact(shape, colmajor):
    M, N, K = shape
    _check_full_bf16(_bf16_case(M, N, K, colmajor, "integer", seed=7), exact=True)


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_normal_operands_within_bound(shape, colmajor):
    M, N, K = shape
    _check_full_bf16(_bf16_case(M, N, K, colmajor, "normal", seed=11))


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
def test_big_tile_path_with_tails(colmajor):
    """Large enough for the 256x256 tiles, with a ragged edge in every dimension."""
    _check_full_bf16(_bf16_case(2048 + 77, 2048 + 133, 513, colmajor, "normal", seed=3))


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
def test_misaligned_operands(colmajor):
    """Base pointers off 16-byte alignment and odd leading dimensions take the
    predicated load path; padding holds NaN and must never reach C."""
    M, N, K = 301, 283, 190
    g = inputs.generator(5)
    A = inputs.normal_bf16((M, K), g)
    B = inputs.normal_bf16((N, K) if colmajor else (K, N), g)
    lda = K + 3
    rows_b, cols_b = B.shape
    ldb = cols_b + 5
    nan = torch.tensor(float("nan")).to(torch.bfloat16)
    Ast = torch.full((M * lda + 1,), nan.item(), dtype=torch.bfloat16)
    Ast[1:].view(M, lda)[:, :K] = A
    Bst = torch.full((rows_b * ldb + 1,), nan.item(), dtype=torch.bfloat16)
    Bst[1:].view(rows_b, ldb)[:, :cols_b] = B
    Ad, Bd = Ast.to(DEV), Bst.to(DEV)
    ldc = N + 7
    Cst = torch.full((M * ldc,), -12345.0, dtype=torch.float32, device=DEV)
    P.note(f"misaligned {'NT' if colmajor else 'NN'} {M}x{N}x{K}")
    fn = dg.gemm_bf16_nt if colmajor else dg.gemm_bf16
    rc = fn(M, N, K, Ad.data_ptr() + 2, lda, Bd.data_ptr() + 2, ldb, Cst.data_ptr(), ldc,
            P.stream())
    assert rc == 0
    torch.cuda.synchronize()
    Cfull = Cst.view(M, ldc).cpu().numpy()
    assert (Cfull[:, N:] == -12345.0).all(), "C written outside M x N"
    want, mag = P.oracle_bf16(P.bits16(A), P.bits16(B), colmajor)
    P.assert_within_bound(Cfull[:, :N], want, mag, "misaligned")


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
def test_nan_padding_and_guard_band(colmajor):
    """Aligned padded operands (fast path) with NaN in the padding; C has a
    sentinel guard band that must stay untouched."""
    M, N, K = 520, 264, 200
    g = inputs.generator(6)
    A = inputs.normal_bf16((M, K), g)
    B = inputs.normal_bf16((N, K) if colmajor else (K, N), g)
    lda = K + 56  # multiple of 8 -> direct loads
    rows_b, cols_b = B.shape
    ldb = cols_b + 40
    Ast = torch.full((M, lda), float("nan"), dtype=torch.bfloat16)
    Ast[:, :K] = A
    Bst = torch.full((rows_b, ldb), float("nan"), dtype=torch.bfloat16)
    Bst[:, :cols_b] = B
    ldc = N + 9
    C = torch.full((M + 3, ldc), 777.0, dtype=torch.float32, device=DEV)
    P.note(f"guard {'NT' if colmajor else 'NN'} {M}x{N}x{K}")
    fn = dg.gemm_bf16_nt if colmajor else dg.gemm_bf16
    Ad, Bd = Ast.to(DEV), Bst.to(DEV)
    rc = fn(M, N, K, Ad.data_ptr(), lda, Bd.data_ptr(), ldb, C.data_ptr(), ldc, P.stream())
    assert rc == 0
    torch.cuda.synchronize()
    Ch = C.cpu().numpy()
    assert (Ch[:, N:] == 777.0).all() and (Ch[M:] == 777.0).all(), "guard band overwritten"
    want, mag = P.oracle_bf16(P.bits16(A), P.bits16(B), colmajor)
    P.assert_within_bound(Ch[:M, :N], want, mag, "guard")


@pytest.mark.parametrize("colmajor", [False, True], ids=["nn", "nt"])
def test_nan_and_inf_propagation(colmajor):
    M, N, K = 300, 300, 160
    prob = _bf16_case(M, N, K, colmajor, "normal", seed=8)
    A = prob.A.clone()
    B = prob.B.clone()
    A[17, 33] = float("nan")
    A[40, 5] = float("inf")
    if colmajor:
        B[9, 5] = 0.0  # column 9 of B meets the infinity with a zero
    else:
        B[5, 9] = 0.0
    P.note("nan/inf propagation")
    C = P.run_bf16(A.to(DEV), B.to(DEV), colmajor).cpu().numpy()
    want, mag = P.oracle_bf16(P.bits16(A), P.bits16(B), colmajor)
    assert np.isnan(C[17]).all() and np.isnan(C[40, 9])
    P.assert_within_bound(C, want, mag, "nan/inf")


def test_deterministic_repeats():
    prob = _bf16_case(1024, 1024, 1024, True, "normal", seed=9)
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    P.note("determinism 1024^3 NT x5")
    first = P.run_bf16(A, B, True).clone()
    for _ in range(4):
        assert torch.equal(P.run_bf16(A, B, True), first)


def test_k_zero_and_empty():
    P.note("K=0 zero fill, empty M/N")
    A = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((0, 7), dtype=torch.bfloat16, device=DEV)
    C = torch.full((5, 7), 3.0, device=DEV)
    rc = dg.gemm_bf16(5, 7, 0, 0, 1, 0, 7, C.data_ptr(), 7, P.stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert (C == 0).all()
    C2 = torch.full((4, 4), 3.0, device=DEV)
    assert dg.gemm_bf16(0, 4, 4, 0, 4, 0, 4, C2.data_ptr(), 4, P.stream()) == 0
    assert dg.gemm_bf16_nt(4, 0, 4, 0, 4, 0, 4, C2.data_ptr(), 4, P.stream()) == 0
    torch.cuda.synchronize()
    assert (C2 == 3.0).all()


def test_tensor_helper_layouts():
    """dg.bf16 picks NN or NT from the strides of B."""
    prob = _bf16_case(200, 300, 100, True, "normal", seed=12)
    A, Bt = prob.A.to(DEV), prob.B.to(DEV)
    P.note("tensor helper")
    c_nt = dg.bf16(A, Bt.t())
    c_nn = dg.bf16(A, Bt.t().contiguous())
    torch.cuda.synchronize()
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), True)
    P.assert_within_bound(c_nt.cpu().numpy(), want, mag, "helper NT")
    P.assert_within_bound(c_nn.cpu().numpy(), want, mag, "helper NN")


# ---------------------------------------------------------------- fast (256 x 256) path

# Shapes large enough for the 256 x 256 kernel (enough tiles for every CU),
# with partial tiles in M and N and a partial last k-tile; K = 40 and 24 are
# shorter than one k-tile (no pipelined k-tile, only the tail).
FAST_BF16 = [(4096 + 77, 4096 + 133, 513, True), (4096 + 77, 4096 + 8, 520, False),
             (4096 + 200, 4096 + 64, 1000, True), (4096, 4096, 256, False),
             (4096 + 77, 4096 + 136, 40, True), (4096 + 77, 4096 + 8, 24, False)]


@pytest.mark.parametrize("case", FAST_BF16, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{'nt' if c[3] else 'nn'}")
@pytest.mark.parametrize("dist", ["normal", "integer"])
def test_fast_path_bf16_tails(case, dist):
    """Every output of the 256 x 256 direct-load kernel against the oracle."""
    M, N, K, colmajor = case
    prob = _bf16_case(M, N, K, colmajor, dist, seed=31)
    P.note(f"fast path bf16 {'NT' if colmajor else 'NN'} {M}x{N}x{K} {dist}")
    C = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), colmajor).cpu().numpy()
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), colmajor)
    if dist == "integer":
        P.assert_exact(C, want, prob.name)
    P.assert_within_bound(C, want, mag, prob.name)


# 256 x 256 MX kernels, every output against the oracle: the scale ring (K a
# multiple of 512), the word-scale pipeline (K a multiple of 128), and the
# 64-code k-tile pipeline with 4 stages, taken when K is 64 mod 128 or when
# the scale arrays are only 2-byte aligned (scale_offset = 2).
FAST_MX = [(4096 + 40, 4096 + 200, 512, 0), (4096 + 40, 4096 + 8, 384, 0), (4096 + 40, 4096 + 8, 192, 0),
           (4096 + 40, 4096 + 72, 256, 2)]


def _mx_scales_at(S: torch.Tensor, offset: int) -> torch.Tensor:
    """A device copy of the scale codes starting `offset` bytes past a 256-byte
    boundary (the view keeps the storage alive)."""
    buf = torch.zeros(S.numel() + 256, dtype=torch.uint8, device=DEV)
    view = buf[offset:offset + S.numel()].view(S.shape)
    view.copy_(S.to(DEV))
    return view


@pytest.mark.parametrize("shape", FAST_MX, ids=lambda s: "x".join(map(str, s[:3])) + f"_soff{s[3]}")
@pytest.mark.parametrize("dist", ["normal", "integer"])
def test_fast_path_mx_tails(shape, dist):
    M, N, K, soff = shape
    prob = inputs.mx_problem(M, N, K, dist=dist, seed=32)
    P.note(f"fast path mx {M}x{N}x{K} scale offset {soff} {dist}")
    SA, SB = _mx_scales_at(prob.SA, soff), _mx_scales_at(prob.SB, soff)
    C = P.run_mx(prob.A.to(DEV), prob.B.to(DEV), SA, SB).cpu().numpy()
    want, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    if dist == "integer":
        P.assert_exact(C, want, prob.name)
    P.assert_within_bound(C, want, mag, prob.name)


# ---------------------------------------------------------------- 2-byte aligned rows

# (M, N, K, b_colmajor, lda pad, ldb pad, element offset of A and B): large
# enough for 256 x 256 tiles, with leading dimensions and base pointers that
# keep rows off 16-byte (and, for odd values, off 4-byte) alignment, so the
# register-load kernel runs; K tails of every kind (none, partial, K < 32).
REG_BF16 = [(3600 + 17, 3500 + 3, 333, False, 3, 1, 1), (3584 + 1, 3840 + 5, 1001, True, 1, 5, 1),
            (3584, 3584, 512, False, 1, 3, 0), (3600, 3600, 17, True, 2, 2, 3),
            (3520 + 9, 3520 + 31, 64 + 2, False, 0, 2, 2), (3600 + 1, 3600 + 5, 512, False, 1, 1, 1),
            # 192-column tiles (16 x 16 of them fill 256 CUs where 256-column
            # tiles would leave a quarter idle)
            (3900 + 1, 2900 + 3, 333, False, 3, 1, 1), (4000, 3000, 1001, True, 1, 5, 1),
            (3850, 2890, 17, True, 2, 2, 3), (4001, 3003, 512, False, 1, 1, 1),
            (4096, 3072, 64 + 2, False, 0, 2, 2)]


@pytest.mark.parametrize("case", REG_BF16, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}_{'nt' if c[3] else 'nn'}")
@pytest.mark.parametrize("dist", ["normal", "integer"])
def test_unaligned_rows_big_tiles(case, dist):
    M, N, K, colmajor, pa, pb, off = case
    prob = _bf16_case(M, N, K, colmajor, dist, seed=51)
    nan = float("nan")
    lda = K + pa
    rows_b, cols_b = prob.B.shape
    ldb = cols_b + pb
    # the padding and the elements around each operand hold NaN
    Ast = torch.full((M * lda + off + 8,), nan, dtype=torch.bfloat16)
    Ast[off:off + M * lda].view(M, lda)[:, :K] = prob.A
    Bst = torch.full((rows_b * ldb + off + 8,), nan, dtype=torch.bfloat16)
    Bst[off:off + rows_b * ldb].view(rows_b, ldb)[:, :cols_b] = prob.B
    Ad, Bd = Ast.to(DEV), Bst.to(DEV)
    ldc = N + 3
    Cst = torch.full((M, ldc), -12345.0, dtype=torch.float32, device=DEV)
    P.note(f"unaligned rows {'NT' if colmajor else 'NN'} {M}x{N}x{K} lda {lda} ldb {ldb} off {off} {dist}")
    P.run_bf16(Ad[off:], Bd[off:], colmajor, out=Cst, lda=lda, ldb=ldb, ldc=ldc, M=M, N=N, K=K)
    Cfull = Cst.cpu().numpy()
    assert (Cfull[:, N:] == -12345.0).all(), "C written outside M x N"
    C = np.ascontiguousarray(Cfull[:, :N])
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), colmajor)
    if dist == "integer":
        P.assert_exact(C, want, prob.name)
    P.assert_within_bound(C, want, mag, prob.name)


# ---------------------------------------------------------------- small-M path

# (M, N, K, pad): row-major A and B with padded leading dimensions (multiples
# of 8 elements, the small-M kernel's alignment), K tails not divisible by 32
SMALL_M = [(1, 2048, 256, 0), (5, 2056, 1000, 8), (16, 4096, 777, 7), (17, 2048, 300, 4),
           (33, 2304, 513, 15), (64, 2048, 96, 0), (16, 8192 + 24, 1024, 0)]


@pytest.mark.parametrize("case", SMALL_M, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
@pytest.mark.parametrize("dist", ["normal", "integer"])
def test_small_m_path(case, dist):
    M, N, K, pad = case
    prob = _bf16_case(M, N, K, False, dist, seed=41)
    lda = (K + pad + 7) // 8 * 8
    ldb = (N + 7) // 8 * 8
    Ast = torch.full((M, lda), float("nan"), dtype=torch.bfloat16)
    Ast[:, :K] = prob.A
    Bst = torch.full((K, ldb), float("nan"), dtype=torch.bfloat16)
    Bst[:, :N] = prob.B
    P.note(f"small-M {M}x{N}x{K} lda {lda} {dist}")
    C = P.run_bf16(Ast.to(DEV), Bst.to(DEV), False, M=M, N=N, K=K, lda=lda, ldb=ldb).cpu().numpy()
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), False)
    if dist == "integer":
        P.assert_exact(C, want, prob.name)
    P.assert_within_bound(C, want, mag, prob.name)


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["square4096_nn", "ragged4001x3003x2050_nn", "skinny16x8192x8192_nn"])
def test_workload_full_size(name):
    """The workloads at full size, in the benchmark's launch configuration,
    every output against the oracle."""
    prob = inputs.workload(name, seed=0)
    P.note(f"{name} full size (every output)")
    C = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), prob.b_colmajor).cpu().numpy()
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), prob.b_colmajor)
    P.assert_within_bound(C, want, mag, name)


def test_headline_workload_lines():
    """8192^3 NT at full size: whole rows and whole columns that cross every
    256-row and 256-column tile band (one inside each band, both sides of
    several band boundaries, the first and the last), against the oracle."""
    prob = inputs.workload("square8192_nt", seed=0)
    P.note("square8192_nt full size (rows and columns over every tile band)")
    C = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), prob.b_colmajor).cpu().numpy()
    rows = P.band_lines(prob.M, 256, seed=1)
    cols = P.band_lines(prob.N, 256, seed=2)
    P.check_lines_bf16(C, P.bits16(prob.A), P.bits16(prob.B), True, rows, cols, "square8192_nt")


# ---------------------------------------------------------------- MX fp8

MX_SHAPES = [(32, 32, 32), (256, 256, 256), (300, 200, 96), (129, 257, 160), (512, 384, 512),
             (2048 + 40, 1024 + 8, 640), (1, 1, 64)]


@pytest.mark.parametrize("shape", MX_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mx_integer_bit_exact(shape):
    M, N, K = shape
    prob = inputs.mx_problem(M, N, K, dist="integer", seed=21)
    P.note(f"mx integer {M}x{N}x{K}")
    C = P.run_mx(prob.A.to(DEV), prob.B.to(DEV), prob.SA.to(DEV), prob.SB.to(DEV)).cpu().numpy()
    want, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    P.assert_exact(C, want, prob.name)


@pytest.mark.parametrize("shape", MX_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mx_quantized_normal_within_bound(shape):
    M, N, K = shape
    prob = inputs.mx_problem(M, N, K, dist="normal", seed=22)
    P.note(f"mx normal {M}x{N}x{K}")
    C = P.run_mx(prob.A.to(DEV), prob.B.to(DEV), prob.SA.to(DEV), prob.SB.to(DEV)).cpu().numpy()
    want, mag = P.oracle_mx(prob.A, prob.B, prob.SA, prob.SB)
    P.assert_within_bound(C, want, mag, prob.name)


def test_mx_scale_spread_and_nan():
    """Wide spread of scale codes per block, plus a NaN scale and a NaN element."""
    M, N, K = 320, 288, 384
    prob = inputs.mx_problem(M, N, K, dist="normal", seed=23)
    g = torch.Generator().manual_seed(24)
    SA = torch.randint(100, 150, prob.SA.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    SB = torch.randint(100, 150, prob.SB.shape, generator=g, dtype=torch.int32).to(torch.uint8)
    A = prob.A.clone()
    SB[7, 3] = 255
    A[11, 200] = 0x7F
    P.note("mx scale spread / NaN")
    C = P.run_mx(A.to(DEV), prob.B.to(DEV), SA.to(DEV), SB.to(DEV)).cpu().numpy()
    want, mag = P.oracle_mx(A, prob.B, SA, SB)
    assert np.isnan(C[:, 7]).all() and np.isnan(C[11]).all()
    P.assert_within_bound(C, want, mag, "mx spread")


def test_mx_full_size_workload():
    """MX 8192^3 at full size: whole rows and columns over every tile band,
    plus sampled positions at the tile edges."""
    prob = inputs.workload("mx8192", seed=0)
    P.note("mx8192 full size (rows and columns over every tile band)")
    C = P.run_mx(prob.A.to(DEV), prob.B.to(DEV), prob.SA.to(DEV), prob.SB.to(DEV)).cpu().numpy()
    rows = P.band_lines(prob.M, 256, seed=3)
    cols = P.band_lines(prob.N, 256, seed=4)
    P.check_lines_mx(C, prob.A, prob.B, prob.SA, prob.SB, rows, cols, "mx8192")
    r, c = P.sample_positions(prob.M, prob.N, 1024, seed=5)
    want, mag = P.oracle_mx_at(prob.A, prob.B, prob.SA, prob.SB, r, c)
    P.assert_within_bound(C[r, c], want, mag, "mx8192 (sampled)")
