"""GPU checks of gemm_bf16_splitk_noalloc through the C ABI: the split-K
entry point for callers that cannot allocate, whose partial products live in
the library's fixed per-GPU scratch array.  Its plan and kernels are those of
gemm_bf16_splitk, so its output must equal gemm_bf16_splitk's (with a caller
workspace) bit for bit, and the oracle within the acceptance bound (exact for
integer operands).  Two calls in a row reuse the array, the second with a
smaller product; a plan larger than the array is refused with C untouched."""
import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _operands(prob):
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    ldb = prob.K if prob.b_colmajor else prob.N
    return A, B, ldb


def _noalloc(prob, splits, C):
    A, B, ldb = _operands(prob)
    M, N, K = prob.M, prob.N, prob.K
    return dg.gemm_bf16_splitk_noalloc(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor, C.data_ptr(),
                                       N, dg.GEMM_OUT_F32, None, None, None, splits, P.stream())


def _with_workspace(prob, splits):
    A, B, ldb = _operands(prob)
    M, N, K = prob.M, prob.N, prob.K
    C = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    rc, used, nbytes = dg.gemm_bf16_splitk_workspace(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor,
                                                     C.data_ptr(), N, dg.GEMM_OUT_F32, None, None, None, splits)
    assert rc == dg.GEMM_OK
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    rc = dg.gemm_bf16_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor, C.data_ptr(), N,
                             dg.GEMM_OUT_F32, None, None, None, splits, ws.data_ptr(), ws.numel() * 4, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return C.cpu().numpy().astype(np.float64), used


def _check(prob, splits, exact):
    M, N = prob.M, prob.N
    want_ws, used = _with_workspace(prob, splits)
    assert used > 1, "the case should split"
    C = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    P.note(f"no-alloc split-K {prob.name} {'NT' if prob.b_colmajor else 'NN'} splits={splits} ({used} used)")
    rc = _noalloc(prob, splits, C)
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want_ws), "differs from gemm_bf16_splitk"
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), prob.b_colmajor)
    if exact:
        P.assert_exact(got, want, prob.name)
    P.assert_within_bound(got, want, mag, prob.name)


@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_noalloc_two_calls_second_smaller(exact):
    dist = "integer" if exact else "normal"
    # 256 x 256 partial kernel, planned ranges, K ending inside a k-tile
    big = inputs.bf16_problem(1000, 777, 4104, dist=dist, b_colmajor=True, seed=111)
    _check(big, 0, exact)
    # the array still holds the first call's planes: the second, smaller call
    # must not depend on them
    small = inputs.bf16_problem(300, 520, 1024, dist=dist, b_colmajor=False, seed=112)
    _check(small, 2, exact)


def test_noalloc_small_m_and_stream_k_plans():
    # small-M partial kernel (row-major B), then a stream-K style plan
    # (289 tiles: whole rounds straight to C, 33 left-over tiles split)
    _check(inputs.bf16_problem(16, 2048, 8192, dist="integer", b_colmajor=False, seed=113), 0, True)
    _check(inputs.bf16_problem(4352, 4352, 1024, dist="integer", b_colmajor=True, seed=114), 0, True)


def test_noalloc_refuses_a_plan_larger_than_the_array():
    prob = inputs.bf16_problem(1024, 1024, 32768, dist="integer", b_colmajor=True, seed=115)
    C = torch.full((1024, 1024), -7.0, dtype=torch.float32, device=DEV)
    # 32 ranges x 4 MiB planes = 128 MiB > 64 MiB
    rc, used, nbytes = dg.gemm_bf16_splitk_plan(1024, 1024, 32768, True, 32)
    assert used == 32 and nbytes > dg.GEMM_SCRATCH_BYTES
    P.note("no-alloc split-K: plan larger than the scratch array")
    assert _noalloc(prob, 32, C) == dg.GEMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (C == -7.0).all().item(), "C changed by a refused call"
    # the library's own plan (16 ranges, 64 MiB) fits exactly
    rc, used, nbytes = dg.gemm_bf16_splitk_plan(1024, 1024, 32768, True, 0)
    assert used == 16 and nbytes == dg.GEMM_SCRATCH_BYTES
    assert _noalloc(prob, 0, C) == dg.GEMM_OK
    torch.cuda.synchronize()
    r = P.band_lines(1024, 256, 116)
    P.check_lines_bf16(C.cpu().numpy().astype(np.float64), P.bits16(prob.A), P.bits16(prob.B), True, r, r,
                       prob.name, exact=True)


def test_noalloc_unsplit_and_empty():
    # a product that fills the GPU runs unsplit (as gemm_bf16 / gemm_bf16_nt)
    prob = inputs.bf16_problem(4096, 4096, 256, dist="integer", b_colmajor=True, seed=117)
    C = torch.full((4096, 4096), -7.0, dtype=torch.float32, device=DEV)
    P.note("no-alloc split-K unsplit 4096x4096x256")
    assert _noalloc(prob, 0, C) == dg.GEMM_OK
    torch.cuda.synchronize()
    ref = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), True)
    assert torch.equal(C, ref)
    assert dg.gemm_bf16_splitk_noalloc(0, 4, 4, 0, 4, 0, 4, 1, 0, 4, dg.GEMM_OUT_F32, None, None, None, 0,
                                       P.stream()) == dg.GEMM_OK
    assert dg.gemm_bf16_splitk_noalloc(4, 4, 4, 0, 4, 0, 4, 1, 0, 4, dg.GEMM_OUT_F32, None, None, None, -1,
                                       P.stream()) == dg.GEMM_ERR_INVALID_ARG
