"""GPU checks of the dynamic tile schedule (gemm_bf16_dynamic) through the C
ABI.  Every tile is computed once, by the same kernel arithmetic as the static
walk, so C must equal gemm_bf16's / gemm_bf16_nt's bit for bit; the oracle
pins the result itself (exact for integer operands, within the acceptance
bound |C - exact| <= 1e-3 sum_k |a||b| otherwise, on every output).  Cases:
tile counts that are and are not multiples of the grid (so the queues run
dry at different times and work is stolen across XCDs), a partial
last k-tile, repeated calls on one workspace, products the direct-load kernel
does not take (unchanged fallback, workspace untouched) and workspace errors."""
import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
WS = dg.GEMM_DYNAMIC_WORKSPACE_BYTES


def _dynamic(prob, ws, C=None):
    M, N, K = prob.M, prob.N, prob.K
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    ldb = K if prob.b_colmajor else N
    if C is None:
        C = torch.full((M, N), -7.0, dtype=torch.float32, device=DEV)
    rc = dg.gemm_bf16_dynamic(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, prob.b_colmajor, C.data_ptr(), N,
                              ws.data_ptr(), ws.numel() * ws.element_size(), P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return C


# (M, N, K, b_colmajor): 17 x 17 = 289 tiles (one full round plus 33), 16 x 24
# = 384 tiles (1.5 rounds), 1024 tiles with a partial k-tile, NN and NT
SHAPES = [(4352, 4352, 512, True), (4096, 6144, 256, False), (8192, 8192, 264, True), (4096 + 77, 4096 + 8, 200, False)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}_{'nt' if s[3] else 'nn'}")
@pytest.mark.parametrize("exact", [True, False], ids=["integer", "normal"])
def test_dynamic_matches_static_and_oracle(shape, exact):
    M, N, K, colmajor = shape
    prob = inputs.bf16_problem(M, N, K, dist="integer" if exact else "normal", b_colmajor=colmajor, seed=93)
    P.note(f"dynamic {prob.name} {'NT' if colmajor else 'NN'}")
    ws = torch.full((WS // 4,), 0x7fffffff, dtype=torch.int32, device=DEV)  # garbage counters on entry
    got = _dynamic(prob, ws).cpu().numpy().astype(np.float64)
    ref = P.run_bf16(prob.A.to(DEV), prob.B.to(DEV), colmajor).cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), "dynamic schedule differs from the static walk"
    want, mag = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), colmajor)
    if exact:
        P.assert_exact(got, want, prob.name)
    P.assert_within_bound(got, want, mag, prob.name)


def test_dynamic_repeated_calls_share_a_workspace():
    prob = inputs.bf16_problem(4352, 4352, 256, dist="integer", b_colmajor=True, seed=95)
    ws = torch.empty(WS // 4, dtype=torch.int32, device=DEV)
    P.note("dynamic repeated calls")
    first = _dynamic(prob, ws).cpu()
    for _ in range(3):
        again = _dynamic(prob, ws).cpu()
        assert torch.equal(first, again)


def test_dynamic_fallback_leaves_workspace():
    """A product below the 256 x 256 kernel's size runs the static path."""
    prob = inputs.bf16_problem(300, 260, 200, dist="integer", b_colmajor=False, seed=96)
    ws = torch.full((WS // 4,), 12345, dtype=torch.int32, device=DEV)
    P.note("dynamic fallback 300x260x200")
    got = _dynamic(prob, ws).cpu().numpy().astype(np.float64)
    assert (ws == 12345).all().item()
    want, _ = P.oracle_bf16(P.bits16(prob.A), P.bits16(prob.B), False)
    P.assert_exact(got, want, prob.name)


def test_dynamic_rejects_bad_workspace():
    prob = inputs.bf16_problem(4096, 4096, 64, dist="integer", b_colmajor=True, seed=97)
    A, B = prob.A.to(DEV), prob.B.to(DEV)
    C = torch.full((4096, 4096), -7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(WS // 4 + 4, dtype=torch.int32, device=DEV)
    args = (4096, 4096, 64, A.data_ptr(), 64, B.data_ptr(), 64, 1, C.data_ptr(), 4096)
    P.note("dynamic workspace errors")
    assert dg.gemm_bf16_dynamic(*args, 0, WS, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_dynamic(*args, ws.data_ptr(), WS - 1, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_dynamic(*args, ws.data_ptr() + 4, WS, P.stream()) == dg.GEMM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (C == -7.0).all().item()
