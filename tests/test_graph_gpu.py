"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): no
allocation, no host synchronisation and no memset nodes, so a captured call
must replay correctly.  Each case captures one call, then replays it four
times with new operand values copied into the same buffers between replays
(eager work and a synchronisation between replays), and compares every
replay bit for bit with an eager call of the same entry point on the same
operands.  Covers the plain 256 x 256 kernel, the small-M kernel, split-K with
dense planes (partial kernel + reduction), the stream-K style plan (partial
kernel + tile reduction), the dynamic schedule (counter fill kernel + GEMM),
MX-fp8 and the attention forward (causal, GQA)."""
import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bf16_call(kind, M, N, K, colmajor):
    """(operand tensors, call(C) that enqueues the product into C)."""
    A = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.empty((N, K) if colmajor else (K, N), dtype=torch.bfloat16, device=DEV)
    ldb = K if colmajor else N
    ws = None
    if kind in ("splitk", "streamk"):
        rc, used, nbytes = dg.gemm_bf16_splitk_plan(M, N, K, colmajor, 0)
        assert rc == 0 and used > 1
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    elif kind == "dynamic":
        ws = torch.empty(dg.GEMM_DYNAMIC_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)

    def call(C):
        s = P.stream()
        if kind in ("splitk", "streamk"):
            rc = dg.gemm_bf16_splitk(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, colmajor, C.data_ptr(), N,
                                     dg.GEMM_OUT_F32, None, None, None, 0, ws.data_ptr(), ws.numel(), s)
        elif kind == "dynamic":
            rc = dg.gemm_bf16_dynamic(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, colmajor, C.data_ptr(), N,
                                      ws.data_ptr(), ws.numel(), s)
        else:
            fn = dg.gemm_bf16_nt if colmajor else dg.gemm_bf16
            rc = fn(M, N, K, A.data_ptr(), K, B.data_ptr(), ldb, C.data_ptr(), N, s)
        assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)

    def fill(seed):
        prob = inputs.bf16_problem(M, N, K, dist="normal", b_colmajor=colmajor, seed=seed)
        A.copy_(prob.A.to(DEV))
        B.copy_(prob.B.to(DEV))

    return fill, call


def _mx_call(M, N, K):
    A = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    B = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    SA = torch.empty((M, K // 32), dtype=torch.uint8, device=DEV)
    SB = torch.empty((N, K // 32), dtype=torch.uint8, device=DEV)

    def call(C):
        rc = dg.gemm_mxfp8(M, N, K, A.data_ptr(), K, B.data_ptr(), K, SA.data_ptr(), SB.data_ptr(), C.data_ptr(),
                           N, P.stream())
        assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)

    def fill(seed):
        prob = inputs.mx_problem(M, N, K, dist="normal", seed=seed)
        for dst, src in ((A, prob.A), (B, prob.B), (SA, prob.SA), (SB, prob.SB)):
            dst.copy_(src.to(DEV))

    return fill, call


def _attn_call(B, Hq, Hkv, S, D, causal):
    """Attention with O viewed as a (B*Hq*S, D) matrix; lse goes to its own buffer."""
    Q = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device=DEV)
    K = torch.empty((B, Hkv, S, D), dtype=torch.bfloat16, device=DEV)
    V = torch.empty_like(K)
    L = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)

    def call(C):
        rc = dg.attn_fwd_bf16(B, Hq, Hkv, S, S, D, Q.data_ptr(), None, K.data_ptr(), None, V.data_ptr(), None,
                              C.data_ptr(), None, L.data_ptr(), D ** -0.5, causal, P.stream())
        assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)

    def fill(seed):
        prob = inputs.attn_problem(B, Hq, Hkv, S, S, D, causal, seed=seed)
        for dst, src in ((Q, prob.Q), (K, prob.K), (V, prob.V)):
            dst.copy_(src.to(DEV))

    return fill, call


CASES = {
    "fast_nt_4096x4096x512": lambda: _bf16_call("plain", 4096, 4096, 512, True),
    "small_m_16x4096x2048": lambda: _bf16_call("plain", 16, 4096, 2048, False),
    "splitk_planes_1024x1024x8192": lambda: _bf16_call("splitk", 1024, 1024, 8192, True),
    "splitk_small_16x2048x4096": lambda: _bf16_call("splitk", 16, 2048, 4096, False),
    "streamk_4352x4352x1024": lambda: _bf16_call("streamk", 4352, 4352, 1024, True),
    "dynamic_4352x4352x512": lambda: _bf16_call("dynamic", 4352, 4352, 512, True),
    "mx_4096x4096x1024": lambda: _mx_call(4096, 4096, 1024),
    "attention_2x8x2x700x128_causal": lambda: _attn_call(2, 8, 2, 700, 128, True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_call_replays(name):
    fill, call = CASES[name]()
    M_N = {"fast_nt_4096x4096x512": (4096, 4096), "small_m_16x4096x2048": (16, 4096),
           "splitk_planes_1024x1024x8192": (1024, 1024), "splitk_small_16x2048x4096": (16, 2048),
           "streamk_4352x4352x1024": (4352, 4352), "dynamic_4352x4352x512": (4352, 4352),
           "mx_4096x4096x1024": (4096, 4096), "attention_2x8x2x700x128_causal": (2 * 8 * 700, 128)}[name]
    Cg = torch.full(M_N, -7.0, dtype=torch.float32, device=DEV)
    Ce = torch.empty(M_N, dtype=torch.float32, device=DEV)
    P.note(f"graph capture {name}")
    fill(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(Ce)  # warm-up outside the capture (device properties are cached)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(Cg)
    torch.cuda.synchronize()
    for rep in range(4):
        fill(101 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(Ce)
        torch.cuda.synchronize()
        got, want = Cg.cpu().numpy(), Ce.cpu().numpy()
        assert np.isfinite(want).all()
        assert np.array_equal(got, want), f"{name}: replay {rep} differs from the eager call"
