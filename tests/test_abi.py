"""Host-side checks of the C ABI: the library loads, exports every entry point
that include/libgemm.h declares, and rejects bad arguments before touching a
device.  No GPU needed (no call here reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest

import dense_gemm_mxfp8_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgemm.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "attention.h")]


def declared_functions():
    names = []
    for path in HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*((?:gemm|attn)_\w+)\s*\(", text, flags=re.M)
    return names


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"gemm_bf16", "gemm_bf16_nt", "gemm_mxfp8", "gemm_strerror", "gemm_version",
            "attn_fwd_bf16"} <= names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(dg.LIBRARY)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in libgemm.h but not exported"


def test_version_and_messages():
    assert dg.gemm_version() >= 100
    for code in (0, -1, -2, -3, 99):
        assert isinstance(dg.gemm_strerror(code), str) and dg.gemm_strerror(code)


FAKE = 0x1000  # never dereferenced: validation fails first


@pytest.mark.parametrize("fn", ["gemm_bf16", "gemm_bf16_nt"])
def test_bf16_rejects_bad_arguments(fn):
    f = getattr(dg, fn)
    nt = fn.endswith("_nt")
    ok_ldb = 16 if nt else 8   # K=16, N=8
    bad = [
        (-1, 8, 16, FAKE, 16, FAKE, ok_ldb, FAKE, 8),
        (4, -1, 16, FAKE, 16, FAKE, ok_ldb, FAKE, 8),
        (4, 8, -1, FAKE, 16, FAKE, ok_ldb, FAKE, 8),
        (4, 8, 16, FAKE, 15, FAKE, ok_ldb, FAKE, 8),       # lda < K
        (4, 8, 16, FAKE, 16, FAKE, ok_ldb - 1, FAKE, 8),   # ldb too small
        (4, 8, 16, FAKE, 16, FAKE, ok_ldb, FAKE, 7),       # ldc < N
        (4, 8, 16, 0, 16, FAKE, ok_ldb, FAKE, 8),          # null A
        (4, 8, 16, FAKE, 16, 0, ok_ldb, FAKE, 8),          # null B
        (4, 8, 16, FAKE, 16, FAKE, ok_ldb, 0, 8),          # null C
    ]
    for args in bad:
        assert f(*args, 0) == dg.GEMM_ERR_INVALID_ARG, args


def test_mx_rejects_bad_arguments():
    f = dg.gemm_mxfp8
    assert f(4, 8, 48, FAKE, 48, FAKE, 48, FAKE, FAKE, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG
    assert f(4, 8, 64, FAKE, 64, FAKE, 64, 0, FAKE, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG
    assert f(4, 8, 64, FAKE, 64, FAKE, 64, FAKE, 0, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG
    assert f(4, 8, 64, FAKE, 63, FAKE, 64, FAKE, FAKE, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG
    assert f(4, 8, 64, FAKE, 64, FAKE, 60, FAKE, FAKE, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG
    assert f(-4, 8, 64, FAKE, 64, FAKE, 64, FAKE, FAKE, FAKE, 8, 0) == dg.GEMM_ERR_INVALID_ARG


def test_empty_extents_are_a_no_op():
    # M == 0 or N == 0: success without touching any pointer or the device
    assert dg.gemm_bf16(0, 8, 16, 0, 16, 0, 8, 0, 8, 0) == dg.GEMM_OK
    assert dg.gemm_bf16_nt(4, 0, 16, 0, 16, 0, 16, 0, 1, 0) == dg.GEMM_OK
    assert dg.gemm_mxfp8(0, 0, 64, 0, 64, 0, 64, 0, 0, 0, 1, 0) == dg.GEMM_OK


def test_fused_entry_points_reject_bad_epilogue_arguments():
    # checked before any device call
    assert dg.gemm_bf16_fused(4, 4, 4, 16, 4, 16, 4, 0, 16, 4, 7, None, None, None, None) == dg.GEMM_ERR_INVALID_ARG
    # fp32 output needs a 4-byte aligned C, bf16 a 2-byte aligned one
    assert dg.gemm_bf16_fused(4, 4, 4, 16, 4, 16, 4, 1, 18, 4, dg.GEMM_OUT_F32, None, None, None,
                              None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_mxfp8_fused(4, 4, 32, 16, 32, 16, 32, 16, 16, 17, 4, dg.GEMM_OUT_BF16, None, None, None,
                               None) == dg.GEMM_ERR_INVALID_ARG
    # empty extents are still a no-op
    assert dg.gemm_bf16_fused(0, 4, 4, 0, 4, 0, 4, 0, 0, 4, dg.GEMM_OUT_BF16, None, None, None, None) == dg.GEMM_OK


def test_splitk_rejects_negative_splits():
    # checked before any device call
    args = (4, 4, 64, 16, 64, 16, 64, 1, 16, 4, dg.GEMM_OUT_F32, None, None, None)
    assert dg.gemm_bf16_splitk(*args, -1, None, 0, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk_plan(4, 4, 64, 1, -1, 256)[0] == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk_plan(-4, 4, 64, 1, 0, 256)[0] == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk_plan(4, 4, 64, 1, 0, -1)[0] == dg.GEMM_ERR_INVALID_ARG


# (M, N, K, b_colmajor, splits asked, compute units) -> K ranges planned.
# Planned ranges (splits 0): 256 x 256 tiles that give the CUs under 3/4 of
# a round get K cut into about CUs / tiles ranges of at least 512; small-M
# products (row-major B, M <= 64, N >= 2048) the same per 32-column block with
# ranges of at least 1024.  Asked counts are honoured up to 32, with the range
# length rounded up to the partial kernel's k-tile (64, or 32 for small M).
SPLIT_PLANS = [
    ((8192, 8192, 8192, 1, 0, 256), 1),     # 1024 tiles: the GPU is full
    ((4096, 4096, 4096, 0, 0, 256), 1),     # 256 tiles
    ((2048, 2048, 16384, 1, 0, 256), 4),    # 64 tiles x 4 ranges of 4096
    ((2048, 2048, 1024, 1, 0, 256), 2),     # ranges of at least 512
    ((2048, 2048, 16384, 1, 0, 128), 2),    # fewer CUs, fewer ranges
    ((16, 2048, 8192, 0, 0, 256), 4),       # small M: 64 column blocks
    ((16, 8192, 8192, 0, 0, 256), 4),       # small M: 64 wide 128-column strips x 4 ranges
    ((48, 8192, 8192, 0, 0, 256), 1),       # M > 16: 256 column blocks of 32 fill the GPU
    ((16, 8192, 8192, 1, 0, 256), 8),       # column-major B: 32 tiles
    ((1000, 777, 4104, 1, 5, 256), 5),
    ((1000, 1000, 1000, 1, 5, 256), 4),     # 200 -> 256 per range: 4 ranges
    ((1000, 1000, 1000, 1, 100, 256), 16),  # capped at 32, then 64-element ranges
    ((1000, 1000, 1002, 1, 4, 256), 1),     # lda = 1002: rows not 16-byte aligned
    ((0, 1000, 1000, 1, 4, 256), 1),
    # stream-K style: whole rounds unsplit, a last round at most half full split
    ((4352, 4352, 4096, 1, 0, 256), 7),     # 289 tiles: 33 left over, 7 ranges of 640
    ((4096, 6144, 4096, 0, 0, 256), 2),     # 384 tiles: 128 left over
    ((8448, 8192, 8192, 1, 0, 256), 8),     # 1056 tiles: 32 left over, 8 ranges
    ((4352, 4352, 512, 1, 0, 256), 1),      # K too short for two ranges of 512
    ((6656, 4096, 4096, 1, 0, 256), 1),     # 416 tiles: the last round is over half full
]

# tiles left over after the whole rounds of the stream-K style plans above
LEFT_OVER = {(4352, 4352, 4096): 33, (4096, 6144, 4096): 128, (8448, 8192, 8192): 32}


@pytest.mark.parametrize("case,want", SPLIT_PLANS, ids=lambda c: "x".join(map(str, c)) if isinstance(c, tuple) else str(c))
def test_splitk_plan(case, want):
    M, N, K, colmajor, splits, cus = case
    rc, used, nbytes = dg.gemm_bf16_splitk_plan(M, N, K, colmajor, splits, cus)
    assert rc == dg.GEMM_OK
    assert used == want
    if used == 1:
        assert nbytes == 0
    elif (M, N, K) in LEFT_OVER:
        # compact 256 x 256 fp32 partial tiles of the left-over tiles only
        assert nbytes == used * LEFT_OVER[(M, N, K)] * 256 * 256 * 4
    else:
        assert nbytes == used * M * N * 4


def test_dynamic_rejects_bad_workspace_before_any_device_call():
    args = (4, 4, 64, FAKE, 64, FAKE, 64, 1, FAKE, 4)
    W = dg.GEMM_DYNAMIC_WORKSPACE_BYTES
    assert dg.gemm_bf16_dynamic(*args, None, W, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_dynamic(*args, FAKE, W - 1, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_dynamic(*args, FAKE + 4, W, None) == dg.GEMM_ERR_INVALID_ARG
    # empty extents: a no-op
    assert dg.gemm_bf16_dynamic(0, 4, 64, 0, 64, 0, 64, 1, 0, 4, FAKE, W, None) == dg.GEMM_OK


def test_attention_rejects_bad_arguments():
    """Argument checks of attn_fwd_bf16 fail before any device call."""
    F = FAKE * 16  # 16-byte aligned, never dereferenced
    ok = dict(batch=2, heads_q=4, heads_kv=2, seq_q=100, seq_k=90, head_dim=128, Q=F, q_strides=None, K=F,
              k_strides=None, V=F, v_strides=None, O=F, o_strides=None, lse=None, scale=0.1, causal=1, stream=0)
    bad = [
        dict(batch=-1), dict(seq_q=-1), dict(seq_k=-1), dict(heads_q=0), dict(heads_kv=0),
        dict(heads_q=5),                       # not a multiple of heads_kv
        dict(head_dim=96), dict(head_dim=0),   # 64 and 128 only
        dict(scale=0.0), dict(scale=-0.5), dict(scale=float("inf")), dict(scale=float("nan")),
        dict(Q=0), dict(K=0), dict(V=0), dict(O=0),
        dict(Q=F + 2), dict(K=F + 8), dict(V=F + 4), dict(O=F + 4), dict(lse=F + 2),
        dict(q_strides=(0, 0, 129)),           # not a multiple of 8
        dict(k_strides=(0, 0, 64)),            # sequence stride below head_dim
        dict(o_strides=(0, 0, 130)),           # O strides: multiples of 4
        dict(v_strides=(0, -8, 128)),
        dict(seq_k=1 << 23),                   # (seq_k + 64) rows of 256 B pass 2 GiB
    ]
    for change in bad:
        args = dict(ok, **change)
        assert dg.attn_fwd_bf16(**args) == dg.GEMM_ERR_INVALID_ARG, change


def test_attention_out_type_rejects_bad_arguments():
    """attn_fwd_bf16_out checks its output type and the alignment that type
    needs before any device call; every attn_fwd_bf16 rejection holds too."""
    F = FAKE * 16
    ok = dict(batch=2, heads_q=4, heads_kv=2, seq_q=100, seq_k=90, head_dim=128, Q=F, q_strides=None, K=F,
              k_strides=None, V=F, v_strides=None, O=F, o_strides=None, out_type=dg.GEMM_OUT_BF16, lse=None,
              scale=0.1, causal=0, stream=0)
    bad = [
        dict(out_type=3), dict(out_type=-1),
        dict(out_type=dg.GEMM_OUT_E4M3),                      # no fp8 output for attention
        dict(O=F + 4),                                        # bf16 O: 8-byte aligned
        dict(O=F + 8, out_type=dg.GEMM_OUT_F32),              # fp32 O: 16-byte aligned
        dict(o_strides=(0, 0, 130)),                          # multiples of 4 elements
        dict(o_strides=(0, 0, 64)),                           # sequence stride below head_dim
        dict(head_dim=96), dict(Q=F + 2), dict(scale=0.0), dict(O=0),
    ]
    for change in bad:
        args = dict(ok, **change)
        assert dg.attn_fwd_bf16_out(**args) == dg.GEMM_ERR_INVALID_ARG, change


# ---------------------------------------------------------------- no device

NO_DEVICE = pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                               reason="checks the behaviour without a GPU")


@NO_DEVICE
def test_valid_calls_without_a_device_are_unsupported_and_write_nothing():
    """Every entry point checks for a gfx950 device before any work: with no
    device a valid call returns GEMM_ERR_UNSUPPORTED and leaves C untouched
    (here host buffers stand in for the operands; they are never read)."""
    import numpy as np
    M, N, K = 64, 48, 96
    A = np.zeros(M * K, np.uint16)
    B = np.zeros(K * N, np.uint16)
    S = np.full(M * K // 32 + N * K // 32, 127, np.uint8)
    C = np.full(M * N, 12345.0, np.float32)
    W = np.zeros(1 << 16, np.uint8)
    a, b, c, s, w = (x.ctypes.data for x in (A, B, C, S, W))
    UN = dg.GEMM_ERR_UNSUPPORTED
    assert dg.gemm_bf16(M, N, K, a, K, b, N, c, N, 0) == UN
    assert dg.gemm_bf16_nt(M, N, K, a, K, b, K, c, N, 0) == UN
    assert dg.gemm_mxfp8(M, N, K, a, K, b, K, s, s, c, N, 0) == UN
    assert dg.gemm_bf16_fused(M, N, K, a, K, b, N, 0, c, N, dg.GEMM_OUT_BF16, None, None, None, 0) == UN
    assert dg.gemm_mxfp8_fused(M, N, K, a, K, b, K, s, s, c, N, dg.GEMM_OUT_F32, None, None, None, 0) == UN
    # E4M3 output: any C byte address is accepted
    assert dg.gemm_bf16_fused(M, N, K, a, K, b, N, 0, c + 1, N, dg.GEMM_OUT_E4M3, None, None, None, 0) == UN
    assert dg.gemm_bf16_splitk(M, N, K, a, K, b, K, 1, c, N, dg.GEMM_OUT_F32, None, None, None, 2, w, W.size,
                               0) == UN
    assert dg.gemm_bf16_dynamic(M, N, K, a, K, b, N, 0, c, N, w, W.size, 0) == UN
    # K == 0 would zero C: still refused before any work
    assert dg.gemm_bf16(M, N, 0, 0, 1, 0, N, c, N, 0) == UN
    assert dg.gemm_bf16_splitk_plan(M, N, K, 1, 0, 0)[0] == UN          # cus = 0: the device's
    assert dg.gemm_bf16_splitk_workspace(M, N, K, a, K, b, K, 1, c, N, dg.GEMM_OUT_F32, None, None, None,
                                         0, 0)[0] == UN
    assert (C == 12345.0).all()


# ------------------------------------------------- split-K workspace query

F16 = FAKE * 16  # 16-byte aligned, never dereferenced


@pytest.mark.parametrize("case", [
    # (M, N, K, lda, ldb, b_colmajor): padded views whose extent is not a
    # multiple of 8 elements but whose leading dimension is
    (512, 512, 8193, 8200, 8200, 1),
    (512, 520, 8193, 8200, 528, 0),
    (16, 2049, 8192, 8192, 2056, 0),     # small M, row-major B, odd N
    (48, 2049, 8192, 8200, 2056, 0),
])
def test_splitk_workspace_uses_the_real_leading_dimensions(case):
    """gemm_bf16_splitk_plan assumes dense leading dimensions; for padded
    views the workspace query plans with the real ones, as the call does."""
    M, N, K, lda, ldb, colmajor = case
    rc, used, nbytes = dg.gemm_bf16_splitk_workspace(M, N, K, F16, lda, F16, ldb, colmajor, F16, N,
                                                     dg.GEMM_OUT_F32, None, None, None, 0, 256)
    assert rc == dg.GEMM_OK
    assert used > 1 and nbytes == used * M * N * 4
    # the dense-layout query cannot see that these operands split
    assert dg.gemm_bf16_splitk_plan(M, N, K, colmajor, 0, 256)[1] == 1


def test_splitk_workspace_matches_the_plan_for_dense_operands():
    for (M, N, K, colmajor, splits, cus), want in SPLIT_PLANS:
        if M == 0:
            continue
        ldb = K if colmajor else N
        lda = K
        rc, used, nbytes = dg.gemm_bf16_splitk_workspace(M, N, K, F16, lda, F16, ldb, colmajor, F16, N,
                                                         dg.GEMM_OUT_F32, None, None, None, splits, cus)
        assert rc == dg.GEMM_OK and (used, nbytes) == dg.gemm_bf16_splitk_plan(M, N, K, colmajor, splits,
                                                                                cus)[1:]


def test_splitk_workspace_follows_the_epilogue_and_alignment():
    # stream-K style plan (289 tiles): only with the plain fp32 store
    args = (4352, 4352, 4096, F16, 4096, F16, 4096, 1, F16, 4352)
    assert dg.gemm_bf16_splitk_workspace(*args, dg.GEMM_OUT_F32, None, None, None, 0, 256)[1] == 7
    assert dg.gemm_bf16_splitk_workspace(*args, dg.GEMM_OUT_BF16, None, None, None, 0, 256)[1:] == (1, 0)
    assert dg.gemm_bf16_splitk_workspace(*args, dg.GEMM_OUT_F32, None, None, F16, 0, 256)[1:] == (1, 0)
    # operands off 16-byte alignment never split
    assert dg.gemm_bf16_splitk_workspace(2048, 2048, 16384, F16 + 2, 16384, F16, 16384, 1, F16, 2048,
                                         dg.GEMM_OUT_F32, None, None, None, 0, 256)[1:] == (1, 0)
    # argument errors as gemm_bf16_splitk's
    assert dg.gemm_bf16_splitk_workspace(64, 64, 64, F16, 63, F16, 64, 1, F16, 64, dg.GEMM_OUT_F32, None,
                                         None, None, 0, 256)[0] == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk_workspace(64, 64, 64, F16, 64, F16, 64, 1, F16, 64, 5, None, None, None, 0,
                                         256)[0] == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_bf16_splitk_workspace(64, 64, 64, F16, 64, F16, 64, 1, F16, 64, dg.GEMM_OUT_F32, None,
                                         None, None, -1, 256)[0] == dg.GEMM_ERR_INVALID_ARG


# ------------------------------------------------------ tensor helper layout

def test_bf16_helper_layout_keyword():
    """b_colmajor=None infers the layout of B from its strides; True takes B
    as the (N, K) storage of a column-major operand; False needs row-major B."""
    import torch
    A = torch.zeros((5, 7), dtype=torch.bfloat16)
    Bnk = torch.zeros((3, 7), dtype=torch.bfloat16)       # (N, K) storage
    Bkn = torch.zeros((7, 3), dtype=torch.bfloat16)       # row-major (K, N)
    op = dg._bf16_operands
    assert op(A, Bnk.t()) == (5, 3, 7, 7, 7, True)
    assert op(A, Bkn) == (5, 3, 7, 7, 3, False)
    assert op(A, Bnk, True) == (5, 3, 7, 7, 7, True)
    assert op(A, Bkn, False) == (5, 3, 7, 7, 3, False)
    with pytest.raises(ValueError):
        op(A, Bnk.t(), False)      # column-major B where row-major is asked for
    with pytest.raises(ValueError):
        op(A, Bkn.t(), True)       # (N, K) view with unit stride along N
    with pytest.raises(ValueError):
        op(A, Bkn, True)           # (K, N) is not (N, K)


@pytest.mark.parametrize("case,want", [
    ((1024, 1024, 8192, 0, 0), 8),      # 16 tiles: 8 ranges of 1024
    ((1000, 777, 4096, 0, 0), 4),
    ((512, 520, 3584, 2, 0), 2),        # ranges of 2048 and 1536
    ((8192, 8192, 8192, 0, 0), 1),      # the GPU is full
    ((1024, 1024, 8192 - 128, 0, 0), 1),  # K not a multiple of 512: no split kernel
    ((1024, 1024, 8192, 0, 4), 1),      # scales 4 bytes off 16-byte alignment
    ((1024, 1024, 8192, 100, 0), 8),    # asked counts are cut to ranges of at least 1024
])
def test_mxfp8_splitk_plan(case, want):
    M, N, K, splits, soff = case
    rc, used, nbytes = dg.gemm_mxfp8_splitk_workspace(M, N, K, F16, K, F16, K, F16 + soff, F16 + soff, F16, N,
                                                      dg.GEMM_OUT_F32, None, None, None, splits, 256)
    assert rc == dg.GEMM_OK
    assert used == want and nbytes == (used * M * N * 4 if used > 1 else 0)


def test_mxfp8_splitk_rejects_bad_arguments():
    args = (64, 64, 1024, F16, 1024, F16, 1024, F16, F16, F16, 64, dg.GEMM_OUT_F32, None, None, None)
    assert dg.gemm_mxfp8_splitk(*args, -1, None, 0, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_mxfp8_splitk_workspace(*args, -1, 256)[0] == dg.GEMM_ERR_INVALID_ARG
    bad_k = (64, 64, 1000, F16, 1024, F16, 1024, F16, F16, F16, 64, dg.GEMM_OUT_F32, None, None, None)
    assert dg.gemm_mxfp8_splitk(*bad_k, 0, None, 0, None) == dg.GEMM_ERR_INVALID_ARG
    assert dg.gemm_mxfp8_splitk_workspace(*bad_k, 0, 256)[0] == dg.GEMM_ERR_INVALID_ARG
