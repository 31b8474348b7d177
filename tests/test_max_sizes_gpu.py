"""GPU parity at the largest operand sizes, through the C ABI.

Two limits of the addressing are crossed on purpose:
  - operands and outputs past 4 GiB, whose byte offsets need 64 bits, on the
    256 x 256 direct-load kernel (tile-local 32-bit buffer descriptors over
    64-bit tile bases);
  - operand spans past the 2 GiB one 32-bit buffer descriptor can cover
    (all K rows of row-major B; 256 rows of A and B when K passes 4 Mi),
    which route the call to the kernels with 64-bit addressing.
Operands are integers small enough that every partial sum stays below 2^24,
so each sampled output must equal the oracle's exact sum bit for bit.
Positions cover tile edges, the last rows and columns and, for the 4 GiB
case, rows whose A and C offsets lie past 2^32 bytes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from dense_gemm_mxfp8_amd import inputs
from tests import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(300)]

DEV = "cuda:0"


def _check(M, N, K, colmajor, lo, hi, seed, extra_rows=()):
    P.note(f"max size {'NT' if colmajor else 'NN'} {M}x{N}x{K} ints [{lo},{hi}] seed={seed}")
    g = inputs.generator(seed)
    A = inputs.integer_bf16_large(M, K, g, lo, hi)
    B = inputs.integer_bf16_large(N, K, g, lo, hi) if colmajor else inputs.integer_bf16_large(K, N, g, lo, hi)
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = P.run_bf16(Ad, Bd, colmajor)
    rows, cols = P.sample_positions(M, N, 64, seed)
    rng = np.random.default_rng(seed + 1)
    for r in extra_rows:
        rows = np.concatenate([rows, np.full(4, r, np.int64)])
        cols = np.concatenate([cols, rng.integers(0, N, 4)])
    got = C[torch.from_numpy(rows).to(DEV), torch.from_numpy(cols).to(DEV)].cpu().numpy()
    assert torch.isfinite(C).all()
    del C, Ad, Bd
    want, _ = P.oracle_bf16_at(P.bits16(A), P.bits16(B), colmajor, rows, cols)
    P.assert_exact(got, want, f"{M}x{N}x{K}")


def test_nt_operand_and_output_past_4gib():
    """A (270000 x 8192 bf16, 4.4 GB) and C (270000 x 4000 fp32, 4.3 GB) past
    2^32 bytes, ragged in M and N, on the direct-load 256 x 256 kernel."""
    M, N, K = 270000, 4000, 8192
    past_a = (1 << 32) // (2 * K)      # first row of A beyond 4 GiB
    past_c = (1 << 32) // (4 * N)      # first row of C beyond 4 GiB
    _check(M, N, K, True, -4, 4, 501, extra_rows=(past_a - 1, past_a, past_c - 1, past_c, M - 1))


def test_nn_b_span_past_2gib():
    """Row-major B of 32768 x 32776 bf16 (2.15 GB): all K rows of B no longer
    fit one descriptor, so the call takes the 64-bit-addressed kernel."""
    _check(300, 32776, 32768, False, -4, 4, 502)


def test_nt_k_past_4mi():
    """K = 4 Mi + 32 (a partial last k-tile): 256 rows of A or B span more
    than 2 GiB.  Entries in {-1, 0, 1} (A and B: 264 x 4194336 bf16, 2.2 GB
    each), so every partial sum stays within 4 Mi + 32 < 2^24."""
    _check(264, 264, (1 << 22) + 32, True, -1, 1, 503)


def test_attention_past_4gib():
    """Attention with Q (32 x 64 x 8292 x 128 bf16, 4.35 GB) and its fp32
    output (8.7 GB) past 2^32 bytes across batch and heads, GQA 8:1, 80 keys
    (one full and one partial key block), against the oracle's rows, with
    the bound of the attention parity tests."""
    import dense_gemm_mxfp8_amd as dg
    import oracle
    from tests.test_attention_gpu import check, qk_abs_max, to_dev
    B, Hq, Hkv, Sq, Sk, D = 32, 64, 8, 8292, 80, 128
    P.note(f"max size attention {B}x{Hq}x{Hkv}x{Sq}x{Sk}x{D}")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, False, dist="normal", seed=504)
    Qd, Kd, Vd = to_dev(p)
    Od, Ld = dg.attention(Qd, Kd, Vd, lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(Od).all() and torch.isfinite(Ld).all()
    q_past = (1 << 32) // (Sq * D * 2)   # first (b Hq + h) whose Q rows lie past 4 GiB
    o_past = (1 << 32) // (Sq * D * 4)   # the same for the fp32 output
    rng = np.random.default_rng(7)
    rows = []
    for bh in (0, o_past - 1, o_past, q_past - 1, q_past, B * Hq - 1):
        for i in (0, 127, 128, Sq - 1, int(rng.integers(Sq))):
            rows.append((bh // Hq, bh % Hq, i))
    rows = np.array(rows, np.int64)
    ri = [torch.from_numpy(rows[:, c]).to(DEV) for c in range(3)]
    O = Od[ri[0], ri[1], ri[2]].cpu().numpy()
    L = Ld[ri[0], ri[1], ri[2]].cpu().numpy()
    del Od, Ld, Qd, Kd, Vd
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    Ow, Om, Lw = oracle.attention_fwd_at(Qb, Kb, Vb, p.scale, False, rows)
    check(O, L, Ow, Om, Lw, p.scale, D, Sk, qk_abs_max(Qb, Kb, rows), "attention past 4 GiB")
