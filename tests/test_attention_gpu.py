"""GPU parity of the fused attention forward (attn_fwd_bf16) against the CPU
oracle, through the C ABI.

Acceptance bound (floating point), elementwise for output (b, h, i, d):
  |O_gpu - O| <= rel * sum_j p(i, j) |V(j, d)|      (the oracle's Omag)
  rel = 2^-8 (1 + 2^-6)                  the probabilities enter the value
                                         product rounded to bf16 (unit
                                         roundoff 2^-8); the row sums use the
                                         unrounded values
      + 4 gamma(Sk)                      fp32 sums over the keys (numerator
                                         and row sum), gamma(n) = n u/(1-n u),
                                         u = 2^-24
      + 4 scale gamma(D) max_j sum_d |q(i,d)| |k(j,d)|
                                         fp32 score sums over d, which move
                                         each weight by exp of that error
      + 2^-20                            exp2, the fma that applies the scale,
                                         and the final division (reciprocal
                                         and one fma step, within 2 ulp)
      + 1e-30 absolute                   weights below fp32's normal range
                                         (2^-126) flush to 0 on the GPU, which
                                         moves O by at most Sk 2^-126 max|v|,
                                         under 1e-30 for every case here
  |lse_gpu - lse| <= 4 scale gamma(D) max|qk| + 4 gamma(Sk) + 2^-20 (1 + |lse|)
Cases whose probabilities are exact (equal scores; one score thousands above
the rest) with integer V must match bit for bit: the sums are then exact and
O must equal their IEEE quotient (the kernel forms it from the reciprocal of
the row sum and one fma residual step).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import dense_gemm_mxfp8_amd as dg
from dense_gemm_mxfp8_amd import inputs
import oracle
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def dense_strides(t):
    return (t.stride(0), t.stride(1), t.stride(2))


def run(Q, K, V, scale, causal, want_lse=True, O=None):
    """attn_fwd_bf16 through the C ABI on device tensors of shape
    (B, H, S, D) (any strides with a contiguous last dimension)."""
    B, Hq, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    if O is None:
        O = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.float32, device=DEV)
    L = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV) if want_lse else None
    rc = dg.attn_fwd_bf16(B, Hq, Hkv, Sq, Sk, D, Q.data_ptr(), dense_strides(Q), K.data_ptr(),
                          dense_strides(K), V.data_ptr(), dense_strides(V), O.data_ptr(), dense_strides(O),
                          L.data_ptr() if want_lse else None, scale, causal, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return O.cpu().numpy(), (L.cpu().numpy() if want_lse else None)


def qk_abs_max(Qb, Kb, rows=None):
    """max over keys of sum_d |q(i,d)| |k(j,d)| per query row, GQA-aware."""
    q = np.abs(((Qb.astype(np.uint32) << 16).view(np.float32)).astype(np.float64))
    k = np.abs(((Kb.astype(np.uint32) << 16).view(np.float32)).astype(np.float64))
    g = q.shape[1] // k.shape[1]
    if rows is None:
        kk = np.repeat(k, g, axis=1)
        return np.einsum("bhid,bhjd->bhij", q, kk).max(axis=-1, initial=0.0)
    out = []
    for b, h, i in rows:
        out.append((k[b, h // g] @ q[b, h, i]).max(initial=0.0))
    return np.array(out)


def check(O, L, Ow, Omag, Lw, scale, D, Sk, qkmax, what):
    rel = 2.0 ** -8 * (1 + 2.0 ** -6) + 4 * gamma(Sk) + 4 * scale * gamma(D) * qkmax[..., None] + 2.0 ** -20
    lim = rel * Omag + 1e-30
    assert np.isfinite(O).all() == np.isfinite(Ow).all(), f"{what}: finiteness differs"
    err = np.abs(O.astype(np.float64) - Ow)
    bad = err > lim
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside the bound, first at {idx.tolist()}, "
                             f"worst err/bound {(err / np.maximum(lim, 1e-300)).max():.3g}")
    if L is not None:
        empty = np.isneginf(Lw)
        assert np.isneginf(L[empty]).all(), f"{what}: empty rows must have lse = -inf"
        tl = 4 * scale * gamma(D) * qkmax + 4 * gamma(Sk) + 2.0 ** -20 * (1 + np.abs(np.where(empty, 0, Lw)))
        e = np.abs(L[~empty].astype(np.float64) - Lw[~empty])
        assert (e <= tl[~empty]).all(), f"{what}: lse off by up to {e.max():.3g}"


def to_dev(p):
    return p.Q.to(DEV), p.K.to(DEV), p.V.to(DEV)


# B, Hq, Hkv, Sq, Sk, D
SHAPES = [
    (1, 2, 2, 128, 128, 128),      # one query block, two key blocks
    (2, 4, 2, 300, 257, 128),      # ragged query and key tails, GQA 2:1
    (1, 4, 1, 200, 70, 64),        # Sq > Sk: causal rows with no key
    (1, 2, 2, 70, 333, 64),        # Sq < Sk
    (2, 2, 1, 1, 1000, 128),       # one query row
    (1, 3, 3, 129, 64, 64),        # one key block, a second query block of one row
    (1, 8, 2, 513, 513, 128),      # several blocks each way, GQA 4:1
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_attention_normal(shape, causal):
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = 1000 + sum(shape) + int(causal)
    P.note(f"attention normal {shape} causal={causal} seed={seed}")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, causal, dist="normal", seed=seed)
    O, L = run(*to_dev(p), p.scale, causal)
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    Ow, Om, Lw = oracle.attention_fwd(Qb, Kb, Vb, p.scale, causal)
    check(O, L, Ow, Om, Lw, p.scale, D, Sk, qk_abs_max(Qb, Kb), f"{shape} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 300, 257, 128), (2, 2, 2, 70, 200, 64), (1, 1, 1, 200, 70, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_attention_uniform_exact(shape, causal):
    """q = 0: every visible key has probability exactly 1/n; integer V makes
    o(i) = (sum of n integers) / n, one IEEE division: bit-exact."""
    B, Hq, Hkv, Sq, Sk, D = shape
    P.note(f"attention uniform exact {shape} causal={causal}")
    g = inputs.generator(7 + Sq)
    Q = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16)
    K = inputs.normal_bf16((B, Hkv, Sk, D), g)
    V = inputs.integer_bf16((B, Hkv, Sk, D), g)
    O, L = run(Q.to(DEV), K.to(DEV), V.to(DEV), 1.0 / math.sqrt(D), causal)
    Ow, _, Lw = oracle.attention_fwd(P.bits16(Q), P.bits16(K), P.bits16(V), 1.0 / math.sqrt(D), causal)
    P.assert_exact(O, Ow, f"uniform {shape} causal={causal}")
    empty = np.isneginf(Lw)
    assert np.isneginf(L[empty]).all()
    assert np.allclose(L[~empty], Lw[~empty], rtol=2.0 ** -22, atol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_attention_one_hot_exact(D, causal):
    """q(i) = 64 e_a(i), k(j) = 64 e_b(j): the matching key scores 4096 and
    the rest 0, so every weight but one underflows to 0 and o(i) = v(j*)
    exactly; this pins which key row and which d lands where in every tile.
    Rows whose key is masked or missing average their visible keys exactly
    only when all scores are equal, so they are checked within the bound."""
    B, Hq, Hkv, Sq, Sk = 1, 2, 1, D + 30, D
    P.note(f"attention one-hot D={D} causal={causal}")
    rng = np.random.default_rng(D + causal)
    Qf = np.zeros((B, Hq, Sq, D), np.float32)
    Kf = np.zeros((B, Hkv, Sk, D), np.float32)
    for h in range(Hq):
        Qf[0, h, np.arange(Sq), rng.integers(0, D, Sq)] = 64.0
    Kf[0, 0, np.arange(Sk), rng.permutation(D)[:Sk]] = 64.0
    Vf = rng.integers(-100, 101, size=(B, Hkv, Sk, D)).astype(np.float32)
    Q, K, V = (torch.from_numpy(x).to(torch.bfloat16) for x in (Qf, Kf, Vf))
    scale = 1.0 / math.sqrt(D)
    O, L = run(Q.to(DEV), K.to(DEV), V.to(DEV), scale, causal)
    Qb, Kb, Vb = P.bits16(Q), P.bits16(K), P.bits16(V)
    Ow, Om, Lw = oracle.attention_fwd(Qb, Kb, Vb, scale, causal)
    # rows whose maximum is one key 4096 above the rest: exact
    s = np.einsum("bhid,bjd->bhij", Qf, Kf[:, 0])
    vis = np.ones((Sq, Sk), bool) if not causal else (np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + Sk - Sq)
    hit = ((s == 4096.0) & vis[None, None]).any(-1)
    assert hit.sum() >= 16
    P.assert_exact(O[hit], Ow[hit], f"one-hot D={D} causal={causal}")
    check(O, L, Ow, Om, Lw, scale, D, Sk, qk_abs_max(Qb, Kb), f"one-hot D={D} causal={causal}")


def test_attention_bshd_strides():
    """[B][S][H][D] storage passed as strided (B, H, S, D) views."""
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 150, 190, 128
    P.note("attention BSHD strides")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, True, seed=77)
    Qs = p.Q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Ks = p.K.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Vs = p.V.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Os = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.float32, device=DEV).transpose(1, 2)
    O, L = run(Qs, Ks, Vs, p.scale, True, O=Os)
    O2, L2 = run(*to_dev(p), p.scale, True)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_attention_padded_rows():
    """Sequence strides above the head dimension, with NaN in the padding."""
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 2, 100, 130, 64
    P.note("attention padded rows")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, False, seed=78)

    def pad(t):
        w = torch.full(t.shape[:3] + (D + 24,), float("nan"), dtype=torch.bfloat16)
        w[..., :D] = t
        return w.to(DEV)[..., :D]
    O, L = run(pad(p.Q), pad(p.K), pad(p.V), p.scale, False)
    O2, L2 = run(*to_dev(p), p.scale, False)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_attention_empty_keys_and_rows():
    P.note("attention Sk = 0 and Sq = 0")
    Q = torch.randn(1, 2, 40, 128).to(torch.bfloat16).to(DEV)
    K = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    O, L = run(Q, K, K, 0.1, False)
    assert (O == 0).all() and np.isneginf(L).all()
    Qe = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    Kn = torch.randn(1, 2, 10, 128).to(torch.bfloat16).to(DEV)
    out = torch.empty((1, 2, 0, 128), dtype=torch.float32, device=DEV)
    assert dg.attn_fwd_bf16(1, 2, 2, 0, 10, 128, Qe.data_ptr(), None, Kn.data_ptr(), None, Kn.data_ptr(), None,
                            out.data_ptr(), None, None, 0.1, 1, P.stream()) == dg.GEMM_OK


def test_attention_nan_row():
    """A NaN in query row i makes output row i NaN and leaves the others."""
    B, Hq, Hkv, Sq, Sk, D = 1, 1, 1, 64, 100, 128
    P.note("attention NaN row")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, False, seed=79)
    Q = p.Q.clone()
    Q[0, 0, 5, 17] = float("nan")
    O, _ = run(Q.to(DEV), p.K.to(DEV), p.V.to(DEV), p.scale, False)
    O2, _ = run(*to_dev(p), p.scale, False)
    assert np.isnan(O[0, 0, 5]).all()
    keep = np.ones(Sq, bool)
    keep[5] = False
    assert np.array_equal(O[0, 0, keep], O2[0, 0, keep])


def test_attention_deterministic_and_lse_optional():
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 4, 260, 260, 128
    P.note("attention determinism")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, True, seed=80)
    O1, L1 = run(*to_dev(p), p.scale, True)
    O2, L2 = run(*to_dev(p), p.scale, True)
    O3, _ = run(*to_dev(p), p.scale, True, want_lse=False)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2) and np.array_equal(O1, O3)


def test_attention_tensor_helper():
    P.note("attention tensor helper")
    p = inputs.attn_problem(1, 2, 1, 100, 120, 64, True, seed=81)
    O, L = dg.attention(*to_dev(p), causal=True, lse=True)
    O2, L2 = run(*to_dev(p), p.scale, True)
    assert np.array_equal(O.cpu().numpy(), O2) and np.array_equal(L.cpu().numpy(), L2)


@pytest.mark.parametrize("causal", [False, True])
def test_attention_long_keys(causal):
    """16384 keys (256 key blocks): the longest fp32 sums of the bound's
    gamma(Sk) term, in [B][S][H][D] storage with 8 heads."""
    B, Hq, Hkv, Sq, Sk, D = 1, 8, 2, 300, 16384, 128
    P.note(f"attention long keys causal={causal}")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, causal, seed=95)
    Qs = p.Q.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Ks = p.K.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    Vs = p.V.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    O, L = run(Qs, Ks, Vs, p.scale, causal)
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    rows = np.array([(0, h, i) for h in (0, 5, 7) for i in (0, 1, 150, Sq - 1)], np.int64)
    Ow, Om, Lw = oracle.attention_fwd_at(Qb, Kb, Vb, p.scale, causal, rows)
    check(O[rows[:, 0], rows[:, 1], rows[:, 2]], L[rows[:, 0], rows[:, 1], rows[:, 2]], Ow, Om, Lw, p.scale, D,
          Sk, qk_abs_max(Qb, Kb, rows), f"long keys causal={causal}")


@pytest.mark.parametrize("name", sorted(inputs.ATTN_WORKLOADS))
def test_attention_workload_sampled(name):
    """The benchmark's workloads at full size in its launch configuration:
    sampled rows (first and last rows of query and key blocks, the last row,
    random rows) against the oracle, and every output finite."""
    P.note(f"attention workload {name} (sampled)")
    p = inputs.workload(name, seed=0)
    Qd, Kd, Vd = to_dev(p)
    Od, Ld = dg.attention(Qd, Kd, Vd, causal=p.causal, lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(Od).all() and torch.isfinite(Ld).all()
    rng = np.random.default_rng(5)
    picks = [0, 1, 63, 64, 127, 128, 129, 255, p.Sq - 129, p.Sq - 128, p.Sq - 1]
    rows = [(int(rng.integers(p.B)), int(rng.integers(p.Hq)), i) for i in picks]
    rows += [(int(rng.integers(p.B)), int(rng.integers(p.Hq)), int(rng.integers(p.Sq))) for _ in range(37)]
    rows = np.array(rows, np.int64)
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    Ow, Om, Lw = oracle.attention_fwd_at(Qb, Kb, Vb, p.scale, p.causal, rows)
    O = Od.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    L = Ld.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    check(O, L, Ow, Om, Lw, p.scale, p.D, p.Sk, qk_abs_max(Qb, Kb, rows), name)


@pytest.mark.parametrize("shape", [(2, 4, 2, 300, 257, 128, True), (1, 2, 1, 513, 200, 64, False),
                                   (1, 2, 2, 700, 700, 128, True)], ids=lambda s: "x".join(map(str, s)))
def test_attention_two_groups(shape, monkeypatch):
    """The two-query-group form (ATTN_GROUPS=2: 64 rows per wave, one wave
    per SIMD) against the oracle, and bit-identical to the default form
    (every row goes through the same operations in the same order)."""
    B, Hq, Hkv, Sq, Sk, D, causal = shape
    P.note(f"attention two groups {shape}")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, causal, seed=90 + Sq)
    monkeypatch.setenv("ATTN_GROUPS", "2")
    O, L = run(*to_dev(p), p.scale, causal)
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    Ow, Om, Lw = oracle.attention_fwd(Qb, Kb, Vb, p.scale, causal)
    check(O, L, Ow, Om, Lw, p.scale, D, Sk, qk_abs_max(Qb, Kb), f"two groups {shape}")
    monkeypatch.delenv("ATTN_GROUPS")
    O1, L1 = run(*to_dev(p), p.scale, causal)
    assert np.array_equal(O, O1) and np.array_equal(L, L1)


def run_bf16_out(Q, K, V, scale, causal, O=None):
    """attn_fwd_bf16_out with a bf16 output (NaN-filled beforehand) through
    the C ABI; returns the output's raw bits and lse."""
    B, Hq, Sq, D = Q.shape
    Hkv, Sk = K.shape[1], K.shape[2]
    if O is None:
        O = torch.full((B, Hq, Sq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    L = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=DEV)
    rc = dg.attn_fwd_bf16_out(B, Hq, Hkv, Sq, Sk, D, Q.data_ptr(), dense_strides(Q), K.data_ptr(),
                              dense_strides(K), V.data_ptr(), dense_strides(V), O.data_ptr(), dense_strides(O),
                              dg.GEMM_OUT_BF16, L.data_ptr(), scale, causal, P.stream())
    assert rc == dg.GEMM_OK, dg.gemm_strerror(rc)
    torch.cuda.synchronize()
    return P.bits16(O.cpu()), L.cpu().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 2, 300, 257, 128), (1, 4, 1, 200, 70, 64), (1, 8, 2, 513, 513, 128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_attention_bf16_output(shape, causal):
    """bf16 output: every element is the fp32 output rounded to nearest even
    (bit for bit, against torch's rounding of the fp32 entry point's result),
    lse is unchanged, and against the oracle the bound above plus bf16's
    unit roundoff 2^-8 |O| holds."""
    B, Hq, Hkv, Sq, Sk, D = shape
    seed = 2000 + sum(shape) + int(causal)
    P.note(f"attention bf16 output {shape} causal={causal} seed={seed}")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, causal, dist="normal", seed=seed)
    Ob, Lb = run_bf16_out(*to_dev(p), p.scale, causal)
    O32, L32 = run(*to_dev(p), p.scale, causal)
    want = P.bits16(torch.from_numpy(O32).to(torch.bfloat16))
    assert np.array_equal(Ob, want), f"{(Ob != want).sum()} outputs differ from the rounded fp32 result"
    assert np.array_equal(Lb, L32)
    Qb, Kb, Vb = P.bits16(p.Q), P.bits16(p.K), P.bits16(p.V)
    Ow, Om, Lw = oracle.attention_fwd(Qb, Kb, Vb, p.scale, causal)
    rel = 2.0 ** -8 * (1 + 2.0 ** -6) + 4 * gamma(Sk) + 4 * p.scale * gamma(D) * qk_abs_max(Qb, Kb)[..., None] \
        + 2.0 ** -20
    lim = rel * Om * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Ow) + 1e-30
    O = (Ob.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(O - Ow)
    assert (err <= lim).all(), f"worst err/bound {(err / lim).max():.3g}"


def test_attention_bf16_output_strided_and_helper():
    """bf16 output into a [B][S][H][D] view equals the dense one, and the
    tensor helper's out_dtype=bfloat16 goes through the same entry point."""
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 150, 190, 128
    P.note("attention bf16 output strided + helper")
    p = inputs.attn_problem(B, Hq, Hkv, Sq, Sk, D, True, seed=82)
    Os = torch.full((B, Sq, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    Ob_s, _ = run_bf16_out(*to_dev(p), p.scale, True, O=Os)
    Ob, _ = run_bf16_out(*to_dev(p), p.scale, True)
    assert np.array_equal(Ob_s, Ob)
    Oh = dg.attention(*to_dev(p), causal=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert Oh.dtype == torch.bfloat16 and np.array_equal(P.bits16(Oh.cpu()), Ob)
