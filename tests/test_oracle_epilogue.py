"""The oracle's fused-epilogue definition and its bf16 and E4M3 roundings,
pinned to facts outside the oracle: torch's own float32 -> bfloat16 and
float32 -> float8_e4m3fn conversions (library special cases), the format's
own codes (every finite code rounds to itself), closed forms for the
saturation the library chose, the plain product the epilogue must reduce to,
exact scaling by powers of two, and the transposition identity that tells
row factors from column factors.  No GPU needed."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.timeout(300)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_round_bf16_matches_torch_conversion():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(100000, generator=g) * torch.exp(torch.randn(100000, generator=g) * 25)).float()
    # exact ties between neighbouring bf16 values, subnormals, overflow edge
    lo = torch.tensor([1.0, 1.5, -3.25, 2.0 ** -130, 2.0 ** -127, 3.0e38]).float()
    ties = lo * (1 + 2.0 ** -8)
    special = torch.tensor([0.0, -0.0, float("inf"), -float("inf"), float("nan"),
                            3.3895313892515355e38, 3.4e38, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135]).float()
    x = torch.cat([x, ties, -ties, special])
    want = x.to(torch.bfloat16).double().numpy()
    got = oracle.round_bf16(x.double().numpy())
    same = (want == got) | (np.isnan(want) & np.isnan(got))
    assert same.all(), x.numpy()[~same][:8]
    # the sign of zero survives
    assert np.signbit(oracle.round_bf16(np.array([-0.0]))[0])


def test_epilogue_without_vectors_is_the_product():
    rng = np.random.default_rng(0)
    acc, mag = rng.standard_normal((5, 7)), np.abs(rng.standard_normal((5, 7)))
    t, m = oracle.epilogue(acc, mag)
    assert np.array_equal(t, acc) and np.array_equal(m, mag)


def test_epilogue_on_the_plain_product_and_exact_scaling():
    rng = np.random.default_rng(1)
    A = torch.from_numpy(rng.standard_normal((6, 9))).to(torch.bfloat16)
    B = torch.from_numpy(rng.standard_normal((9, 4))).to(torch.bfloat16)
    acc, mag = oracle.gemm_bf16(_bits(A), _bits(B))
    rs = np.exp2(rng.integers(-3, 4, size=6)).astype(np.float64)
    cs = np.exp2(rng.integers(-3, 4, size=4)).astype(np.float64)
    bias = rng.integers(-5, 6, size=4).astype(np.float64)
    t0, m = oracle.epilogue(acc, mag, rs, cs)
    # powers of two scale exactly
    np.testing.assert_array_equal(t0 / cs[None, :] / rs[:, None], acc)
    np.testing.assert_array_equal(m, mag * rs[:, None] * cs[None, :])
    # the bias is a plain shift (one binary64 rounding)
    t, _ = oracle.epilogue(acc, mag, rs, cs, bias)
    np.testing.assert_allclose(t - bias[None, :], t0, rtol=0, atol=1e-12)


def test_epilogue_transposition_identity():
    # (A B)^T = B^T A^T: the row factors of one are the column factors of the
    # other, which a swapped index in the definition would break (M != N)
    rng = np.random.default_rng(2)
    acc = rng.standard_normal((3, 5))
    mag = np.abs(acc)
    rs, cs = rng.standard_normal(3), rng.standard_normal(5)
    t, _ = oracle.epilogue(acc, mag, rs, cs)
    tt, _ = oracle.epilogue(acc.T, mag.T, cs, rs)
    np.testing.assert_allclose(t.T, tt, rtol=1e-15, atol=0)


def test_epilogue_at_positions_matches_full():
    rng = np.random.default_rng(4)
    acc = rng.standard_normal((6, 8))
    mag = np.abs(acc)
    rs, cs, b = rng.standard_normal(6), rng.standard_normal(8), rng.standard_normal(8)
    t, m = oracle.epilogue(acc, mag, rs, cs, b)
    rows, cols = np.array([0, 5, 3, 2]), np.array([7, 0, 4, 4])
    ts, ms = oracle.epilogue(acc[rows, cols], mag[rows, cols], rs, cs, b, rows=rows, cols=cols)
    np.testing.assert_array_equal(ts, t[rows, cols])
    np.testing.assert_array_equal(ms, m[rows, cols])


def _e4m3_values():
    """The 254 finite E4M3 values, decoded by torch (a library decoder)."""
    codes = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).double().numpy()


def test_round_e4m3_matches_torch_inside_the_range():
    """Inside the format's range torch's float32 -> float8_e4m3fn conversion
    rounds to nearest even like the definition: checked exhaustively at every
    tie between neighbouring values (and just beside each tie), plus random
    values over the whole range, subnormals included."""
    vals = np.unique(np.abs(_e4m3_values()))
    mids = (vals[1:] + vals[:-1]) / 2
    # the tie above 448 (with 480, the value the exponent would reach next)
    mids = np.append(mids, 464.0)
    near = np.concatenate([mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    g = torch.Generator().manual_seed(5)
    rnd = (torch.rand(200000, generator=g).double() * 930 - 465).numpy()
    tiny = (torch.randn(20000, generator=g).double() * 2.0 ** -8).numpy()
    x = np.concatenate([near, -near, rnd, tiny, vals, -vals, [0.0, -0.0]])
    x = x[np.abs(x) <= 464.0].astype(np.float32).astype(np.float64)  # float32 inputs, as torch takes
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    got = oracle.round_e4m3(x)
    assert np.array_equal(want, got), x[want != got][:8]
    assert np.array_equal(np.signbit(want), np.signbit(got))


def test_round_e4m3_codes_round_to_themselves_and_saturate():
    vals = _e4m3_values()
    assert np.array_equal(oracle.round_e4m3(vals), vals)
    assert vals.max() == 448.0 and vals.min() == -448.0
    big = np.array([448.0, 464.0, 464.0001, 479.9, 480.0, 1e6, 3.4e38, np.inf])
    assert (oracle.round_e4m3(big) == 448.0).all() and (oracle.round_e4m3(-big) == -448.0).all()
    assert np.isnan(oracle.round_e4m3(np.array([np.nan]))).all()
    # subnormal edge: the smallest quantum is 2^-9; half of it ties to zero
    assert oracle.round_e4m3(np.array([2.0 ** -10]))[0] == 0.0
    assert oracle.round_e4m3(np.array([3 * 2.0 ** -11]))[0] == 2.0 ** -9
    assert np.signbit(oracle.round_e4m3(np.array([-2.0 ** -11]))[0])
    # nearest even at a normal tie: between 1 (mantissa 000) and 1.125 (001)
    assert oracle.round_e4m3(np.array([1.0625]))[0] == 1.0
    assert oracle.round_e4m3(np.array([1.1875]))[0] == 1.25
