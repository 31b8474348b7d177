"""The seeded input generators: determinism and the MX quantiser's bounds.

The quantiser prepares MX operands (OCP Microscaling v1.0: E4M3 elements, one
E8M0 scale per 32 consecutive K-elements); it is input preparation, not part
of the product, so its output is decoded here with torch's own float8 types
and checked against the encoding's rounding bound.  No GPU needed."""
import numpy as np
import torch

from dense_gemm_mxfp8_amd import inputs


def _decode(codes, scales):
    q = codes.view(torch.float8_e4m3fn).double()
    s = torch.pow(2.0, scales.double() - 127.0)
    R, K = codes.shape
    return (q.reshape(R, K // 32, 32) * s.unsqueeze(2)).reshape(R, K)


def test_generators_are_deterministic():
    a = inputs.workload("tile128_nn", seed=0)
    b = inputs.workload("tile128_nn", seed=0)
    assert torch.equal(a.A.view(torch.int16), b.A.view(torch.int16))
    assert torch.equal(a.B.view(torch.int16), b.B.view(torch.int16))
    c = inputs.bf16_problem(64, 64, 64, dist="uniform", seed=1)
    assert not torch.equal(a.A[:64, :64].view(torch.int16), c.A.view(torch.int16))
    m1 = inputs.mx_problem(64, 32, 128, seed=3)
    m2 = inputs.mx_problem(64, 32, 128, seed=3)
    assert torch.equal(m1.A, m2.A) and torch.equal(m1.SB, m2.SB)


def test_uniform_and_integer_ranges():
    p = inputs.bf16_problem(256, 128, 96, dist="uniform", seed=0)
    assert p.A.float().abs().max() <= 1.0 and p.B.float().abs().max() <= 1.0
    q = inputs.bf16_problem(64, 64, 64, dist="integer", seed=0)
    v = q.A.float()
    assert torch.equal(v, v.round()) and v.abs().max() <= 4


def test_mx_quantiser_round_trip_bound():
    g = inputs.generator(11)
    x = torch.randn((64, 512), generator=g) * torch.exp(torch.randn((64, 1), generator=g) * 3)
    codes, scales = inputs.mx_quantize(x)
    assert codes.dtype == torch.uint8 and scales.shape == (64, 16)
    assert int(scales.max()) <= 254  # 255 (NaN) is never produced
    dec = _decode(codes, scales)
    X = (scales.double() - 127.0).repeat_interleave(32, dim=1)
    v = x.double()
    q = codes.view(torch.float8_e4m3fn).double()
    # saturated: the scaled value lies beyond the largest finite code
    clipped = v.abs() / torch.pow(2.0, X) > 448.0
    # half an ulp of a 3-bit mantissa (2^-4 relative), or half the smallest
    # subnormal step 2^-9 of the scaled value for tiny elements
    bound = torch.maximum(v.abs() * 2.0 ** -4, torch.pow(2.0, X) * 2.0 ** -10)
    ok = (dec - v).abs() <= bound * (1 + 1e-12)
    assert bool(ok[~clipped].all())
    # a saturated element becomes +-448 with its sign
    assert bool((q[clipped].abs() == 448.0).all())
    assert bool((torch.sign(q[clipped]) == torch.sign(v[clipped])).all())
    # the block maximum sets the exponent: floor(log2 amax) - 8
    amax = v.reshape(64, 16, 32).abs().amax(dim=2)
    want = torch.floor(torch.log2(amax)) - 8 + 127
    assert torch.equal(scales.double(), want.clamp(0, 254))


def test_mx_quantiser_zero_block():
    x = torch.zeros((2, 64))
    x[1, 32:] = 1.0
    codes, scales = inputs.mx_quantize(x)
    assert scales[0].tolist() == [127, 127] and scales[1, 0] == 127
    assert int(codes[0].sum()) == 0 and int(codes[1, :32].sum()) == 0
    assert np.allclose(_decode(codes, scales)[1, 32:].numpy(), 1.0)
