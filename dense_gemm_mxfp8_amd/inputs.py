"""Seeded synthetic inputs for the GEMM and attention workloads.

This module only draws random numbers and encodes them (bf16 rounding, the
MX e4m3 / e8m0 quantiser that prepares block-scaled operands).  It performs
no part of the matrix product; the HIP library and the CPU oracle both take
its bytes as given.

All generation happens on the CPU with a ``torch.Generator`` seeded per
workload: A is drawn first, then B, so one seed fixes both operands
(attention: Q, then K, then V).

MX encoding (input preparation, not the product).  The pages name
block-scaled MMA ("Modern GPU Programming For MLSys - 书籍总结", sections
2.4 and 2.6) but do not define the encodings; they are read from the public
OCP Microscaling (MX) v1.0 specification: blocks of 32 consecutive
reduction-axis elements share one E8M0 scale 2^(e-127); elements are OCP
E4M3 ("fn": max finite 448, no infinity).  The shared exponent is
floor(log2(amax)) - 8, where 8 is the largest exponent of E4M3, and each
element is v / 2^X rounded to nearest-even E4M3 with saturation to +-448.
An all-zero block gets scale code 127 and zero codes.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def uniform_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    """i.i.d. uniform[-1, 1) rounded (nearest-even) to bf16."""
    return (torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0).to(torch.bfloat16)


def normal_bf16(shape, gen: torch.Generator) -> torch.Tensor:
    """i.i.d. N(0, 1) rounded (nearest-even) to bf16."""
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def integer_bf16(shape, gen: torch.Generator, lo: int = -4, hi: int = 4) -> torch.Tensor:
    """i.i.d. integers in [lo, hi] (exact in bf16)."""
    return torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32).to(torch.bfloat16)


def integer_bf16_large(rows: int, cols: int, gen: torch.Generator, lo: int = -4, hi: int = 4,
                       chunk_rows: int = 8192) -> torch.Tensor:
    """A [rows, cols] integer_bf16 matrix drawn chunk_rows rows at a time from
    one generator, so that operands of several GiB need only one chunk of
    int32 scratch (deterministic for a given chunk_rows)."""
    out = torch.empty((rows, cols), dtype=torch.bfloat16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = integer_bf16((r1 - r0, cols), gen, lo, hi)
    return out


def mx_quantize(x: torch.Tensor):
    """Quantise a float32 [R, K] tensor (K a multiple of 32) into OCP MX form.

    Returns (codes uint8 [R, K], scales uint8 [R, K/32]): e4m3 codes of
    v / 2^X and the e8m0 code X + 127 of each 32-element block along K."""
    if x.dim() != 2 or x.shape[1] % MX_BLOCK:
        raise ValueError("x must be [R, K] with K a multiple of 32")
    R, K = x.shape
    blocks = x.float().reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = blocks.abs().amax(dim=2)
    # floor(log2(amax)) exactly: amax = m * 2^e with m in [0.5, 1)
    _, e = torch.frexp(amax)
    shared = e.to(torch.int32) - 1 - E4M3_EMAX
    code = torch.clamp(shared + 127, 0, 254)
    code = torch.where(amax == 0, torch.full_like(code, 127), code)
    x_eff = (code - 127).to(torch.int32)
    scaled = torch.ldexp(blocks, (-x_eff).unsqueeze(2).to(torch.float32))
    scaled = torch.clamp(scaled, -E4M3_MAX, E4M3_MAX)
    q = scaled.to(torch.float8_e4m3fn).view(torch.uint8).reshape(R, K)
    return q.contiguous(), code.to(torch.uint8).contiguous()


def integer_e4m3(shape, gen: torch.Generator, lo: int = -8, hi: int = 8) -> torch.Tensor:
    """e4m3 codes of i.i.d. integers in [lo, hi] (all exact in e4m3)."""
    v = torch.randint(lo, hi + 1, shape, generator=gen, dtype=torch.int32).to(torch.float32)
    return v.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


@dataclass
class Bf16Problem:
    """A (M,K) row-major bf16; B stored row-major as (K,N) when not
    b_colmajor, else stored as (N,K) (column-major K x N)."""
    name: str
    M: int
    N: int
    K: int
    A: torch.Tensor
    B: torch.Tensor
    b_colmajor: bool


@dataclass
class MxProblem:
    """A (M,K) e4m3 codes row-major; B stored as (N,K) e4m3 codes (column-major
    K x N); SA (M, K/32) and SB (N, K/32) e8m0 codes."""
    name: str
    M: int
    N: int
    K: int
    A: torch.Tensor
    B: torch.Tensor
    SA: torch.Tensor
    SB: torch.Tensor


def bf16_problem(M: int, N: int, K: int, dist: str = "normal", b_colmajor: bool = False,
                 seed: int = 0, name: str | None = None) -> Bf16Problem:
    g = generator(seed)
    draw = {"normal": normal_bf16, "uniform": uniform_bf16, "integer": integer_bf16}[dist]
    A = draw((M, K), g)
    B = draw((N, K) if b_colmajor else (K, N), g)
    return Bf16Problem(name or f"bf16_{M}x{N}x{K}_{dist}", M, N, K, A.contiguous(), B.contiguous(),
                       b_colmajor)


def mx_problem(M: int, N: int, K: int, dist: str = "normal", seed: int = 0,
               name: str | None = None) -> MxProblem:
    g = generator(seed)
    if dist == "normal":
        A, SA = mx_quantize(torch.randn((M, K), generator=g, dtype=torch.float32))
        B, SB = mx_quantize(torch.randn((N, K), generator=g, dtype=torch.float32))
    elif dist == "integer":
        A = integer_e4m3((M, K), g)
        B = integer_e4m3((N, K), g)
        SA = torch.full((M, K // MX_BLOCK), 127, dtype=torch.uint8)
        SB = torch.full((N, K // MX_BLOCK), 127, dtype=torch.uint8)
    else:
        raise ValueError(dist)
    return MxProblem(name or f"mx_{M}x{N}x{K}_{dist}", M, N, K, A, B, SA, SB)


# The workloads: the single-tile case, the square cases, the ragged and skinny
# cases, and the MX case.
WORKLOADS = {
    "tile128_nn": dict(kind="bf16", M=128, N=128, K=128, dist="uniform", b_colmajor=False),
    "square4096_nn": dict(kind="bf16", M=4096, N=4096, K=4096, dist="normal", b_colmajor=False),
    "square8192_nt": dict(kind="bf16", M=8192, N=8192, K=8192, dist="uniform", b_colmajor=True),
    "ragged4001x3003x2050_nn": dict(kind="bf16", M=4001, N=3003, K=2050, dist="normal",
                                    b_colmajor=False),
    "skinny16x8192x8192_nn": dict(kind="bf16", M=16, N=8192, K=8192, dist="normal",
                                  b_colmajor=False),
    "mx8192": dict(kind="mx", M=8192, N=8192, K=8192, dist="normal"),
    # split-K (K ranges planned by the library): a small output with a long K,
    # and the skinny product with column-major B
    "longk1024x1024x32768_nt": dict(kind="bf16", M=1024, N=1024, K=32768, dist="normal", b_colmajor=True,
                                    splitk=True),
    "skinny16x8192x8192_nt": dict(kind="bf16", M=16, N=8192, K=8192, dist="normal", b_colmajor=True,
                                  splitk=True),
    # the skinny product through split-K: 128-column strips over 4 K ranges
    "skinny16x8192x8192_nn_splitk": dict(kind="bf16", M=16, N=8192, K=8192, dist="normal", splitk=True),
    # MX with a long K through split-K: 16 tiles, 16 ranges of 2048
    "mx1024x1024x32768_splitk": dict(kind="mx", M=1024, N=1024, K=32768, dist="normal", splitk=True),
}


@dataclass
class AttnProblem:
    """Q (B, Hq, Sq, D), K and V (B, Hkv, Sk, D), bf16, dense [B][H][S][D]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    Q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor

    @property
    def scale(self) -> float:
        return 1.0 / float(self.D) ** 0.5


def attn_problem(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, D: int, causal: bool = False,
                 dist: str = "normal", seed: int = 0, name: str | None = None) -> AttnProblem:
    g = generator(seed)
    draw = {"normal": normal_bf16, "uniform": uniform_bf16, "integer": integer_bf16}[dist]
    Q = draw((B, Hq, Sq, D), g)
    K = draw((B, Hkv, Sk, D), g)
    V = draw((B, Hkv, Sk, D), g)
    return AttnProblem(name or f"attn_{B}x{Hq}x{Hkv}x{Sq}x{Sk}x{D}_{dist}", B, Hq, Hkv, Sq, Sk, D, causal,
                       Q.contiguous(), K.contiguous(), V.contiguous())


# Attention forward workloads: 16 heads of dimension 128 (hidden size 2048)
# at sequence length 4096 and batch 4 (16k tokens), unmasked and causal.
ATTN_WORKLOADS = {
    "attn4x16x4096_d128": dict(B=4, Hq=16, Hkv=16, Sq=4096, Sk=4096, D=128, causal=False),
    "attn4x16x4096_d128_causal": dict(B=4, Hq=16, Hkv=16, Sq=4096, Sk=4096, D=128, causal=True),
}


def workload(name: str, seed: int = 0):
    if name in ATTN_WORKLOADS:
        return attn_problem(seed=seed, name=name, **ATTN_WORKLOADS[name])
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    w.pop("splitk", None)
    if kind == "bf16":
        return bf16_problem(seed=seed, name=name, **w)
    return mx_problem(seed=seed, name=name, **w)
