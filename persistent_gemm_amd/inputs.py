"""Seeded synthetic inputs for the Stream-K GEMM workloads.

This module only draws random bytes; it holds none of the GEMM arithmetic, so
both the HIP path and the CPU oracle can consume what it makes.  Every draw
uses one CPU ``torch.Generator`` in the fixed order A, A-scales, B, B-scales,
bias, and returns plain numpy arrays of the exact bytes both sides read.

Distributions (the workloads the Stream-K pages exercise, made synthetic):

* MXFP4: every 4-bit E2M1 code (including -0, code 8) is equally likely; two
  codes per byte with the even K index in the low nibble; one E8M0 scale byte
  per 32 K-elements, uniform on {125, ..., 129} (exponents -2..2).
* bf16: N(0, 1) in fp32, rounded to bf16 by torch.
* fp8: N(0, 1) in fp32, clipped to +-448 and rounded to OCP E4M3FN by torch;
  per-tensor fp32 scales (1.0 unless asked otherwise).
* MXFP8: E4M3FN elements drawn as for fp8, with E8M0 block scales drawn as
  for MXFP4 (one per 32 K-elements, uniform on {125, ..., 129}).
* MXFP6 (E2M3 or E3M2): every 6-bit code equally likely, packed four to
  three bytes (a little-endian bit stream: code k at bits 6k .. 6k+5), with
  E8M0 block scales drawn as for MXFP4.
* bias: N(0, 1) in fp32 rounded to bf16, one value per output column.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "integer_inputs", "exact_inputs", "backward_inputs", "mixed_inputs",
           "pack_fp6"]


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "mxfp4" | "bf16" | "fp8" | "mxfp8" | "mxfp6_e2m3" | "mxfp6_e3m2" | "mxfp4_mxfp8"
    M: int
    N: int
    K: int
    bias: bool
    seed: int
    grid_cap: int = 0     # 0 = every CU
    tile: str | None = None
    caps: tuple = field(default_factory=tuple)
    op: str = "forward"   # "forward" (C = A B^T + bias) or "backward" (dA, dB, dbias of it)
    rotate: int = 0       # input copies a timing loop cycles through (0: one), to keep them out of the 256 MB MALL

    @property
    def flops(self) -> int:
        # the backward makes two products of the forward's size
        return (4 if self.op == "backward" else 2) * self.M * self.N * self.K


# The synthetic workloads; the seed of each is fixed so that tests,
# the bench and the oracle all see the same bytes.
WORKLOADS = {
    "mxfp4_addmm_256x256x512_g5": Workload(
        "mxfp4_addmm_256x256x512_g5", "mxfp4", 256, 256, 512, True, 1000, grid_cap=5, tile="64x64"),
    "bf16_addmm_4096": Workload("bf16_addmm_4096", "bf16", 4096, 4096, 4096, True, 1001),
    # HBM-bound: timed over 10 copies of the inputs (10 x 34 MB > the 256 MB MALL), so bytes come from HBM
    "mxfp4_gemm_16x8192x8192": Workload("mxfp4_gemm_16x8192x8192", "mxfp4", 16, 8192, 8192, False, 1002, rotate=10),
    "mxfp4_addmm_8192": Workload("mxfp4_addmm_8192", "mxfp4", 8192, 8192, 8192, True, 1003),
    "fp8_gemm_4096_capsweep": Workload(
        "fp8_gemm_4096_capsweep", "fp8", 4096, 4096, 4096, False, 1004, caps=(1, 32, 64, 128, 256)),
    # MXFP8 (E4M3 elements, E8M0 block scales) at the large square shape
    "mxfp8_addmm_8192": Workload("mxfp8_addmm_8192", "mxfp8", 8192, 8192, 8192, True, 1005),
    # one MXFP4 and one MXFP8 operand (A E2M1, B E4M3), at the large square shape
    "mxfp4_mxfp8_addmm_8192": Workload("mxfp4_mxfp8_addmm_8192", "mxfp4_mxfp8", 8192, 8192, 8192, True, 1007),
    # MXFP6 (E2M3 and E3M2 elements, E8M0 block scales) at the large square shape
    "mxfp6_e2m3_addmm_8192": Workload("mxfp6_e2m3_addmm_8192", "mxfp6_e2m3", 8192, 8192, 8192, True, 1008),
    "mxfp6_e3m2_addmm_8192": Workload("mxfp6_e3m2_addmm_8192", "mxfp6_e3m2", 8192, 8192, 8192, True, 1009),
    # the bf16 addmm's backward (dA, dB, dbias) at the bf16 forward's shape
    "bf16_addmm_backward_4096": Workload("bf16_addmm_backward_4096", "bf16", 4096, 4096, 4096, True, 1006,
                                         op="backward"),
}


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """uint8 codes[rows][K] (0..63, K % 4 == 0) -> uint8[rows][3K/4]: four codes per three bytes,
    the 24-bit little-endian word of bytes 3j..3j+2 holding code 4j+i at bits 6i .. 6i+5."""
    c = np.asarray(codes, dtype=np.uint32).reshape(codes.shape[0], -1, 4)
    w = c[:, :, 0] | (c[:, :, 1] << 6) | (c[:, :, 2] << 12) | (c[:, :, 3] << 18)
    out = np.empty((codes.shape[0], c.shape[1], 3), dtype=np.uint8)
    for i in range(3):
        out[:, :, i] = (w >> (8 * i)) & 0xFF
    return out.reshape(codes.shape[0], -1)


def make_inputs(dtype: str, M: int, N: int, K: int, *, bias: bool, seed: int,
                scale_lo: int = 125, scale_hi: int = 129, fp8_scales=(1.0, 1.0)) -> dict:
    """Draw one problem.  Returns a dict with keys A, B, SA, SB, bias (None if absent).

    mxfp4: A uint8[M][K/2], B uint8[N][K/2], SA uint8[M][K/32], SB uint8[N][K/32].
    bf16:  A uint16[M][K], B uint16[N][K] (bit patterns); SA = SB = None.
    fp8:   A uint8[M][K], B uint8[N][K] (E4M3FN bytes); SA, SB python floats.
    mxfp8: A uint8[M][K], B uint8[N][K] (E4M3FN bytes), SA uint8[M][K/32], SB uint8[N][K/32].
    mxfp6_e2m3, mxfp6_e3m2: A uint8[M][3K/4], B uint8[N][3K/4] (packed FP6), SA, SB as for MXFP4.
    bias:  uint16[N] bf16 bit patterns, or None.
    """
    g = torch.Generator().manual_seed(seed)
    out = {"dtype": dtype, "M": M, "N": N, "K": K}

    def fp4(rows):
        codes = torch.randint(0, 16, (rows, K), generator=g, dtype=torch.uint8)
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous().numpy()

    def e8m0(rows):
        return torch.randint(scale_lo, scale_hi + 1, (rows, K // 32), generator=g, dtype=torch.uint8).numpy()

    def e4m3(rows):
        x = torch.randn(rows, K, generator=g).clamp(-448.0, 448.0)
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    def fp6(rows):
        return pack_fp6(torch.randint(0, 64, (rows, K), generator=g, dtype=torch.uint8).numpy())

    if dtype == "mxfp4":
        if K % 32:
            raise ValueError("MXFP4 needs K % 32 == 0")
        out["A"] = fp4(M)
        out["SA"] = e8m0(M)
        out["B"] = fp4(N)
        out["SB"] = e8m0(N)
    elif dtype == "bf16":
        out["A"] = _bf16_bits(torch.randn(M, K, generator=g))
        out["SA"] = None
        out["B"] = _bf16_bits(torch.randn(N, K, generator=g))
        out["SB"] = None
    elif dtype == "mxfp8":
        if K % 32:
            raise ValueError("MXFP8 needs K % 32 == 0")
        out["A"] = e4m3(M)
        out["SA"] = e8m0(M)
        out["B"] = e4m3(N)
        out["SB"] = e8m0(N)
    elif dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        if K % 32:
            raise ValueError("MXFP6 needs K % 32 == 0")
        out["A"] = fp6(M)
        out["SA"] = e8m0(M)
        out["B"] = fp6(N)
        out["SB"] = e8m0(N)
    elif dtype == "fp8":
        out["A"] = e4m3(M)
        out["SA"] = float(np.float32(fp8_scales[0]))
        out["B"] = e4m3(N)
        out["SB"] = float(np.float32(fp8_scales[1]))
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    out["bias"] = _bf16_bits(torch.randn(N, generator=g)) if bias else None
    return out


def integer_inputs(dtype: str, M: int, N: int, K: int, *, bias: bool, seed: int, lo: int = -8, hi: int = 8) -> dict:
    """Small-integer operands (values in [lo, hi]) in the bf16, fp8 or MXFP8 encoding.

    Every product and every partial sum of such inputs is an integer far below
    2**24, so any fp32 summation order is exact.  MXFP8 adds block scales
    uniform on {126, 127, 128} (factors 1/2, 1, 2): products are then integers
    times 2**-2 .. 2**2, and sums stay exact while K * 64 * 4 < 2**22.  The
    bias, if drawn, is an integer in [-64, 64].
    """
    g = torch.Generator().manual_seed(seed)
    out = {"dtype": dtype, "M": M, "N": N, "K": K}
    a = torch.randint(lo, hi + 1, (M, K), generator=g).float()
    b = torch.randint(lo, hi + 1, (N, K), generator=g).float()
    if dtype == "bf16":
        out["A"], out["B"] = _bf16_bits(a), _bf16_bits(b)
        out["SA"] = out["SB"] = None
    elif dtype == "fp8":
        out["A"] = a.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out["B"] = b.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out["SA"] = out["SB"] = 1.0
    elif dtype == "mxfp8":
        if K % 32:
            raise ValueError("MXFP8 needs K % 32 == 0")
        out["A"] = a.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out["B"] = b.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        out["SA"] = torch.randint(126, 129, (M, K // 32), generator=g, dtype=torch.uint8).numpy()
        out["SB"] = torch.randint(126, 129, (N, K // 32), generator=g, dtype=torch.uint8).numpy()
    else:
        raise ValueError("integer_inputs covers bf16, fp8 and mxfp8")
    out["bias"] = _bf16_bits(torch.randint(-64, 65, (N,), generator=g).float()) if bias else None
    return out


def exact_inputs(dtype: str, M: int, N: int, K: int, *, bias: bool, seed: int) -> dict:
    """Inputs of `dtype` on which every fp32 partial sum, taken in any order, is exact, so that
    every correct kernel gives the oracle's bits.  Each element is a multiple of a grid step
    q, so each product is a multiple of q_a * q_b; partial sums are then exact while
    sum_k |a*b| stays below 2**24 * q_a * q_b, returned as "exact_below" (the tests check it
    on the oracle's sums).

    * mxfp4: make_inputs (E2M1 steps of 2**-1, scales 2**-2 .. 2**2: q = 2**-3);
    * bf16, fp8, mxfp8: integer_inputs (mxfp8 scales 2**-1 .. 2: q = 2**-1);
    * mxfp6_e2m3: every code (steps of 2**-3), scales on {126, 127, 128}: q = 2**-4;
    * mxfp6_e3m2: codes whose exponent field is 3 .. 6 (magnitudes 1 .. 14, steps of 2**-2
      and up), scales on {126, 127, 128}: q = 2**-3;
    * mxfp4_mxfp8, mxfp8_mxfp4: mixed_inputs with integer E4M3 elements (q = 2**-3 for the
      E2M1 operand, 2**-1 for the E4M3 one).
    """
    if dtype == "mxfp4":
        out = make_inputs(dtype, M, N, K, bias=bias, seed=seed)
        out["exact_below"] = 2.0 ** 18
    elif dtype in ("bf16", "fp8"):
        out = integer_inputs(dtype, M, N, K, bias=bias, seed=seed)
        out["exact_below"] = 2.0 ** 24
    elif dtype == "mxfp8":
        out = integer_inputs(dtype, M, N, K, bias=bias, seed=seed)
        out["exact_below"] = 2.0 ** 22
    elif dtype in ("mxfp4_mxfp8", "mxfp8_mxfp4"):
        a_fmt, b_fmt = dtype.split("_")
        out = mixed_inputs(a_fmt, b_fmt, M, N, K, bias=bias, seed=seed, integer_fp8=True)
        out["exact_below"] = 2.0 ** 20
    elif dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        if K % 32:
            raise ValueError("MXFP6 needs K % 32 == 0")
        g = torch.Generator().manual_seed(seed)
        out = {"dtype": dtype, "M": M, "N": N, "K": K}

        def codes(rows):
            if dtype == "mxfp6_e2m3":
                return torch.randint(0, 64, (rows, K), generator=g, dtype=torch.uint8)
            sign = torch.randint(0, 2, (rows, K), generator=g, dtype=torch.uint8)
            expo = torch.randint(3, 7, (rows, K), generator=g, dtype=torch.uint8)
            mant = torch.randint(0, 4, (rows, K), generator=g, dtype=torch.uint8)
            return (sign << 5) | (expo << 2) | mant

        out["A"] = pack_fp6(codes(M).numpy())
        out["SA"] = torch.randint(126, 129, (M, K // 32), generator=g, dtype=torch.uint8).numpy()
        out["B"] = pack_fp6(codes(N).numpy())
        out["SB"] = torch.randint(126, 129, (N, K // 32), generator=g, dtype=torch.uint8).numpy()
        out["bias"] = _bf16_bits(torch.randint(-64, 65, (N,), generator=g).float()) if bias else None
        out["exact_below"] = 2.0 ** 16 if dtype == "mxfp6_e2m3" else 2.0 ** 18
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def backward_inputs(M: int, N: int, K: int, *, seed: int, integer: bool = False) -> dict:
    """dC uint16[M][N], A uint16[M][K], B uint16[N][K] (bf16 bit patterns), drawn in that order:
    N(0, 1) rounded to bf16, or integers in [-8, 8] with integer=True (every sum then exact)."""
    g = torch.Generator().manual_seed(seed)

    def draw(r, c):
        if integer:
            return _bf16_bits(torch.randint(-8, 9, (r, c), generator=g).float())
        return _bf16_bits(torch.randn(r, c, generator=g))

    dC = draw(M, N)
    A = draw(M, K)
    B = draw(N, K)
    return {"M": M, "N": N, "K": K, "dC": dC, "A": A, "B": B}


def mixed_inputs(a_fmt: str, b_fmt: str, M: int, N: int, K: int, *, bias: bool, seed: int,
                 integer_fp8: bool = False) -> dict:
    """Block-scaled operands of formats a_fmt / b_fmt ("mxfp4" or "mxfp8"), drawn in the order
    A, SA, B, SB, bias as make_inputs does.  MXFP4 codes are uniform over all 16; MXFP8
    elements are N(0, 1) in E4M3FN, or integers in [-8, 8] with integer_fp8=True, whose
    block scales are then uniform on {126, 127, 128} (every sum then stays exact)."""
    if K % 32:
        raise ValueError("MX formats need K % 32 == 0")
    g = torch.Generator().manual_seed(seed)
    out = {"a_fmt": a_fmt, "b_fmt": b_fmt, "M": M, "N": N, "K": K,
           "dtype": a_fmt if a_fmt == b_fmt else f"{a_fmt}_{b_fmt}"}

    def operand(fmt, rows):
        if fmt == "mxfp4":
            codes = torch.randint(0, 16, (rows, K), generator=g, dtype=torch.uint8)
            x = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous().numpy()
            s = torch.randint(125, 130, (rows, K // 32), generator=g, dtype=torch.uint8).numpy()
        elif integer_fp8:
            x = torch.randint(-8, 9, (rows, K), generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            s = torch.randint(126, 129, (rows, K // 32), generator=g, dtype=torch.uint8).numpy()
        else:
            x = torch.randn(rows, K, generator=g).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            x = x.view(torch.uint8).numpy()
            s = torch.randint(125, 130, (rows, K // 32), generator=g, dtype=torch.uint8).numpy()
        return x, s

    out["A"], out["SA"] = operand(a_fmt, M)
    out["B"], out["SB"] = operand(b_fmt, N)
    out["bias"] = _bf16_bits(torch.randn(N, generator=g)) if bias else None
    return out
